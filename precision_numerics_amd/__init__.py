"""pnattn: exact softmax attention forward on AMD Instinct MI355X (gfx950).

The compute lives in ``libpnattn.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/pnattn.h``); this package is its ctypes binding.
"""
from ._binding import (ATTN_BF16, ATTN_F32, ATTN_F64, ATTN_FP8, ATTN_INT8, AttnDeviation,
                       AttnError, AttnProblem, AttnWasserstein, attn_baseline_workspace_size,
                       attn_clock_sample, shader_clock_mhz,
                       attn_bwd_delta, attn_bwd_flash, attn_bwd_workspace_size, attn_deviation,
                       attn_deviation_scratch_size, attn_deviation_noalloc,
                       attn_fwd_baseline, attn_fwd_flash, attn_fwd_flash_debug_s,
                       attn_quantize_fp8, attn_quantize_int8, attn_quantize_int8_tiles,
                       attn_version, attn_wasserstein, attn_wasserstein_scratch_size,
                       default_scale, flops, load, make_problem, LIB_PATH)

__all__ = [
    "ATTN_BF16", "ATTN_F32", "ATTN_F64", "ATTN_FP8", "ATTN_INT8", "AttnDeviation", "AttnError",
    "AttnProblem", "AttnWasserstein", "attn_baseline_workspace_size", "attn_clock_sample",
    "shader_clock_mhz", "attn_bwd_delta",
    "attn_bwd_flash", "attn_bwd_workspace_size",
    "attn_deviation", "attn_deviation_noalloc", "attn_deviation_scratch_size", "attn_fwd_baseline", "attn_fwd_flash",
    "attn_fwd_flash_debug_s", "attn_quantize_fp8", "attn_quantize_int8",
    "attn_quantize_int8_tiles", "attn_version", "attn_wasserstein",
    "attn_wasserstein_scratch_size", "default_scale", "flops", "load", "make_problem",
    "LIB_PATH",
]
