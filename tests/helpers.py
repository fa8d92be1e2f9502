"""Shared test plumbing: move seeded inputs to the GPU (for the HIP path) and
to float64 (for the oracle).  No attention arithmetic lives here."""
from __future__ import annotations

import numpy as np

import synth

BF16_MAX_ABS = 2e-2     # bf16-output tolerances (max |err|, mean |err|)
BF16_MEAN_ABS = 2e-3
F32_REL_NORMWISE = 1e-5  # fp32 I/O: max|err| / max|ref|


def torch_bf16(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def device_inputs(inp: synth.Inputs, device="cuda"):
    """(q, k, v) torch tensors as the kernels read them.  For int8 workloads q
    and k are the fp32 draws (the caller quantises them on the GPU)."""
    import torch
    if inp.cfg.dtype == "bf16":
        return tuple(torch_bf16(x, device) for x in (inp.q, inp.k, inp.v))
    q = torch.from_numpy(inp.q).to(device)
    k = torch.from_numpy(inp.k).to(device)
    if inp.cfg.dtype == "f32":
        return q, k, torch.from_numpy(inp.v).to(device)
    return q, k, torch_bf16(inp.v, device)


def oracle_inputs(inp: synth.Inputs):
    """float64 views of the exact stored values (bf16 widened exactly)."""
    def wide(x):
        if x.dtype == np.uint16:
            return synth.bf16_bits_to_f32(x).astype(np.float64)
        return x.astype(np.float64)
    return wide(inp.q), wide(inp.k), wide(inp.v)


def out_to_f64(t) -> np.ndarray:
    import torch
    return t.float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 \
        else t.cpu().numpy().astype(np.float64)


def error_stats(o, ref) -> dict:
    e = np.abs(np.asarray(o, np.float64) - np.asarray(ref, np.float64))
    return dict(max_abs=float(e.max()), mean_abs=float(e.mean()),
                rel_normwise=float(e.max() / max(np.abs(ref).max(), 1e-300)))


def assert_close(o, ref, out_dtype: str, what=""):
    st = error_stats(o, ref)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    if out_dtype == "f32":
        assert st["rel_normwise"] <= F32_REL_NORMWISE, f"{what}: {st}"
    else:
        assert st["max_abs"] <= BF16_MAX_ABS and st["mean_abs"] <= BF16_MEAN_ABS, f"{what}: {st}"
    return st
