"""ctypes binding of libpnattn (argument marshalling only).

Each function has the name of the C entry point it calls.  Tensors are torch
CUDA tensors (contiguous, BHSD); they supply device pointers and the stream
(torch's current stream unless one is given).  Every step of the attention
computation runs in the library's HIP kernels: there is no host fallback, and
a missing library raises at load time.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpnattn.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = range(5)
ATTN_F32, ATTN_BF16, ATTN_INT8, ATTN_F64, ATTN_FP8 = 0, 1, 2, 3, 4


class AttnProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("heads", ctypes.c_int64),
        ("seq_len", ctypes.c_int64),
        ("head_dim", ctypes.c_int64),
        ("causal", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("p_bf16", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("stabilized", ctypes.c_int32),
        ("beta", ctypes.c_float),
        ("o_f32", ctypes.c_int32),
    ]


class AttnDeviation(ctypes.Structure):
    _fields_ = [
        ("max_abs", ctypes.c_double),
        ("mean_abs", ctypes.c_double),
        ("mean_signed", ctypes.c_double),
        ("rms", ctypes.c_double),
        ("max_ref_abs", ctypes.c_double),
        ("rel_normwise", ctypes.c_double),
        ("n", ctypes.c_int64),
        ("n_nonfinite", ctypes.c_int64),
        ("argmax", ctypes.c_int64),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class AttnWasserstein(ctypes.Structure):
    _fields_ = [
        ("w1", ctypes.c_double),
        ("w2", ctypes.c_double),
        ("winf", ctypes.c_double),
        ("n", ctypes.c_int64),
        ("n_nonfinite", ctypes.c_int64),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_P = ctypes.c_void_p
_SIGNATURES = {
    "attn_fwd_flash": [ctypes.POINTER(AttnProblem), _P, _P, _P, _P, _P, _P, _P, _P],
    "attn_fwd_flash_debug_s": [ctypes.POINTER(AttnProblem), _P, _P, _P, _P, _P, _P, _P, _P],
    "attn_baseline_workspace_size": [ctypes.POINTER(AttnProblem), ctypes.POINTER(ctypes.c_size_t)],
    "attn_fwd_baseline": [ctypes.POINTER(AttnProblem), _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                          _P, _P],
    "attn_deviation_scratch_size": [ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)],
    "attn_deviation": [_P, ctypes.c_int32, _P, ctypes.c_int64, _P, ctypes.c_size_t,
                       ctypes.POINTER(AttnDeviation), _P],
    "attn_deviation_noalloc": [_P, ctypes.c_int32, _P, ctypes.c_int64,
                               ctypes.POINTER(AttnDeviation), _P],
    "attn_quantize_int8": [_P, ctypes.c_int64, ctypes.c_int64, _P, _P, _P],
    "attn_quantize_fp8": [_P, ctypes.c_int64, ctypes.c_int64, _P, _P, _P],
    "attn_quantize_int8_tiles": [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_int64, _P, _P, _P],
    "attn_bwd_delta": [ctypes.POINTER(AttnProblem), _P, _P, _P, _P],
    "attn_bwd_workspace_size": [ctypes.POINTER(AttnProblem), ctypes.POINTER(ctypes.c_size_t)],
    "attn_bwd_flash": [ctypes.POINTER(AttnProblem), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                       ctypes.c_size_t, _P],
    "attn_wasserstein_scratch_size": [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_size_t)],
    "attn_wasserstein": [_P, ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int64, _P,
                         ctypes.c_size_t, ctypes.POINTER(AttnWasserstein), _P],
    "attn_clock_sample": [_P, ctypes.c_int32, _P],
    "attn_status_string": [ctypes.c_int],
    "attn_last_error": [],
    "attn_version": [],
}

_LIB = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libpnattn.so (built by ``precision_numerics_amd.build``)."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m precision_numerics_amd.build` "
                           "(or __graft_entry__.build()) first; there is no fallback path")
    lib = ctypes.CDLL(path)
    for name, argtypes in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_char_p if name in ("attn_status_string", "attn_last_error",
                                                 "attn_version") else ctypes.c_int
    if path == LIB_PATH:
        _LIB = lib
    return lib


def _check(status: int):
    if status != ATTN_OK:
        lib = load()
        msg = lib.attn_last_error().decode() or lib.attn_status_string(status).decode()
        raise AttnError(status, msg)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.float64:
        return ATTN_F64
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.int8:
        return ATTN_INT8
    if t.dtype == torch.uint8:
        return ATTN_FP8
    raise TypeError(f"unsupported q/k dtype {t.dtype}")


def _contig(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous CUDA tensors")


def _expect(t, name, shape, dtypes, like=None, required=True):
    """Raise before any C call when tensor ``t`` does not have the shape and
    one of the dtypes the kernels will assume for it (the C ABI sees only
    pointers, so a mismatch here would make a kernel read or write past an
    allocation), or sits on another device than ``like``."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        names = ", ".join(str(d) for d in dtypes)
        raise TypeError(f"{name} has dtype {t.dtype}, expected {names}")
    if like is not None and t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, q on {like.device}")


def _check_attention(q, k, v, q_scale, k_scale, out, lse, out_f32=False):
    """Shapes and dtypes of the forward's tensors, all implied by q."""
    import torch
    if q.dim() != 4:
        raise ValueError(f"q must be [batch, heads, seq_len, head_dim], got shape {tuple(q.shape)}")
    _dtype_code(q)
    b, h, n, d = q.shape
    _expect(k, "k", q.shape, (q.dtype,), q)
    vtype = torch.float32 if q.dtype == torch.float32 else torch.bfloat16
    _expect(v, "v", q.shape, (vtype,), q)
    _expect(out, "out", q.shape, (torch.float32 if out_f32 else vtype,), q, required=False)
    _expect(lse, "lse", (b, h, n), (torch.float32,), q, required=False)
    scaled = q.dtype in (torch.int8, torch.uint8)
    for name, s in (("q_scale", q_scale), ("k_scale", k_scale)):
        if scaled:
            _expect(s, name, (b, h, n), (torch.float32,), q)
        elif s is not None:
            raise ValueError(f"{name} is only for int8 / fp8 q and k")


def _check_rows(x, codes, scales, code_dtype):
    import torch
    if x.dim() < 1:
        raise ValueError("x must have at least one dimension")
    _expect(x, "x", x.shape, (torch.float32,))
    _expect(codes, "codes", x.shape, (code_dtype,), x, required=False)
    _expect(scales, "scales", x.shape[:-1], (torch.float32,), x, required=False)


def make_problem(q, *, causal: bool, p_bf16: bool = True, softmax_scale: float = 0.0,
                 dtype: Optional[int] = None, beta: Optional[float] = None,
                 out_f32: bool = False) -> AttnProblem:
    """beta (> 1) selects the stabilised flash variant; None the standard one.
    out_f32 asks for O in fp32 whatever the input dtype."""
    b, h, n, d = q.shape
    return AttnProblem(b, h, n, d, int(bool(causal)),
                       _dtype_code(q) if dtype is None else dtype, int(bool(p_bf16)),
                       float(softmax_scale), 0 if beta is None else 1,
                       0.0 if beta is None else float(beta), int(bool(out_f32)))


def _out_like(q, v, out_f32=False):
    import torch
    dt = torch.float32 if out_f32 else v.dtype
    return torch.empty(q.shape[:-1] + (v.shape[-1],), dtype=dt, device=v.device)


def attn_fwd_flash(q, k, v, *, causal: bool, p_bf16: bool = True, softmax_scale: float = 0.0,
                   q_scale=None, k_scale=None, out=None, lse=None, beta=None, out_f32=False,
                   stream=None):
    """FlashAttention forward; returns ``out`` ([B,H,N,d], dtype of v, or
    fp32 with out_f32).

    beta (> 1, bf16 inputs only) runs the stabilised variant, whose
    normaliser is beta*r_m (r_m > 0) or 0 (r_m < 0) when the row max r_m
    occurs more than once."""
    _check_attention(q, k, v, q_scale, k_scale, out, lse, out_f32)
    _contig(q, k, v, q_scale, k_scale, out, lse)
    out = _out_like(q, v, out_f32) if out is None else out
    prob = make_problem(q, causal=causal, p_bf16=p_bf16, softmax_scale=softmax_scale, beta=beta,
                        out_f32=out_f32)
    _check(load().attn_fwd_flash(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale),
                                 _ptr(k_scale), _ptr(out), _ptr(lse), _stream(stream)))
    return out


def attn_fwd_flash_debug_s(q, k, v, *, causal: bool, p_bf16: bool = True,
                           softmax_scale: float = 0.0, q_scale=None, k_scale=None, out=None,
                           s_out=None, stream=None):
    """Int8 flash forward that also writes its int32 score tiles to s_out."""
    import torch
    _check_attention(q, k, v, q_scale, k_scale, out, None)
    b, h, n, _ = q.shape
    _expect(s_out, "s_out", (b, h, n, n), (torch.int32,), q)
    _contig(q, k, v, q_scale, k_scale, out, s_out)
    out = _out_like(q, v) if out is None else out
    prob = make_problem(q, causal=causal, p_bf16=p_bf16, softmax_scale=softmax_scale)
    _check(load().attn_fwd_flash_debug_s(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(q_scale), _ptr(k_scale), _ptr(out), _ptr(s_out),
                                         _stream(stream)))
    return out, s_out


def attn_baseline_workspace_size(prob: AttnProblem) -> int:
    n = ctypes.c_size_t(0)
    _check(load().attn_baseline_workspace_size(ctypes.byref(prob), ctypes.byref(n)))
    return n.value


def attn_fwd_baseline(q, k, v, *, causal: bool, p_bf16: bool = True, softmax_scale: float = 0.0,
                      q_scale=None, k_scale=None, workspace=None, out=None, out_f32=False,
                      stream=None):
    """Baseline attention (S and P in the workspace); returns (out, workspace)."""
    import torch
    _check_attention(q, k, v, q_scale, k_scale, out, None, out_f32)
    if workspace is not None and workspace.device != q.device:
        raise ValueError(f"workspace is on {workspace.device}, q on {q.device}")
    _contig(q, k, v, q_scale, k_scale, out, workspace)
    out = _out_like(q, v, out_f32) if out is None else out
    prob = make_problem(q, causal=causal, p_bf16=p_bf16, softmax_scale=softmax_scale,
                        out_f32=out_f32)
    need = attn_baseline_workspace_size(prob)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(load().attn_fwd_baseline(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale),
                                    _ptr(k_scale), _ptr(workspace), nbytes, _ptr(out),
                                    _stream(stream)))
    return out, workspace


def attn_deviation_scratch_size(n: int) -> int:
    b = ctypes.c_size_t(0)
    _check(load().attn_deviation_scratch_size(int(n), ctypes.byref(b)))
    return b.value


def attn_deviation(o_test, o_ref, *, scratch=None, stream=None) -> dict:
    """Deviation summary of o_test (fp32/bf16) against o_ref (fp64), on the GPU."""
    import torch
    if o_test.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"o_test has dtype {o_test.dtype}, expected float32 or bfloat16")
    if o_ref.dtype != torch.float64:
        raise TypeError("o_ref must be float64")
    n = o_test.numel()
    if o_ref.numel() != n:
        raise ValueError("o_test and o_ref differ in size")
    if o_ref.device != o_test.device or (scratch is not None and scratch.device != o_test.device):
        raise ValueError("o_test, o_ref and scratch must be on one device")
    _contig(o_test, o_ref, scratch)
    need = attn_deviation_scratch_size(n)
    if scratch is None:
        scratch = torch.empty(max(need, 1), dtype=torch.uint8, device=o_test.device)
    res = AttnDeviation()
    _check(load().attn_deviation(_ptr(o_test), _dtype_code(o_test), _ptr(o_ref), n, _ptr(scratch),
                                 scratch.numel() * scratch.element_size(), ctypes.byref(res),
                                 _stream(stream)))
    return res.as_dict()


def attn_deviation_noalloc(o_test, o_ref, *, stream=None) -> dict:
    """attn_deviation with the library's own scratch array (no allocation)."""
    import torch
    if o_test.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"o_test has dtype {o_test.dtype}, expected float32 or bfloat16")
    if o_ref.dtype != torch.float64:
        raise TypeError("o_ref must be float64")
    n = o_test.numel()
    if o_ref.numel() != n:
        raise ValueError("o_test and o_ref differ in size")
    if o_ref.device != o_test.device:
        raise ValueError("o_test and o_ref must be on one device")
    _contig(o_test, o_ref)
    res = AttnDeviation()
    _check(load().attn_deviation_noalloc(_ptr(o_test), _dtype_code(o_test), _ptr(o_ref), n,
                                         ctypes.byref(res), _stream(stream)))
    return res.as_dict()


def attn_quantize_int8(x, *, codes=None, scales=None, stream=None):
    """Per-row int8 quantisation of fp32 x[..., d]; returns (codes, scales)."""
    import torch
    _check_rows(x, codes, scales, torch.int8)
    _contig(x, codes, scales)
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    codes = torch.empty(x.shape, dtype=torch.int8, device=x.device) if codes is None else codes
    scales = (torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
              if scales is None else scales)
    _check(load().attn_quantize_int8(_ptr(x), rows, d, _ptr(codes), _ptr(scales),
                                     _stream(stream)))
    return codes, scales


def attn_quantize_int8_tiles(x, tile_rows: int, *, codes=None, scales=None, stream=None):
    """Per-tile int8 quantisation of fp32 x[..., n, d] (tiles of tile_rows
    rows inside each leading index); returns (codes, per-row scales)."""
    import torch
    if x.dim() < 2:
        raise ValueError("x must be [..., n, d]")
    _check_rows(x, codes, scales, torch.int8)
    _contig(x, codes, scales)
    n, d = x.shape[-2], x.shape[-1]
    groups = x.numel() // (n * d) if n * d else 0
    codes = torch.empty(x.shape, dtype=torch.int8, device=x.device) if codes is None else codes
    scales = (torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
              if scales is None else scales)
    _check(load().attn_quantize_int8_tiles(_ptr(x), groups, n, d, int(tile_rows), _ptr(codes),
                                           _ptr(scales), _stream(stream)))
    return codes, scales


def attn_quantize_fp8(x, *, codes=None, scales=None, stream=None):
    """Per-row E4M3 fp8 quantisation of fp32 x[..., d]; returns (codes as
    uint8 bytes, scales)."""
    import torch
    _check_rows(x, codes, scales, torch.uint8)
    _contig(x, codes, scales)
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if codes is None else codes
    scales = (torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
              if scales is None else scales)
    _check(load().attn_quantize_fp8(_ptr(x), rows, d, _ptr(codes), _ptr(scales),
                                    _stream(stream)))
    return codes, scales


def attn_bwd_delta(o, d_o, *, delta=None, stream=None):
    """delta = rowsum(d_o * o) over the last axis ([B,H,N,d] -> [B,H,N] fp32)."""
    import torch
    if o.dim() != 4:
        raise ValueError(f"o must be [batch, heads, seq_len, head_dim], got {tuple(o.shape)}")
    if o.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"o has dtype {o.dtype}, expected float32 or bfloat16")
    _expect(d_o, "d_o", o.shape, (o.dtype,), o)
    b, h, n, d = o.shape
    _expect(delta, "delta", (b, h, n), (torch.float32,), o, required=False)
    _contig(o, d_o, delta)
    delta = (torch.empty((b, h, n), dtype=torch.float32, device=o.device)
             if delta is None else delta)
    code = ATTN_F32 if o.dtype == torch.float32 else ATTN_BF16
    prob = AttnProblem(b, h, n, d, 0, code, 1, 0.0, 0, 0.0, 0)
    _check(load().attn_bwd_delta(ctypes.byref(prob), _ptr(o), _ptr(d_o), _ptr(delta),
                                 _stream(stream)))
    return delta


def attn_wasserstein_scratch_size(n: int, a_dtype: int, b_dtype: int) -> int:
    b = ctypes.c_size_t(0)
    _check(load().attn_wasserstein_scratch_size(int(n), int(a_dtype), int(b_dtype),
                                                ctypes.byref(b)))
    return b.value


def attn_wasserstein(a, b, *, scratch=None, stream=None) -> dict:
    """W1, W2 and W_inf between the value distributions of a and b (same
    number of elements; fp32, bf16 or fp64 each), on the GPU."""
    import torch
    n = a.numel()
    if b.numel() != n:
        raise ValueError("a and b differ in size")
    ta, tb = _dtype_code(a), _dtype_code(b)
    if ATTN_INT8 in (ta, tb) or ATTN_FP8 in (ta, tb):
        raise TypeError("a and b must be float32, bfloat16 or float64")
    if b.device != a.device or (scratch is not None and scratch.device != a.device):
        raise ValueError("a, b and scratch must be on one device")
    _contig(a, b, scratch)
    need = attn_wasserstein_scratch_size(n, ta, tb)
    if scratch is None:
        scratch = torch.empty(max(need, 1), dtype=torch.uint8, device=a.device)
    res = AttnWasserstein()
    _check(load().attn_wasserstein(_ptr(a), ta, _ptr(b), tb, n, _ptr(scratch),
                                   scratch.numel() * scratch.element_size(), ctypes.byref(res),
                                   _stream(stream)))
    return res.as_dict()


def attn_bwd_workspace_size(prob: AttnProblem) -> int:
    n = ctypes.c_size_t(0)
    _check(load().attn_bwd_workspace_size(ctypes.byref(prob), ctypes.byref(n)))
    return n.value


def attn_bwd_flash(q, k, v, o, d_o, lse, *, causal: bool, softmax_scale: float = 0.0,
                   dq=None, dk=None, dv=None, workspace=None, stream=None):
    """FlashAttention backward (bf16); returns (dq, dk, dv)."""
    import torch
    if q.dim() != 4:
        raise ValueError(f"q must be [batch, heads, seq_len, head_dim], got {tuple(q.shape)}")
    if q.dtype != torch.bfloat16:
        raise TypeError(f"q has dtype {q.dtype}; the backward is built for bfloat16")
    b, h, n, _ = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("d_o", d_o)):
        _expect(t, name, q.shape, (torch.bfloat16,), q)
    _expect(lse, "lse", (b, h, n), (torch.float32,), q)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _expect(t, name, q.shape, (torch.bfloat16,), q, required=False)
    _contig(q, k, v, o, d_o, lse, dq, dk, dv, workspace)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    prob = make_problem(q, causal=causal, softmax_scale=softmax_scale)
    need = attn_bwd_workspace_size(prob)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(load().attn_bwd_flash(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                 _ptr(d_o), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream)))
    return dq, dk, dv


def attn_clock_sample(out, *, stream=None):
    """Enqueue one clock sample per row of ``out`` (an int64 [slots, 3]
    CUDA tensor): (location, shader-clock counter, 100 MHz counter)."""
    import torch
    if out.dim() != 2 or out.shape[1] != 3 or out.dtype != torch.int64:
        raise ValueError("out must be an int64 [slots, 3] tensor")
    _contig(out)
    _check(load().attn_clock_sample(_ptr(out), out.shape[0], _stream(stream)))
    return out


def shader_clock_mhz(before, after) -> Optional[float]:
    """Average shader clock between two clock samples (host arrays of
    [slots, 3]), compared on each location (CU) found in both; None when
    there is none."""
    first = {}
    for row in before:
        first.setdefault(int(row[0]), row)
    rates = []
    done = set()
    for row in after:
        loc = int(row[0])
        if loc in first and loc not in done:
            done.add(loc)
            dr = int(row[2]) - int(first[loc][2])
            if dr > 0:
                rates.append(100.0 * (int(row[1]) - int(first[loc][1])) / dr)
    return sum(rates) / len(rates) if rates else None


def attn_version() -> str:
    return load().attn_version().decode()


def flops(batch: int, heads: int, seq_len: int, head_dim: int, causal: bool) -> float:
    """MFMA contraction flops over visible (query, key) pairs (QK^T and PV)."""
    if causal:
        return 2.0 * batch * heads * head_dim * seq_len * (seq_len + 1)
    return 4.0 * batch * heads * seq_len * seq_len * head_dim


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
