"""FP64 CPU oracle for attention with 8-bit floating-point (E4M3) Q and K.

TEST INFRASTRUCTURE ONLY (see ``oracle.attention``): only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it, and it shares nothing with the HIP library.

What it computes, and the passages it follows
---------------------------------------------
* The format is E4M3 of "FP8 Formats for Deep Learning" (in the reference
  list of "Why Low-Precision Transformer Training Fails"): one sign bit, four
  exponent bits with bias 7, three mantissa bits; exponent field 0 holds the
  subnormals m/8 * 2^-6; no infinities; the single pattern with all exponent
  and mantissa bits set (per sign) is NaN, so the largest finite magnitude is
  1.75 * 2^8 = 448.
* Quantising Q and K to 8 bits inside the FlashAttention forward workflow is
  the INT-FlashAttention idea ("INT-FlashAttention", abstract), here with the
  E4M3 format instead of INT8.  The pages give neither the scale granularity
  nor the rounding; the reading, the same as for the INT8 path, is one fp32
  scale per row:
      absmax = max_k |x_k|                       (exact in float32)
      scale  = float32(absmax / 448)             (IEEE fp32 division)
      scale  = 1 if that is 0
      code_k = E4M3(float32(x_k / scale))        (round to nearest, ties to
                                                  even; magnitudes above 448
                                                  saturate to 448)
  The sign bit of a code is the sign bit of its input (so -0.0 and negative
  values that round to zero give the code 0x80).
* Scores are scale * sq_i * sk_j * (Qd Kd^T)_ij with Qd, Kd the decoded
  values: every product of two E4M3 values and every partial sum over
  d <= 128 terms is exact in float64 (significands of at most 8 bits,
  magnitudes between 2^-18 and 2^25), so the dot products are exact.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .attention import attention_head, default_scale

__all__ = ["E4M3_MAX", "e4m3_decode", "e4m3_encode", "quantize_fp8", "fp8_scores",
           "attention_fp8_head", "attention_fp8"]

E4M3_MAX = 448.0


def _e4m3_value(code: int) -> float:
    """Value of one E4M3 bit pattern, from its fields."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
# finite non-negative magnitudes in code order (codes 0x00..0x7e), increasing
_MAGS = _TABLE[:0x7F]


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of uint8 E4M3 codes."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to the even code, magnitudes
    above 448 saturate to 448, NaN gives 0x7f), as uint8."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    hi = np.searchsorted(_MAGS, a, side="left")      # first magnitude >= a
    hi = np.minimum(hi, len(_MAGS) - 1)              # above 448: hi is 448 and
    lo = np.maximum(hi - 1, 0)                       # always the nearer one
    d_lo = a - _MAGS[lo]
    d_hi = _MAGS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo)
    code = mag.astype(np.uint16) | np.where(np.signbit(x), 0x80, 0).astype(np.uint16)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def quantize_fp8(x) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row E4M3 quantisation of float32 rows x[..., d] (reading above).
    Returns (codes uint8 [..., d], scales float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    absmax = np.max(np.abs(x), axis=-1)
    scale = (absmax / np.float32(E4M3_MAX)).astype(np.float32)
    scale = np.where(scale == np.float32(0.0), np.float32(1.0), scale).astype(np.float32)
    ratio = (x / scale[..., None]).astype(np.float32)
    return e4m3_encode(ratio), scale


def fp8_scores(q_codes, k_codes) -> np.ndarray:
    """Exact dot products of decoded E4M3 codes, Qd Kd^T (float64)."""
    qd = e4m3_decode(q_codes)
    kd = e4m3_decode(k_codes)
    return qd @ np.swapaxes(kd, -1, -2)


def attention_fp8_head(q_codes, q_scale, k_codes, k_scale, v, *, causal: bool,
                       scale: float, block_rows: int = 512):
    """Exact attention of one head with scores scale * sq_i * sk_j * D_ij,
    D = Qd Kd^T of the decoded codes."""
    qd = e4m3_decode(q_codes)
    kd = e4m3_decode(k_codes)
    sq = np.asarray(q_scale, dtype=np.float64)
    sk = np.asarray(k_scale, dtype=np.float64)

    def scores(r0, r1, kend):
        dots = qd[r0:r1] @ kd[:kend].T             # exact
        return scale * sq[r0:r1, None] * sk[None, :kend] * dots

    return attention_head(qd, kd, v, causal=causal, scale=scale,
                          block_rows=block_rows, scores_fn=scores)


def attention_fp8(q_codes, q_scale, k_codes, k_scale, v, *, causal: bool,
                  scale: Optional[float] = None, block_rows: int = 512):
    """[B, H, N, d] E4M3 codes + [B, H, N] scales, v [B, H, N, dv]."""
    q_codes = np.asarray(q_codes)
    if scale is None:
        scale = default_scale(q_codes.shape[-1])
    lead = q_codes.shape[:-2]
    n, d = q_codes.shape[-2:]
    qc = q_codes.reshape(-1, n, d)
    kc = np.asarray(k_codes).reshape(-1, n, d)
    qs = np.asarray(q_scale).reshape(-1, n)
    ks = np.asarray(k_scale).reshape(-1, n)
    vv = np.asarray(v)
    vf = vv.reshape((-1,) + vv.shape[-2:])
    o = np.empty(vf.shape, dtype=np.float64)
    lse = np.empty((qc.shape[0], n), dtype=np.float64)
    for u in range(qc.shape[0]):
        o[u], lse[u] = attention_fp8_head(qc[u], qs[u], kc[u], ks[u], vf[u], causal=causal,
                                          scale=scale, block_rows=block_rows)
    return o.reshape(vv.shape), lse.reshape(lead + (n,))
