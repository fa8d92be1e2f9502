"""FP64 CPU oracle for exact softmax attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` call it.  It shares no code with the HIP kernels or their
binding; the two sides meet only at the seeded inputs of ``synth``.

What it computes, and the passages it follows
---------------------------------------------
* FlashAttention computes *exact* attention, tile by tile, without storing the
  score matrix ("FlashAttention: Fast and Memory-Efficient Exact Attention",
  cited in the reference list of "Is Flash Attention Stable?"; the
  "INT-FlashAttention" record, abstract: FlashAttention lowers memory use by
  working through the GPU memory hierarchy).  The tiling of Q into T_r blocks
  of B_r rows and K, V into T_c blocks of B_c rows ("Why Low-Precision
  Transformer Training Fails", Algorithm 1, first step) changes only the
  order of rounding, so the oracle is the plain definition, not an emulation
  of any tiling:

      S = scale * Q K^T  (+ causal mask: key j visible to query i iff j <= i)
      P = row-softmax(S),   O = P V,   lse_i = m_i + ln(sum_j exp(S_ij - m_i))

  evaluated in float64 on the exact values the GPU receives.
* The deviation of a low-precision forward output from a high-precision one
  of the same isolated forward pass ("Is Flash Attention Stable?", abstract;
  O_lp versus O_hp in "Why Low-Precision Transformer Training Fails",
  Figures 5 and 6) is summarised by :func:`deviation`.
* The quantity the backward pass derives from the forward output,
  delta = rowsum(dO * O) ("Why Low-Precision Transformer Training Fails",
  Figure 5 caption and the section that isolates the error in O: delta_lp
  computed from the low-precision O), is :func:`attention_delta`.
* INT8 attention compatible with the FlashAttention forward workflow
  ("INT-FlashAttention", abstract): the scores are the exact integer dot
  products of int8 codes times the per-row scales.  The pages do not give the
  scale granularity; the reading used here is one fp32 scale per row equal to
  absmax/127 (:func:`quantize_int8`).

Every function states the passage or reading it follows.  Row blocks of at
most ``block_rows`` queries bound the memory of one S block; each output
element is still one softmax row times V, exactly as defined.
"""
from __future__ import annotations

import math
import os
from typing import Optional, Tuple

import numpy as np

__all__ = [
    "default_scale", "attention", "attention_head", "int8_scores",
    "attention_int8", "attention_int8_head", "quantize_int8", "quantize_int8_tiles", "deviation",
    "attention_probabilities", "attention_delta", "attention_backward_head", "run_heads",
]


def default_scale(head_dim: int) -> float:
    """Softmax scale 1/sqrt(head_dim) (the pages do not print it; the usual
    scaled dot-product reading).  Exactly 0.125 for head_dim 64."""
    return 1.0 / math.sqrt(head_dim)


def _visible_mask(r0: int, r1: int, kend: int) -> np.ndarray:
    """Causal visibility for query rows r0..r1-1 and keys 0..kend-1:
    key j is visible to query i iff j <= i."""
    rows = np.arange(r0, r1)[:, None]
    cols = np.arange(kend)[None, :]
    return cols <= rows


def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, *,
                   causal: bool, scale: float, block_rows: int = 512,
                   scores_fn=None) -> Tuple[np.ndarray, np.ndarray]:
    """Exact attention of one (batch, head) unit in float64.

    q: [N, d], k: [N, d], v: [N, dv] (any real dtype; widened to float64).
    ``scores_fn(r0, r1, kend)`` may replace ``scale * q[r0:r1] @ k[:kend].T``
    (the int8 path passes its exact-integer scores through it).
    Returns (O [N, dv] float64, lse [N] float64, natural log).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    o = np.empty((n, v.shape[1]), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    for r0 in range(0, n, block_rows):
        r1 = min(n, r0 + block_rows)
        kend = r1 if causal else k.shape[0]
        if scores_fn is None:
            s = scale * (q[r0:r1] @ k[:kend].T)
        else:
            s = scores_fn(r0, r1, kend)
        if causal:
            s = np.where(_visible_mask(r0, r1, kend), s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        ell = e.sum(axis=1, keepdims=True)
        p = e / ell
        o[r0:r1] = p @ v[:kend]
        lse[r0:r1] = m[:, 0] + np.log(ell[:, 0])
    return o, lse


def attention_probabilities(q, k, *, causal: bool, scale: float) -> np.ndarray:
    """The full softmax matrix P of one head (float64); tiny shapes only."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n = q.shape[0]
    s = scale * (q @ k.T)
    if causal:
        s = np.where(_visible_mask(0, n, k.shape[0]), s, -np.inf)
    top = s.max(axis=1, keepdims=True)
    w = np.exp(s - top)
    return w / w.sum(axis=1, keepdims=True)


def attention(q, k, v, *, causal: bool, scale: Optional[float] = None,
              block_rows: int = 512) -> Tuple[np.ndarray, np.ndarray]:
    """Exact attention over [B, H, N, d] (or [N, d]) arrays, float64.

    Returns (O, lse) with O shaped like v and lse shaped like q[..., 0].
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    if scale is None:
        scale = default_scale(q.shape[-1])
    lead = q.shape[:-2]
    qf = q.reshape((-1,) + q.shape[-2:])
    kf = k.reshape((-1,) + k.shape[-2:])
    vf = v.reshape((-1,) + v.shape[-2:])
    o = np.empty(qf.shape[:-1] + (vf.shape[-1],), dtype=np.float64)
    lse = np.empty(qf.shape[:-1], dtype=np.float64)
    for u in range(qf.shape[0]):
        o[u], lse[u] = attention_head(qf[u], kf[u], vf[u], causal=causal,
                                      scale=scale, block_rows=block_rows)
    return (o.reshape(lead + (q.shape[-2], v.shape[-1])),
            lse.reshape(lead + (q.shape[-2],)))


# ---------------------------------------------------------------------------
# int8 Q/K path ("INT-FlashAttention", abstract; scale granularity is a reading)
# ---------------------------------------------------------------------------

def quantize_int8(x) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric per-row int8 quantisation of float32 rows x[..., d].

    Reading (the pages stop before the quantiser is described):
      absmax = max_k |x_k|                       (exact in float32)
      scale  = float32(absmax / 127)             (IEEE fp32 division)
      scale  = 1 if that is 0 (all-zero row, or underflow)
      code_k = clamp(round_half_even(float32(x_k / scale)), -127, 127)
    Returns (codes int8 [..., d], scales float32 [...]).
    """
    x = np.asarray(x, dtype=np.float32)
    absmax = np.max(np.abs(x), axis=-1)
    scale = (absmax / np.float32(127.0)).astype(np.float32)
    scale = np.where(scale == np.float32(0.0), np.float32(1.0), scale).astype(np.float32)
    ratio = (x / scale[..., None]).astype(np.float32)
    codes = np.clip(np.rint(ratio), -127.0, 127.0).astype(np.int8)
    return codes, scale


def quantize_int8_tiles(x, tile_rows: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per-tile int8 quantisation of float32 x[..., n, d]: the rows of each
    leading index are cut into tiles of ``tile_rows`` consecutive rows (the
    last one ragged), and every tile shares one scale:
      absmax_t = max over the tile's rows and columns of |x|
      scale_t  = float32(absmax_t / 127), 1 if that is 0
      code     = clamp(round_half_even(float32(x / scale_t)), -127, 127)
    (the per-row rule of ``quantize_int8`` with a coarser scale granularity,
    the per-block scales named among the pages' low-precision variants).
    Returns (codes int8 [..., n, d], scales float32 [..., n]) with every row
    carrying its tile's scale, so the int8 attention consumes them as is."""
    x = np.asarray(x, dtype=np.float32)
    assert tile_rows >= 1
    n = x.shape[-2]
    codes = np.empty(x.shape, dtype=np.int8)
    scales = np.empty(x.shape[:-1], dtype=np.float32)
    for r0 in range(0, n, tile_rows):
        r1 = min(n, r0 + tile_rows)
        tile = x[..., r0:r1, :]
        absmax = np.max(np.abs(tile), axis=(-2, -1))
        scale = (absmax / np.float32(127.0)).astype(np.float32)
        scale = np.where(scale == np.float32(0.0), np.float32(1.0), scale).astype(np.float32)
        ratio = (tile / scale[..., None, None]).astype(np.float32)
        codes[..., r0:r1, :] = np.clip(np.rint(ratio), -127.0, 127.0).astype(np.int8)
        scales[..., r0:r1] = scale[..., None]
    return codes, scales


def int8_scores(q_codes, k_codes) -> np.ndarray:
    """Exact integer dot products D = Qc Kc^T of int8 codes, as int64.

    Evaluated as a float64 matmul of integer-valued arrays: every partial sum
    is an integer of magnitude <= d * 127^2 < 2^53, so each one is exact.
    """
    qf = np.asarray(q_codes, dtype=np.float64)
    kf = np.asarray(k_codes, dtype=np.float64)
    d = qf.shape[-1]
    assert d * 127 * 127 < 2 ** 53
    kt = np.swapaxes(kf, -1, -2)
    return np.rint(qf @ kt).astype(np.int64)


def attention_int8_head(q_codes, q_scale, k_codes, k_scale, v, *, causal: bool,
                        scale: float, block_rows: int = 512):
    """Exact attention of one head with scores scale * sq_i * sk_j * D_ij."""
    qf = np.asarray(q_codes, dtype=np.float64)
    kf = np.asarray(k_codes, dtype=np.float64)
    sq = np.asarray(q_scale, dtype=np.float64)
    sk = np.asarray(k_scale, dtype=np.float64)

    def scores(r0, r1, kend):
        dots = qf[r0:r1] @ kf[:kend].T             # exact integers
        return scale * sq[r0:r1, None] * sk[None, :kend] * dots

    return attention_head(qf, kf, v, causal=causal, scale=scale,
                          block_rows=block_rows, scores_fn=scores)


def attention_int8(q_codes, q_scale, k_codes, k_scale, v, *, causal: bool,
                   scale: Optional[float] = None, block_rows: int = 512):
    """[B, H, N, d] int8 codes + [B, H, N] scales, v [B, H, N, dv]."""
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
        o[u], lse[u] = attention_int8_head(qc[u], qs[u], kc[u], ks[u], vf[u],
                                           causal=causal, scale=scale,
                                           block_rows=block_rows)
    return o.reshape(vv.shape), lse.reshape(lead + (n,))


# ---------------------------------------------------------------------------
# delta = rowsum(dO * O), the backward pass's per-row term
# ---------------------------------------------------------------------------

def attention_delta(o, d_o) -> np.ndarray:
    """delta_i = sum_c dO[i, c] * O[i, c] over the last axis, in float64
    ("Why Low-Precision Transformer Training Fails": delta = rowsum(dO o O),
    Figure 5 caption).  o and d_o: [..., N, d] of the same shape."""
    o64 = np.asarray(o, dtype=np.float64)
    g64 = np.asarray(d_o, dtype=np.float64)
    assert o64.shape == g64.shape
    prod = g64 * o64
    return prod.sum(axis=-1)


def attention_backward_head(q, k, v, o, d_o, *, causal: bool, scale: float):
    """Gradients (dQ, dK, dV) of one head's attention in float64, given the
    stored forward output o and the upstream gradient d_o.

    The chain rule through O = P V, P = row-softmax(S), S = scale Q K^T:
        dV = P^T dO,  dP = dO V^T,
        dS = P o (dP - delta 1^T),  delta = rowsum(dO o O)
        dQ = scale dS K,  dK = scale dS^T Q
    ("Why Low-Precision Transformer Training Fails": delta = rowsum(dO o O),
    Figure 5 caption; the section isolating the error in O computes delta
    from the stored low-precision O, so delta here is formed from the o
    passed in; with the exact O this is the exact gradient, since
    rowsum(dP o P) = rowsum(dO o O)).  P is recomputed exactly from q, k.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    g = np.asarray(d_o, dtype=np.float64)
    p = attention_probabilities(q, k, causal=causal, scale=scale)
    delta = (g * o).sum(axis=1)
    dv = p.T @ g
    dp = g @ v.T
    ds = p * (dp - delta[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


# ---------------------------------------------------------------------------
# deviation of a low-precision output from the high-precision one
# ---------------------------------------------------------------------------

def deviation(o_test, o_ref) -> dict:
    """Summary of e = o_test - o_ref over all elements (float64).

    Elements where e is not finite are counted in ``n_nonfinite`` and left out
    of every other statistic.  ``argmax`` is the flat index of the first
    element with the largest |e| (-1 if none is finite); ``max_ref_abs`` is
    over the finite reference values; ``rel_normwise`` = max_abs/max_ref_abs.
    """
    t = np.asarray(o_test, dtype=np.float64).ravel()
    r = np.asarray(o_ref, dtype=np.float64).ravel()
    assert t.shape == r.shape
    n = t.size
    e = t - r
    fin = np.isfinite(e)
    n_fin = int(fin.sum())
    ref_fin = np.isfinite(r)
    max_ref = float(np.abs(r[ref_fin]).max()) if ref_fin.any() else 0.0
    if n_fin == 0:
        nan = float("nan")
        return dict(n=n, n_nonfinite=n, max_abs=nan, mean_abs=nan,
                    mean_signed=nan, rms=nan, max_ref_abs=max_ref,
                    rel_normwise=nan, argmax=-1)
    a = np.where(fin, np.abs(e), -1.0)
    arg = int(np.argmax(a))
    ef = e[fin]
    max_abs = float(a[arg])
    if max_ref > 0:
        rel = max_abs / max_ref
    else:
        rel = 0.0 if max_abs == 0 else float("inf")
    return dict(n=n, n_nonfinite=n - n_fin, max_abs=max_abs,
                mean_abs=float(np.abs(ef).sum() / n_fin),
                mean_signed=float(ef.sum() / n_fin),
                rms=float(math.sqrt((ef * ef).sum() / n_fin)),
                max_ref_abs=max_ref, rel_normwise=rel, argmax=arg)


# ---------------------------------------------------------------------------
# running many heads on the host's cores
# ---------------------------------------------------------------------------

_POOL_STATE = {}


def _pool_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:                              # pragma: no cover
        pass


def _pool_unit(u):
    fn, args, kw = _POOL_STATE["job"]
    return u, fn(u, *args, **kw)


def run_heads(fn, units, *args, workers: Optional[int] = None, **kw):
    """Evaluate ``fn(unit, *args, **kw)`` for each unit in a fork pool of
    ``workers`` processes (one BLAS thread each).  Returns (results in unit
    order, workers used)."""
    units = list(units)
    if workers is None:
        workers = len(os.sched_getaffinity(0))
    workers = max(1, min(workers, len(units)))
    if workers == 1:
        return [fn(u, *args, **kw) for u in units], 1
    import multiprocessing as mp
    _POOL_STATE["job"] = (fn, args, kw)
    ctx = mp.get_context("fork")
    try:
        with ctx.Pool(workers, initializer=_pool_init) as pool:
            out = dict(pool.imap_unordered(_pool_unit, units))
    finally:
        _POOL_STATE.pop("job", None)
    return [out[u] for u in units], workers
