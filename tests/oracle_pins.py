"""Pins of the FP64 oracle to things other than itself.

Each ``check_*`` takes a module that exposes the oracle's API and raises
AssertionError when the module disagrees with what the mathematics fixes:
a high-precision brute force written differently (no max shift, decimal
arithmetic), a library routine (torch's float64 scaled-dot-product attention
on the CPU), closed forms and invariants of softmax attention, and exact
integer arithmetic for the int8 path.  ``test_oracle.py`` runs them on the
oracle; ``test_oracle_mutants.py`` runs them on copies of the oracle with one
planted mistake each and requires every copy to fail at least one of them.
"""
from __future__ import annotations

import math
from decimal import Decimal, getcontext

import numpy as np

PINS = []


def pin(fn):
    PINS.append(fn)
    return fn


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# brute force: scalar decimal arithmetic, softmax without a max shift
# ---------------------------------------------------------------------------

def brute_force_attention(q, k, v, causal, scale):
    """sum_j exp(s_ij) v_j / sum_j exp(s_ij) at 50 significant digits."""
    getcontext().prec = 50
    n, d = q.shape
    dv = v.shape[1]
    sc = Decimal(scale)
    out = np.zeros((n, dv))
    lse = np.zeros(n)
    for i in range(n):
        num = [Decimal(0)] * dv
        den = Decimal(0)
        for j in range(k.shape[0]):
            if causal and j > i:
                continue
            dot = sum((Decimal(float(q[i, t])) * Decimal(float(k[j, t])) for t in range(d)),
                      Decimal(0))
            w = (sc * dot).exp()
            den += w
            for c in range(dv):
                num[c] += w * Decimal(float(v[j, c]))
        for c in range(dv):
            out[i, c] = float(num[c] / den)
        lse[i] = float(den.ln())
    return out, lse


@pin
def check_brute_force(ora):
    for seed, (n, d, dv, causal) in enumerate([(1, 3, 2, False), (5, 4, 3, True),
                                               (6, 3, 5, False), (7, 2, 2, True)]):
        rng = _rng(100 + seed)
        q = rng.standard_normal((n, d)) * 1.7
        k = rng.standard_normal((n, d)) * 1.3
        v = rng.standard_normal((n, dv))
        scale = 1.0 / math.sqrt(d)
        o, lse = ora.attention(q, k, v, causal=causal, scale=scale, block_rows=3)
        ob, lb = brute_force_attention(q, k, v, causal, scale)
        assert np.allclose(o, ob, rtol=0, atol=1e-13), np.abs(o - ob).max()
        assert np.allclose(lse, lb, rtol=0, atol=1e-13), np.abs(lse - lb).max()


# ---------------------------------------------------------------------------
# library routine: torch float64 SDPA on the CPU
# ---------------------------------------------------------------------------

@pin
def check_torch_sdpa(ora):
    import torch
    import torch.nn.functional as F
    rng = _rng(7)
    for causal in (False, True):
        for (b, h, n, d, block) in [(2, 3, 37, 16, 8), (1, 2, 130, 64, 64)]:
            q = rng.standard_normal((b, h, n, d))
            k = rng.standard_normal((b, h, n, d))
            v = rng.standard_normal((b, h, n, d))
            o, _ = ora.attention(q, k, v, causal=causal, block_rows=block)
            ref = F.scaled_dot_product_attention(
                torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                is_causal=causal, scale=1.0 / math.sqrt(d)).numpy()
            assert np.allclose(o, ref, rtol=0, atol=1e-12), np.abs(o - ref).max()


# ---------------------------------------------------------------------------
# closed forms and invariants
# ---------------------------------------------------------------------------

@pin
def check_default_scale(ora):
    assert ora.default_scale(64) == 0.125
    # 1/sqrt(128) = sqrt(2)/16
    assert abs(ora.default_scale(128) - math.sqrt(2.0) / 16.0) <= 2.0 ** -56
    assert ora.default_scale(1) == 1.0


@pin
def check_two_key_closed_form(ora):
    """One query, two keys: O = sigma(s1 - s0) v1 + (1 - sigma) v0."""
    for a in (-3.0, -0.25, 0.0, 0.7, 5.0):
        q = np.array([[a, 0.0]])
        k = np.array([[0.0, 1.0], [1.0, 1.0]])          # s0 = 0, s1 = a * scale
        v = np.array([[2.0, -1.0], [-4.0, 3.0]])
        scale = 1.0 / math.sqrt(2.0)
        o, lse = ora.attention(q, k, v, causal=False, scale=scale)
        w1 = 1.0 / (1.0 + math.exp(-a * scale))
        expect = w1 * v[1] + (1.0 - w1) * v[0]
        assert np.allclose(o[0], expect, rtol=0, atol=1e-15)
        assert abs(lse[0] - math.log(1.0 + math.exp(a * scale))) < 1e-14


@pin
def check_zero_query_is_mean(ora):
    """Q = 0 gives equal weights: the column mean of V, or of the causal prefix."""
    rng = _rng(11)
    n, d = 45, 8
    q = np.zeros((n, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    o, lse = ora.attention(q, k, v, causal=False, block_rows=16)
    assert np.allclose(o, v.mean(axis=0)[None, :], rtol=0, atol=1e-14)
    assert np.allclose(lse, math.log(n), rtol=0, atol=1e-14)
    o, lse = ora.attention(q, k, v, causal=True, block_rows=16)
    prefix = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.allclose(o, prefix, rtol=0, atol=1e-14)
    assert np.allclose(lse, np.log(np.arange(1, n + 1)), rtol=0, atol=1e-14)


@pin
def check_key_value_permutation(ora):
    """Non-causal attention is invariant to permuting keys with their values."""
    rng = _rng(12)
    n, d = 50, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    perm = rng.permutation(n)
    o1, l1 = ora.attention(q, k, v, causal=False, block_rows=16)
    o2, l2 = ora.attention(q, k[perm], v[perm], causal=False, block_rows=16)
    assert np.allclose(o1, o2, rtol=0, atol=1e-13)
    assert np.allclose(l1, l2, rtol=0, atol=1e-13)


@pin
def check_rows_of_p_sum_to_one(ora):
    rng = _rng(13)
    for causal in (False, True):
        q, k = (rng.standard_normal((33, 5)) * 2 for _ in range(2))
        p = ora.attention_probabilities(q, k, causal=causal, scale=0.6)
        assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        assert (p >= 0).all()
        if causal:
            assert (np.triu(p, 1) == 0).all()


@pin
def check_probabilities_drive_output(ora):
    """O equals P V for the P the oracle reports (and P matches brute force)."""
    rng = _rng(14)
    q, k, v = (rng.standard_normal((9, 4)) for _ in range(3))
    for causal in (False, True):
        p = ora.attention_probabilities(q, k, causal=causal, scale=0.5)
        o, _ = ora.attention(q, k, v, causal=causal, scale=0.5, block_rows=4)
        assert np.allclose(o, p @ v, rtol=0, atol=1e-14)
        ones = np.eye(9)
        pb, _ = brute_force_attention(q, k, ones, causal, 0.5)
        assert np.allclose(p, pb, rtol=0, atol=1e-14)


@pin
def check_causal_special_rows(ora):
    """Causal row 0 sees only key 0 (O_0 = V_0); N = 1 gives O = V; a constant
    V gives that constant; adding one vector to every key changes nothing."""
    rng = _rng(15)
    n, d = 40, 6
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    o, _ = ora.attention(q, k, v, causal=True, block_rows=8)
    assert np.array_equal(o[0], v[0])
    o1, _ = ora.attention(q[:1], k[:1], v[:1], causal=False)
    assert np.allclose(o1, v[:1], rtol=0, atol=1e-15)
    const = np.tile(rng.standard_normal((1, d)), (n, 1))
    for causal in (False, True):
        oc, _ = ora.attention(q, k, const, causal=causal, block_rows=8)
        assert np.allclose(oc, const, rtol=0, atol=1e-14)
        u = rng.standard_normal((1, d))
        oa, la = ora.attention(q, k, v, causal=causal, block_rows=8)
        ob, lb = ora.attention(q, k + u, v, causal=causal, block_rows=8)
        assert np.allclose(oa, ob, rtol=0, atol=1e-12)
        shift = (q @ u.T)[:, 0] / math.sqrt(d)
        assert np.allclose(lb - la, shift, rtol=0, atol=1e-12)


@pin
def check_large_scores_hard_limit(ora):
    """Huge scores must not overflow: the softmax tends to a hard argmax."""
    rng = _rng(16)
    n, d = 24, 4
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    q = 4000.0 * k[[5, 17, 3]]                 # each query aligns with one key
    o, lse = ora.attention(q, k, v, causal=False, scale=1.0, block_rows=2)
    s = q @ k.T
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.allclose(o, v[np.argmax(s, axis=1)], rtol=0, atol=1e-12)
    assert np.allclose(lse, s.max(axis=1), rtol=1e-15, atol=0)
    q2 = np.concatenate([q, -q])              # row maxima of very different size
    p = ora.attention_probabilities(q2, k, causal=False, scale=1.0)
    s2 = q2 @ k.T
    assert np.all(np.isfinite(p))
    assert np.array_equal(np.argmax(p, axis=1), np.argmax(s2, axis=1))
    assert np.allclose(p.max(axis=1), 1.0, rtol=0, atol=1e-12)


@pin
def check_blocking_is_invisible(ora):
    """The row-block size is a memory measure only: results agree to rounding."""
    rng = _rng(17)
    q, k, v = (rng.standard_normal((2, 2, 70, 8)) for _ in range(3))
    for causal in (False, True):
        ref, lref = ora.attention(q, k, v, causal=causal, block_rows=70)
        for br in (1, 3, 16, 64):
            o, l = ora.attention(q, k, v, causal=causal, block_rows=br)
            assert np.allclose(o, ref, rtol=0, atol=1e-14)
            assert np.allclose(l, lref, rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# int8 path
# ---------------------------------------------------------------------------

@pin
def check_int8_scores_exact(ora):
    """D equals the Python-integer dot products, including the extremes."""
    rng = _rng(18)
    qc = rng.integers(-127, 128, size=(2, 11, 128), dtype=np.int64).astype(np.int8)
    kc = rng.integers(-127, 128, size=(2, 13, 128), dtype=np.int64).astype(np.int8)
    qc[0, 0, :] = 127
    kc[0, 0, :] = 127
    kc[0, 1, :] = -127
    dots = ora.int8_scores(qc, kc)
    assert dots.dtype == np.int64
    for b in range(2):
        for i in range(11):
            for j in range(13):
                exact = sum(int(x) * int(y) for x, y in zip(qc[b, i], kc[b, j]))
                assert dots[b, i, j] == exact
    assert dots[0, 0, 0] == 128 * 127 * 127
    assert dots[0, 0, 1] == -128 * 127 * 127


@pin
def check_int8_attention_matches_dequantised(ora):
    """int8 attention equals float attention on the dequantised rows
    sq_i * code_i (the scores are scale * sq_i * sk_j * D_ij)."""
    rng = _rng(19)
    n, d = 21, 16
    qc = rng.integers(-127, 128, size=(n, d)).astype(np.int8)
    kc = rng.integers(-127, 128, size=(n, d)).astype(np.int8)
    sq = rng.uniform(0.001, 0.03, size=n).astype(np.float32)
    sk = rng.uniform(0.001, 0.03, size=n).astype(np.float32)
    v = rng.standard_normal((n, d))
    for causal in (False, True):
        o, lse = ora.attention_int8(qc, sq, kc, sk, v, causal=causal, block_rows=5)
        qd = qc.astype(np.float64) * sq.astype(np.float64)[:, None]
        kd = kc.astype(np.float64) * sk.astype(np.float64)[:, None]
        ob, lb = brute_force_attention(qd, kd, v, causal, 1.0 / math.sqrt(d))
        assert np.allclose(o, ob, rtol=0, atol=1e-13)
        assert np.allclose(lse, lb, rtol=0, atol=1e-13)


@pin
def check_quantiser(ora):
    # a row whose absmax is 127 has scale exactly 1: codes are rint(x), with
    # ties to even
    row = np.array([[127.0, 0.5, 1.5, 2.5, -2.5, -0.5, 3.49, -126.5]], np.float32)
    codes, scale = ora.quantize_int8(row)
    assert scale.dtype == np.float32 and scale[0] == 1.0
    assert codes.tolist() == [[127, 0, 2, 2, -2, 0, 3, -126]]
    # absmax = 0 -> scale 1, codes 0
    codes, scale = ora.quantize_int8(np.zeros((2, 8), np.float32))
    assert (codes == 0).all() and (scale == 1.0).all()
    # random rows: the absmax element maps to +-127, codes are odd-symmetric,
    # and every code reconstructs its value within half a step
    rng = _rng(20)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    codes, scale = ora.quantize_int8(x)
    c2, s2 = ora.quantize_int8(-x)
    assert np.array_equal(c2, -codes) and np.array_equal(s2, scale)
    am = np.abs(x).max(axis=1)
    # fp64 quotient rounded once to fp32 is the correctly rounded fp32 quotient
    # (53 >= 2*24 + 2), an independent route to the same scale
    assert np.array_equal(scale, (am.astype(np.float64) / 127).astype(np.float32))
    idx = np.abs(x).argmax(axis=1)
    assert (np.abs(codes[np.arange(64), idx]) == 127).all()
    err = np.abs(codes.astype(np.float64) * scale[:, None] - x.astype(np.float64))
    assert (err <= scale[:, None].astype(np.float64) * (0.5 + 1e-5)).all()
    assert codes.dtype == np.int8 and np.abs(codes.astype(int)).max() <= 127


# ---------------------------------------------------------------------------
# deviation summary
# ---------------------------------------------------------------------------

@pin
def check_deviation(ora):
    rng = _rng(21)
    ref = rng.integers(-4096, 4096, size=1000) / 1024.0        # exact binary values
    # a single spike
    test = ref.copy()
    test[417] += 0.25
    st = ora.deviation(test, ref)
    assert st["max_abs"] == 0.25 and st["argmax"] == 417
    assert st["mean_abs"] == 0.25 / 1000 and st["mean_signed"] == 0.25 / 1000
    assert abs(st["rms"] - math.sqrt(0.0625 / 1000)) < 1e-18
    assert st["n"] == 1000 and st["n_nonfinite"] == 0
    assert st["max_ref_abs"] == np.abs(ref).max()
    assert st["rel_normwise"] == 0.25 / np.abs(ref).max()
    # a constant negative offset: signed mean is the offset, mean |e| its size
    st = ora.deviation(ref - 2.0 ** -10, ref)
    assert st["mean_signed"] == -(2.0 ** -10) and st["mean_abs"] == 2.0 ** -10
    assert st["max_abs"] == 2.0 ** -10 and st["argmax"] == 0
    # ties in |e| report the first index; non-finite elements are counted
    test = ref.copy()
    test[[10, 20]] += 1.0
    test[30] = np.nan
    test[40] = np.inf
    st = ora.deviation(test, ref)
    assert st["argmax"] == 10 and st["max_abs"] == 1.0 and st["n_nonfinite"] == 2
    assert st["mean_abs"] == 2.0 / 998
    assert ora.deviation(ref, ref)["max_abs"] == 0.0


# ---------------------------------------------------------------------------
# delta = rowsum(dO * O)
# ---------------------------------------------------------------------------

@pin
def check_delta(ora):
    """Brute force with exact float sums; closed forms (dO = O gives the row's
    squared norm, a unit dO picks one column); and the backward identity
    rowsum(dO o O) = rowsum(P o (dO V^T)) for O = P V, which ties delta to
    the attention probabilities."""
    rng = _rng(41)
    o = rng.standard_normal((3, 5, 7))
    g = rng.standard_normal((3, 5, 7))
    got = ora.attention_delta(o, g)
    assert got.shape == (3, 5)
    for a in range(3):
        for i in range(5):
            exact = math.fsum(float(g[a, i, c]) * float(o[a, i, c]) for c in range(7))
            assert abs(got[a, i] - exact) <= 1e-14 * max(1.0, abs(exact))
    sq = ora.attention_delta(o, o)
    assert np.allclose(sq, (o ** 2).sum(-1), rtol=1e-14, atol=0)
    e2 = np.zeros_like(o)
    e2[..., 2] = 1.0
    assert np.array_equal(ora.attention_delta(o, e2), o[..., 2])
    # delta through the attention probabilities
    q = rng.standard_normal((9, 4))
    k = rng.standard_normal((9, 4))
    v = rng.standard_normal((9, 6))
    d_o = rng.standard_normal((9, 6))
    for causal in (False, True):
        out, _ = ora.attention(q, k, v, causal=causal, scale=0.5)
        p = ora.attention_probabilities(q, k, causal=causal, scale=0.5)
        via_p = (p * (d_o @ v.T)).sum(axis=1)
        assert np.allclose(ora.attention_delta(out, d_o), via_p, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# Wasserstein distances between empirical distributions
# ---------------------------------------------------------------------------

def _brute_force_w(u, v):
    """Optimal transport between two uniform samples of equal size by
    enumeration of every pairing: W_1, W_2, W_inf."""
    import itertools
    n = len(u)
    best1 = best2 = bestinf = math.inf
    for perm in itertools.permutations(range(n)):
        gaps = [abs(u[i] - v[perm[i]]) for i in range(n)]
        best1 = min(best1, math.fsum(gaps) / n)
        best2 = min(best2, math.fsum(g * g for g in gaps) / n)
        bestinf = min(bestinf, max(gaps))
    return best1, math.sqrt(best2), bestinf


def _lp_transport(u, v, power):
    """min sum_ij |u_i - v_j|^power g_ij over couplings g of the uniform
    distributions on u (n atoms) and v (m atoms): the transport linear
    program, solved by scipy's HiGHS."""
    from scipy.optimize import linprog
    n, m = len(u), len(v)
    cost = np.abs(np.subtract.outer(np.asarray(u), np.asarray(v))) ** power
    a_eq = np.zeros((n + m, n * m))
    for i in range(n):
        a_eq[i, i * m:(i + 1) * m] = 1.0
    for j in range(m):
        a_eq[n + j, j::m] = 1.0
    b_eq = np.concatenate((np.full(n, 1.0 / n), np.full(m, 1.0 / m)))
    res = linprog(cost.ravel(), A_eq=a_eq, b_eq=b_eq, bounds=(0, None), method="highs")
    assert res.status == 0
    return res.fun


@pin
def check_wasserstein(ora):
    """W_p from the quantile functions against: enumeration of every pairing
    (equal sizes, with ties), the transport linear program (unequal sizes),
    the distribution-function area formula and scipy for p = 1, and closed
    forms (point masses, a two-point law, shifts, scaling, symmetry)."""
    rng = _rng(51)
    for n in range(1, 7):
        for trial in range(3):
            u = rng.standard_normal(n).round(1 if trial == 2 else 12)
            v = rng.standard_normal(n).round(1 if trial == 2 else 12)
            w = ora.wasserstein(u, v)
            b1, b2, binf = _brute_force_w(list(u), list(v))
            assert abs(w["w1"] - b1) <= 1e-12 and abs(w["w2"] - b2) <= 1e-12, (w, b1, b2)
            assert w["winf"] == binf and w["n_nonfinite"] == 0
    for n, m in ((1, 3), (2, 3), (3, 5), (4, 6), (7, 2)):
        u = rng.standard_normal(n)
        v = rng.standard_normal(m) * 2.0 + 0.3
        w = ora.wasserstein(u, v)
        assert abs(w["w1"] - _lp_transport(u, v, 1)) <= 1e-9
        assert abs(w["w2"] ** 2 - _lp_transport(u, v, 2)) <= 1e-9
        assert abs(w["w1"] - ora.wasserstein1_cdf(u, v)) <= 1e-12
    from scipy.stats import wasserstein_distance
    for n, m in ((50, 50), (37, 91), (500, 3)):
        u = rng.standard_normal(n) ** 3
        v = rng.gamma(2.0, size=m) - 1.0
        ref = wasserstein_distance(u, v)
        assert abs(ora.wasserstein(u, v)["w1"] - ref) <= 1e-12 * max(1.0, ref)
        assert abs(ora.wasserstein1_cdf(u, v) - ref) <= 1e-12 * max(1.0, ref)
    # closed forms
    w = ora.wasserstein([2.5], [-1.0])
    assert w["w1"] == 3.5 and w["w2"] == 3.5 and w["winf"] == 3.5
    w = ora.wasserstein([0.0, 1.0], [0.0])
    assert w["w1"] == 0.5 and abs(w["w2"] - math.sqrt(0.5)) <= 1e-15 and w["winf"] == 1.0
    assert ora.wasserstein1_cdf([0.0, 1.0], [0.0]) == 0.5
    u = rng.standard_normal(1000)
    w = ora.wasserstein(u, u + 0.75)       # a shift moves every quantile by 0.75
    for key in ("w1", "w2", "winf"):
        assert abs(w[key] - 0.75) <= 1e-12
    w0 = ora.wasserstein(u, rng.permutation(u))
    assert w0["w1"] == 0.0 and w0["winf"] == 0.0
    v = rng.standard_normal(700)
    a, b = ora.wasserstein(u, v), ora.wasserstein(v, u)
    c = ora.wasserstein(-3.0 * u, -3.0 * v)
    for key in ("w1", "w2", "winf"):
        assert abs(a[key] - b[key]) <= 1e-15 * max(1.0, a[key])
        assert abs(c[key] - 3.0 * a[key]) <= 1e-12 * max(1.0, a[key])
    # non-finite inputs
    w = ora.wasserstein([1.0, float("nan"), float("inf")], [0.0, 1.0, 2.0])
    assert w["n_nonfinite"] == 2 and math.isnan(w["w1"]) and math.isnan(w["winf"])


# ---------------------------------------------------------------------------
# E4M3 fp8 Q/K path
# ---------------------------------------------------------------------------

def _torch_e4m3():
    import torch
    return torch, torch.float8_e4m3fn


@pin
def check_e4m3_codec(ora):
    """Decode and encode against torch's float8_e4m3fn (all 256 patterns;
    round to nearest even inside the range), closed forms for ties,
    saturation, signed zero and NaN, and the round trip of every code."""
    torch, f8 = _torch_e4m3()
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(f8).float().double().numpy()
    got = ora.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))
    rng = _rng(61)
    x = np.concatenate([rng.standard_normal(20000) * 40.0,
                        rng.standard_normal(5000) * 2.0 ** -8,           # subnormal range
                        ora.e4m3_decode(rng.integers(0, 0x7f, 3000)) * (1 + 2.0 ** -4),
                        (ora.e4m3_decode(np.arange(1, 0x7e)) +
                         ora.e4m3_decode(np.arange(2, 0x7f))) / 2]).astype(np.float32)
    x = x[np.abs(x) < 464]
    tq = torch.from_numpy(x).to(f8).view(torch.uint8).numpy()
    assert np.array_equal(ora.e4m3_encode(x), tq)
    fin_codes = np.array([c for c in range(256) if (c & 0x7f) != 0x7f], dtype=np.uint8)
    assert np.array_equal(ora.e4m3_encode(ora.e4m3_decode(fin_codes)), fin_codes)
    assert ora.e4m3_decode([0x38])[0] == 1.0 and ora.e4m3_decode([0x7e])[0] == 448.0
    assert ora.e4m3_decode([0x01])[0] == 2.0 ** -9 and ora.e4m3_decode([0x08])[0] == 2.0 ** -6
    enc = ora.e4m3_encode(np.array([1.0625, 1.1875, 449.0, 1e4, -1e4, -0.0, 2.0 ** -10,
                                    3 * 2.0 ** -10, np.nan]))
    assert list(enc) == [0x38, 0x3A, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x02, 0x7F], list(enc)


@pin
def check_fp8_quantiser(ora):
    """Per-row E4M3 quantiser: the row maximum maps to +-448, every code is
    finite, the dequantised value is within half a spacing (1/16 relative,
    or 2^-10 * scale in the subnormal range) of x, and an all-zero row gets
    scale 1 and zero codes."""
    rng = _rng(67)
    x = (rng.standard_normal((40, 96)) * np.exp(rng.standard_normal((40, 1)) * 3)).astype(np.float32)
    x[3] = 0.0
    codes, scale = ora.quantize_fp8(x)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32 and scale.shape == (40,)
    assert np.all((codes & 0x7F) != 0x7F)
    assert scale[3] == 1.0 and not codes[3].any()
    vals = ora.e4m3_decode(codes)
    for r in range(40):
        if r == 3:
            continue
        i = int(np.argmax(np.abs(x[r])))
        assert abs(vals[r, i]) == 448.0
        assert np.array_equal(np.signbit(vals[r]), np.signbit(x[r]))
        err = np.abs(vals[r] * np.float64(scale[r]) - x[r].astype(np.float64))
        bound = np.maximum(np.abs(x[r]) / 16.0, 2.0 ** -10 * scale[r]) * (1 + 1e-6)
        assert np.all(err <= bound)
    assert np.float32(np.abs(x[0]).max() / np.float32(448.0)) == scale[0]


@pin
def check_fp8_scores_and_attention(ora):
    """Dot products of decoded codes equal exact integer arithmetic (every
    value is an integer multiple of 2^-9), and fp8 attention equals the
    plain oracle on the dequantised Q and K."""
    rng = _rng(71)
    qc = rng.integers(0, 256, (6, 16)).astype(np.uint8)
    kc = rng.integers(0, 256, (5, 16)).astype(np.uint8)
    qc[(qc & 0x7F) == 0x7F] = 0x3C
    kc[(kc & 0x7F) == 0x7F] = 0xB1
    got = ora.fp8_scores(qc, kc)
    qi = [[int(round(float(v) * 512)) for v in row] for row in ora.e4m3_decode(qc)]
    ki = [[int(round(float(v) * 512)) for v in row] for row in ora.e4m3_decode(kc)]
    for i in range(6):
        for j in range(5):
            exact = sum(a * b for a, b in zip(qi[i], ki[j]))
            assert got[i, j] == exact / 2.0 ** 18
    q = rng.standard_normal((2, 3, 40, 32)).astype(np.float32)
    k = rng.standard_normal((2, 3, 40, 32)).astype(np.float32) * 3
    v = rng.standard_normal((2, 3, 40, 32))
    qq, qs = ora.quantize_fp8(q)
    kq, ks = ora.quantize_fp8(k)
    for causal in (False, True):
        o, lse = ora.attention_fp8(qq, qs, kq, ks, v, causal=causal, scale=0.3)
        qd = ora.e4m3_decode(qq) * qs[..., None].astype(np.float64)
        kd = ora.e4m3_decode(kq) * ks[..., None].astype(np.float64)
        o2, lse2 = ora.attention(qd, kd, v, causal=causal, scale=0.3)
        assert np.allclose(o, o2, rtol=1e-12, atol=1e-13)
        assert np.allclose(lse, lse2, rtol=1e-12, atol=1e-13)


@pin
def check_int8_tile_quantiser(ora):
    """Per-tile int8 scales: one-row tiles reproduce the per-row quantiser,
    whole-head tiles use the head's absmax, every tile's maximum maps to
    +-127 with rows sharing its scale, tiles restart at every head, and a
    hand-worked tile (scale 0.5: ties to even) gives its codes exactly."""
    rng = _rng(73)
    x = (rng.standard_normal((2, 3, 37, 20)) * np.exp(rng.standard_normal((2, 3, 37, 1)))
         ).astype(np.float32)
    c1, s1 = ora.quantize_int8_tiles(x, 1)
    c0, s0 = ora.quantize_int8(x)
    assert np.array_equal(c1, c0) and np.array_equal(s1, s0)
    cn, sn = ora.quantize_int8_tiles(x, 10 ** 6)
    head_max = np.abs(x).max(axis=(-2, -1))
    assert np.array_equal(sn, np.repeat((head_max / np.float32(127))[..., None], 37, axis=-1))
    for t in (4, 16):
        ct, st = ora.quantize_int8_tiles(x, t)
        for r0 in range(0, 37, t):
            r1 = min(37, r0 + t)
            tile_s = st[..., r0:r1]
            assert np.all(tile_s == tile_s[..., :1])
            amax = np.abs(ct[..., r0:r1, :].astype(np.int32)).max(axis=(-2, -1))
            assert np.all(amax == 127)
            assert np.array_equal(tile_s[..., 0],
                                  (np.abs(x[..., r0:r1, :]).max(axis=(-2, -1)) / np.float32(127)))
    y = np.zeros((1, 5, 2), dtype=np.float32)
    y[0, :, 0] = [63.5, -0.25, 0.75, 1.25, 0.0]
    y[0, :, 1] = [-63.5, 0.5, 20.0, -0.75, 0.0]
    cy, sy = ora.quantize_int8_tiles(y, 2)   # tiles: rows 0-1, 2-3, 4
    assert list(sy[0]) == [0.5, 0.5, np.float32(20.0) / np.float32(127), np.float32(20.0) / np.float32(127), 1.0]
    assert list(cy[0, 0]) == [127, -127] and list(cy[0, 1]) == [0, 1]   # -0.5 -> 0, 1.0 -> 1
    assert list(cy[0, 4]) == [0, 0]


# ---------------------------------------------------------------------------
# attention backward (dQ, dK, dV)
# ---------------------------------------------------------------------------

def _torch_grads(q, k, v, g, causal, scale):
    import torch
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * (tq @ tk.T)
    if causal:
        n = s.shape[0]
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    out = torch.softmax(s, dim=1) @ tv
    out.backward(torch.tensor(g, dtype=torch.float64))
    return out.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pin
def check_backward(ora):
    """Gradients against torch float64 autograd of the plain attention (a
    library routine), against central finite differences of
    L = sum(dO o O), closed forms (each dS row sums to 0, so the dK rows sum
    to 0; the dV rows sum to the dO rows; equal keys give dQ = 0), and the
    stored-O reading: perturbing o by E shifts dQ and dK by exactly the
    delta change rowsum(dO o E) and leaves dV alone."""
    rng = _rng(83)
    for causal in (False, True):
        for n, d, dv_ in ((1, 3, 2), (5, 4, 3), (9, 6, 5)):
            q = rng.standard_normal((n, d))
            k = rng.standard_normal((n, d))
            v = rng.standard_normal((n, dv_))
            g = rng.standard_normal((n, dv_))
            o, tq, tk, tv = _torch_grads(q, k, v, g, causal, 0.7)
            dq, dk, dvv = ora.attention_backward_head(q, k, v, o, g, causal=causal, scale=0.7)
            for a, b in ((dq, tq), (dk, tk), (dvv, tv)):
                assert np.allclose(a, b, rtol=1e-10, atol=1e-12), np.abs(a - b).max()
            assert np.allclose(dk.sum(axis=0), 0.0, atol=1e-12)
            assert np.allclose(dvv.sum(axis=0), g.sum(axis=0), rtol=1e-12, atol=1e-12)
            e = rng.standard_normal(o.shape) * 1e-3
            dq2, dk2, dv2 = ora.attention_backward_head(q, k, v, o + e, g, causal=causal, scale=0.7)
            p = ora.attention_probabilities(q, k, causal=causal, scale=0.7)
            dd = (g * e).sum(axis=1)
            assert np.allclose(dq2 - dq, -0.7 * (dd[:, None] * (p @ k)), rtol=1e-9, atol=1e-14)
            assert np.allclose(dk2 - dk, -0.7 * ((p * dd[:, None]).T @ q), rtol=1e-9, atol=1e-14)
            assert np.array_equal(dv2, dvv)
    # central differences of L(q, k, v) = sum(g o O)
    n, d = 6, 4
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    for causal in (False, True):
        def loss(qq, kk, vv):
            return float((g * ora.attention(qq, kk, vv, causal=causal, scale=0.9)[0]).sum())
        o = ora.attention(q, k, v, causal=causal, scale=0.9)[0]
        grads = ora.attention_backward_head(q, k, v, o, g, causal=causal, scale=0.9)
        h = 1e-6
        for which, grad in enumerate(grads):
            for (i, j) in ((0, 0), (2, 3), (5, 1)):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][i, j] += h
                up = loss(*args)
                args[which][i, j] -= 2 * h
                dn = loss(*args)
                fd = (up - dn) / (2 * h)
                assert abs(fd - grad[i, j]) <= 1e-6 * max(1.0, abs(fd)), (which, i, j, fd, grad[i, j])
    # equal keys: constant score rows, dQ = 0
    kk = np.tile(rng.standard_normal((1, d)), (n, 1))
    o = ora.attention(q, kk, v, causal=False, scale=0.9)[0]
    dq, _, _ = ora.attention_backward_head(q, kk, v, o, g, causal=False, scale=0.9)
    assert np.allclose(dq, 0.0, atol=1e-12)
