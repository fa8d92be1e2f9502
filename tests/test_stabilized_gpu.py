"""The stabilised FlashAttention variant on the GPU ("Why Low-Precision
Transformer Training Fails", Figure 7 and Algorithm 1: when a row's maximum
score r_m is repeated, the normaliser becomes beta*r_m for r_m > 0 and 0 for
r_m < 0, so no unnormalised probability is exactly 1).

* The normaliser cancels in exact arithmetic, so the FP64 oracle still
  defines the output: parity is checked at the bf16 tolerances.
* Rows whose running maximum is never repeated take the standard path: the
  output is bitwise that of the standard kernel.
* A closed-form case pins the arithmetic: with exactly representable inputs
  the standard kernel's output is exactly 0, while the stabilised one follows
  from the shifted normaliser and the bf16 rounding of the probabilities.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from helpers import assert_close, device_inputs, oracle_inputs, out_to_f64, torch_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _print(*a):
    print(*a, flush=True)


def _bf16_round(x):
    """float64 value of x rounded to fp32, then to bf16 (nearest even)."""
    bits = synth.f32_to_bf16_bits(np.asarray(x, np.float32).reshape(-1))
    return synth.bf16_bits_to_f32(bits).astype(np.float64).reshape(np.shape(x))


def _forward(q, k, v, beta, causal=False, p_bf16=True, lse=False):
    import precision_numerics_amd as pna
    lse_t = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda") if lse else None
    o = pna.attn_fwd_flash(q, k, v, causal=causal, p_bf16=p_bf16, beta=beta, lse=lse_t)
    torch.cuda.synchronize()
    return o, lse_t


@pytest.mark.parametrize("beta", [1.5, 4.0])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p_bf16", [True, False])
def test_stabilized_matches_oracle(lib, beta, d, causal, p_bf16):
    for n in (1, 3, 65, 200, 300):
        cfg = synth.small(synth.CONFIGS["c2"], batch=2, heads=2, seq_len=n, head_dim=d,
                          causal=causal)
        inp = synth.make_inputs(cfg, seed=500 + n)
        q, k, v = device_inputs(inp)
        _print(f"stabilized beta={beta} d={d} causal={causal} p_bf16={p_bf16} n={n}")
        o, lse = _forward(q, k, v, beta, causal, p_bf16, lse=True)
        ref, lse_ref = oracle.attention(*oracle_inputs(inp), causal=causal)
        assert_close(out_to_f64(o), ref, "bf16", f"stabilized n={n}")
        lse = lse.cpu().numpy().astype(np.float64)
        assert np.abs(lse - lse_ref).max() <= 1e-4 * max(1.0, np.abs(lse_ref).max())


def test_stabilized_on_lowrank_workload(lib):
    """Rank-4 correlated Q, K (the long-sequence workload's recipe) at a size
    the oracle finishes quickly: repeated maxima are common there."""
    cfg = synth.small(synth.CONFIGS["c4"], batch=1, heads=2, seq_len=1024)
    inp = synth.make_inputs(cfg)
    q, k, v = device_inputs(inp)
    ref, _ = oracle.attention(*oracle_inputs(inp), causal=True)
    for p_bf16 in (True, False):
        o, _ = _forward(q, k, v, 2.0, True, p_bf16)
        st = assert_close(out_to_f64(o), ref, "bf16", f"low-rank p_bf16={p_bf16}")
        _print(f"low-rank stabilized p_bf16={p_bf16}: {st}")


def _prefix_max_unique(scores: np.ndarray, margin: float) -> np.ndarray:
    """Rows whose running maximum over every key prefix is attained once, with
    the runner-up at least `margin` below it (so fp32 rounding cannot tie)."""
    ok = np.ones(scores.shape[:-1], bool)
    top = np.full(scores.shape[:-1], -np.inf)
    second = np.full(scores.shape[:-1], -np.inf)
    for j in range(scores.shape[-1]):
        s = scores[..., j]
        new_top = np.maximum(top, s)
        second = np.where(s > top, top, np.maximum(second, s))
        top = new_top
        ok &= (top - second) > margin
    return ok


def test_unique_max_rows_match_standard_bitwise(lib):
    cfg = synth.small(synth.CONFIGS["c2"], batch=1, heads=4, seq_len=300, head_dim=64,
                      causal=False)
    inp = synth.make_inputs(cfg, seed=77)
    q, k, v = device_inputs(inp)
    o_std, _ = _forward(q, k, v, None)
    o_stb, _ = _forward(q, k, v, 3.0)
    qq, kk, _ = oracle_inputs(inp)
    scores = np.einsum("bhqd,bhkd->bhqk", qq, kk)
    rows = _prefix_max_unique(scores, 1e-3)
    assert rows.mean() > 0.9
    a = o_std.view(torch.int16).cpu().numpy()
    b = o_stb.view(torch.int16).cpu().numpy()
    assert np.array_equal(a[rows], b[rows])


def _tie_case(sign: int, d=64, n=16):
    """Keys 0 and 8 (different lane halves of the kernel's score tile) share
    the row maximum; every other key scores lower.  V column 0 is chosen so
    that the standard kernel's output there is exactly 0."""
    q = np.zeros((1, 1, n, d), np.float32)
    k = np.zeros((1, 1, n, d), np.float32)
    v = np.zeros((1, 1, n, d), np.float32)
    if sign > 0:
        q[..., 0] = 4.0
        k[:, :, [0, 8], 0] = 4.0       # dot 16 -> scaled score 2 (repeated max)
        # other keys: dot 0 -> score 0;  P2 = exp(-2), bf16(P2) = 139/1024
        v[:, :, [0, 8], 0] = 139.0 / 128.0
        v[:, :, 1, 0] = -16.0          # 2 * 139/128 - 16 * 139/1024 = 0
    elif sign < 0:
        q[..., 0] = -4.0
        k[:, :, [0, 8], 0] = 1.0       # dot -4 -> scaled -0.5 (repeated max)
        k[:, :, [i for i in range(n) if i not in (0, 8)], 0] = 4.0   # dot -16 -> -2
        v[:, :, [0, 8], 0] = 57.0 / 64.0  # bf16(exp(-1.5)) = 57/256
        v[:, :, 1, 0] = -8.0            # 2 * 57/64 - 8 * 57/256 = 0
    else:
        q[..., 0] = 4.0                 # keys 0, 8: dot 0 (repeated max 0)
        k[:, :, [i for i in range(n) if i not in (0, 8)], 0] = -4.0  # dot -16
        v[:, :, [0, 8], 0] = 139.0 / 1024.0
        v[:, :, 1, 0] = -2.0            # 2 * 139/1024 - 2 * 139/1024 = 0
    return q, k, v


def _expected_col0(q, k, v, normaliser, scale):
    """O[...,0] of one row from the FlashAttention arithmetic with the given
    normaliser (natural-log units): P = exp(s - m) in fp32, l = sum P, the
    P.V product on bf16(P) with exact accumulation (the inputs are dyadic)."""
    s = scale * (k[0, 0] @ q[0, 0, 0])              # scores of row 0 (all rows alike)
    p = np.exp(s - normaliser).astype(np.float32).astype(np.float64)
    return float((_bf16_round(p) * v[0, 0, :, 0]).sum() / p.sum())


@pytest.mark.parametrize("sign", [1, -1, 0])
def test_repeated_max_closed_form(lib, sign):
    beta = 2.0
    q, k, v = _tie_case(sign)
    scale = 1.0 / 8.0
    s = scale * (k[0, 0] @ q[0, 0, 0])
    r = float(s.max())
    assert (s == r).sum() == 2
    tq, tk, tv = (torch_bf16(synth.f32_to_bf16_bits(x)) for x in (q, k, v))
    o_std, _ = _forward(tq, tk, tv, None)
    o_stb, _ = _forward(tq, tk, tv, beta)
    std = out_to_f64(o_std)[0, 0, :, 0]
    stb = out_to_f64(o_stb)[0, 0, :, 0]
    exp_std = _expected_col0(q, k, v, r, scale)
    m_stab = beta * r if r > 0 else (0.0 if r < 0 else r)
    assert m_stab - r < MAX_SHIFT_NAT          # inside the range guard
    exp_stb = _expected_col0(q, k, v, m_stab, scale)
    _print(f"sign={sign}: standard {std[0]!r} (expected {exp_std!r}), "
           f"stabilized {stb[0]!r} (expected {exp_stb!r})")
    assert exp_std == 0.0
    assert np.all(std == 0.0)
    if sign == 0:
        assert np.array_equal(o_std.view(torch.int16).cpu(), o_stb.view(torch.int16).cpu())
    else:
        assert abs(exp_stb) > 1e-3
        assert np.all(np.abs(stb - exp_stb) <= 4e-3 * abs(exp_stb) + 1e-7)


# the kernel's range guard: the normaliser stays within 64 (log2 units) of
# the running row max
MAX_SHIFT_NAT = 64.0 * np.log(2.0)


def _far_tie_case(sign: int, d=64, n=40):
    """A repeated row maximum far from 0: r_m = 60.5 (sign > 0; beta = 4 puts
    the page's normaliser 181.5 above it) or r_m = -120 (sign < 0; the
    normaliser 0 is 120 above it).  Either way every exp of the unguarded
    rule underflows in fp32.  Keys 0 and 8 carry the maximum, every other key
    scores at least 60 lower, so the exact output of every row is the mean
    of V rows 0 and 8 (to within e^-60)."""
    q = np.zeros((1, 1, n, d), np.float32)
    k = np.zeros((1, 1, n, d), np.float32)
    v = np.zeros((1, 1, n, d), np.float32)
    rest = [i for i in range(n) if i not in (0, 8)]
    if sign > 0:
        q[..., 0] = 22.0
        k[:, :, [0, 8], 0] = 22.0          # dot 484 -> scaled 60.5
    else:
        q[..., 0] = -32.0
        k[:, :, [0, 8], 0] = 30.0          # dot -960 -> scaled -120
        k[:, :, rest, 0] = 60.0            # dot -1920 -> -240
    v[:, :, :, :] = np.arange(d, dtype=np.float32) / 8.0 - 3.0
    v[:, :, 0, :] = 1.5
    v[:, :, 8, :] = -0.25                  # mean of rows 0 and 8: 0.625
    v[:, :, rest, 1] = 100.0               # weight e^-60 or less: invisible
    return q, k, v


@pytest.mark.parametrize("sign", [1, -1])
@pytest.mark.parametrize("p_bf16", [True, False])
def test_range_guard_keeps_far_repeated_max_finite(lib, sign, p_bf16):
    """The page's rule alone would give O = 0/0 here; with the guard the
    largest probability is 2^-64 (exactly, after the bf16 rounding of P) and
    the output is the exact softmax's: the mean of V rows 0 and 8, as the
    FP64 oracle and the standard kernel give."""
    beta = 4.0
    q, k, v = _far_tie_case(sign)
    scale = 1.0 / 8.0
    s = scale * (k[0, 0] @ q[0, 0, 0])
    r = float(s.max())
    assert (s == r).sum() == 2 and np.sort(s)[-3] <= r - 60
    m_rule = beta * r if r > 0 else 0.0
    assert (m_rule - r) * np.log2(np.e) > 149      # fp32 exp2 underflows everywhere
    tq, tk, tv = (torch_bf16(synth.f32_to_bf16_bits(x)) for x in (q, k, v))
    o_std, _ = _forward(tq, tk, tv, None, p_bf16=p_bf16)
    o_stb, lse = _forward(tq, tk, tv, beta, p_bf16=p_bf16, lse=True)
    ref, lse_ref = oracle.attention(*(x.astype(np.float64) for x in (q, k, v)), causal=False)
    stb, std = out_to_f64(o_stb), out_to_f64(o_std)
    _print(f"sign={sign} p_bf16={p_bf16}: r_m={r} stabilized O[0,:4]={stb[0, 0, 0, :4]} "
           f"ref={ref[0, 0, 0, :4]}")
    assert np.all(np.isfinite(stb))
    want = 0.5 * (v[0, 0, 0] + v[0, 0, 8]).astype(np.float64)
    assert np.array_equal(stb[0, 0], np.broadcast_to(want, stb[0, 0].shape))
    assert np.array_equal(std, stb)
    assert np.abs(ref - want).max() <= 1e-12
    assert np.abs(lse.cpu().numpy().astype(np.float64) - lse_ref).max() <= 1e-4 * abs(r)
