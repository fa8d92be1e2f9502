"""Wasserstein distances on the GPU (W1, W2, W_inf between the value
distributions of two tensors: "Is Flash Attention Stable?", abstract, and
"Statistical Aspects of Wasserstein Distances" in its reference list),
against the FP64 oracle's quantile-function definition.

The GPU radix-sorts both inputs and pairs order statistics; the oracle
integrates the two quantile functions.  Sorted pairs are the same on both
sides, so W_inf (a max of exact fp64 differences) is bitwise equal; W1 and
W2 differ only by the order of the fp64 sums (relative 1e-12).  Inputs
cover every dtype pair, ties, signed zeros, subnormals, huge magnitudes,
sizes that are not multiples of the tile or the workgroup chunk, and
non-finite values; then the attention outputs of one workload.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from helpers import device_inputs, oracle_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TORCH_DT = {"f32": "float32", "bf16": "bfloat16", "f64": "float64"}


def _print(*a):
    print(*a, flush=True)


def _draw(rng, n, kind):
    if kind == "normal":
        x = rng.standard_normal(n)
    elif kind == "ties":
        x = rng.integers(-3, 4, n).astype(np.float64) * 0.5
    elif kind == "wide":
        x = rng.standard_normal(n) * np.exp2(rng.integers(-140, 120, n))
    else:  # signed zeros and (fp32/bf16) subnormals among normal values
        x = rng.standard_normal(n)
        u = rng.random(n)
        x[u < 0.2] = 0.0
        x[(u >= 0.2) & (u < 0.4)] = -0.0
        x[(u >= 0.4) & (u < 0.5)] *= 1e-39
    return x


def _as(x, dt):
    """(device tensor, exact float64 values it holds)."""
    t = torch.from_numpy(np.ascontiguousarray(x)).to(getattr(torch, TORCH_DT[dt]))
    return t.cuda(), t.double().numpy()


def _check(pna, a_np, b_np, what):
    got = pna.attn_wasserstein(a_np[0], b_np[0])
    ref = oracle.wasserstein(a_np[1], b_np[1])
    assert got["n"] == a_np[1].size and got["n_nonfinite"] == 0, (what, got)
    assert got["winf"] == ref["winf"], (what, got, ref)
    for key in ("w1", "w2"):
        assert abs(got[key] - ref[key]) <= 1e-12 * max(ref[key], 1e-300), (what, key, got, ref)
    return got


@pytest.mark.parametrize("n", [1, 2, 63, 257, 4096, 70001, 81920, (1 << 20) + 3])
@pytest.mark.parametrize("dts", [("bf16", "f64"), ("f32", "f64"), ("bf16", "bf16"),
                                 ("f32", "bf16"), ("f64", "f64")])
def test_matches_oracle(lib, n, dts):
    import precision_numerics_amd as pna
    rng = np.random.default_rng(n * 7 + len(dts[0]))
    for kind in ("normal", "ties", "wide", "zeros"):
        a = _as(_draw(rng, n, kind), dts[0])
        b = _as(_draw(rng, n, kind) * 1.5 + 0.25, dts[1])
        _print(f"wasserstein n={n} {dts} {kind}")
        _check(pna, a, b, f"n={n} {dts} {kind}")


def test_identities(lib):
    import precision_numerics_amd as pna
    rng = np.random.default_rng(3)
    x = rng.standard_normal(300_001)
    a = _as(x, "f64")
    perm = _as(x[rng.permutation(x.size)], "f64")
    w = pna.attn_wasserstein(a[0], perm[0])        # same distribution, another order
    assert w["w1"] == 0.0 and w["w2"] == 0.0 and w["winf"] == 0.0
    shift = _as(x + 0.5, "f64")                     # every quantile moves by 0.5
    w = pna.attn_wasserstein(a[0], shift[0])
    for key in ("w1", "w2", "winf"):
        assert abs(w[key] - 0.5) <= 1e-12
    w2 = pna.attn_wasserstein(shift[0], a[0])      # symmetric, and reproducible
    assert w2 == pna.attn_wasserstein(shift[0], a[0])
    assert w2["w1"] == w["w1"] and w2["winf"] == w["winf"]


def test_nonfinite(lib):
    import precision_numerics_amd as pna
    x = np.arange(1000, dtype=np.float64)
    y = x.copy()
    y[10], y[500] = np.nan, -np.inf
    for dt in ("f32", "bf16", "f64"):
        w = pna.attn_wasserstein(_as(x, dt)[0], _as(y, dt)[0])
        assert w["n_nonfinite"] == 2 and np.isnan(w["w1"]) and np.isnan(w["winf"])


def test_attention_outputs(lib):
    """Flash and baseline bf16 outputs of a workload against the FP64 oracle
    output, and against each other: the distances the GPU computes equal the
    oracle's on the same arrays."""
    import precision_numerics_amd as pna
    cfg = synth.small(synth.CONFIGS["c2"], batch=2, heads=4, seq_len=700)
    inp = synth.make_inputs(cfg, seed=31)
    q, k, v = device_inputs(inp)
    o_f = pna.attn_fwd_flash(q, k, v, causal=cfg.causal)
    o_b, _ = pna.attn_fwd_baseline(q, k, v, causal=cfg.causal)
    ref, _ = oracle.attention(*oracle_inputs(inp), causal=cfg.causal)
    ref_t = torch.from_numpy(np.ascontiguousarray(ref)).cuda()
    f64 = (o_f, o_f.double().cpu().numpy())
    b64 = (o_b, o_b.double().cpu().numpy())
    r64 = (ref_t, ref)
    wf = _check(pna, f64, r64, "flash vs fp64")
    wb = _check(pna, b64, r64, "baseline vs fp64")
    wfb = _check(pna, f64, b64, "flash vs baseline")
    _print(f"W1 flash-fp64 {wf['w1']:.3e}, baseline-fp64 {wb['w1']:.3e}, "
           f"flash-baseline {wfb['w1']:.3e}")
