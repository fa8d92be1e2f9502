"""FlashAttention backward on the GPU against the FP64 oracle.

The kernels take the stored bf16 O (delta = rowsum(dO o O) from it, as "Why
Low-Precision Transformer Training Fails" has the backward do, Figure 5
caption) and the forward's lse; the oracle gets the same O and recomputes P
exactly.  Error sources on the GPU side: P and dS rounded to bf16 for the
bf16 products (relative 2^-9 each), fp32 accumulation, and the bf16
rounding of dQ, dK, dV (relative 2^-9).  Tolerances per output tensor:
max|err| <= 1e-2 * max|ref| + atol and mean|err| <= 5e-3 * mean|ref| + atol,
where atol bounds the fp32 cancellation in dP - delta (two fp32 sums of d
products, computed by different kernels) carried through dQ = scale dS K or
dK = scale dS^T Q: atol = scale * max|K or Q| * 2 d 2^-23 max|dO| max|V|.
Where P is a single 1 (one visible key) the exact dQ is 0 and only that
cancellation remains.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from helpers import device_inputs, oracle_inputs, out_to_f64, torch_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

REL_MAX = 1e-2
REL_MEAN = 5e-3


def _print(*a):
    print(*a, flush=True)


def _grads(pna, q, k, v, causal, seed):
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
    o = pna.attn_fwd_flash(q, k, v, causal=causal, lse=lse)
    rng = np.random.default_rng(seed)
    g_bits = synth.f32_to_bf16_bits(rng.standard_normal(q.shape).astype(np.float32))
    d_o = torch_bf16(g_bits.reshape(q.shape))
    dq, dk, dv = pna.attn_bwd_flash(q, k, v, o, d_o, lse, causal=causal)
    torch.cuda.synchronize()
    return o, d_o, (dq, dk, dv)


def _atol(d, scale, other, g, v):
    return scale * np.abs(other).max() * 2 * d * 2.0 ** -23 * np.abs(g).max() * np.abs(v).max()


def _check(got, ref, what, atol):
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    assert np.all(np.isfinite(got)), what
    assert mx <= REL_MAX * np.abs(ref).max() + atol, (what, mx, np.abs(ref).max(), atol)
    assert mean <= REL_MEAN * np.abs(ref).mean() + atol, (what, mean, np.abs(ref).mean(), atol)
    return mx / max(np.abs(ref).max(), 1e-30), mean / max(np.abs(ref).mean(), 1e-30)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_tiny_shapes(lib, d, causal):
    import precision_numerics_amd as pna
    for n in (1, 3, 65, 200, 300):
        cfg = synth.small(synth.CONFIGS["c2"], batch=2, heads=2, seq_len=n, head_dim=d,
                          causal=causal)
        inp = synth.make_inputs(cfg, seed=900 + n)
        q, k, v = device_inputs(inp)
        o, d_o, grads = _grads(pna, q, k, v, causal, seed=n)
        qf, kf, vf = (x.reshape(4, n, d) for x in oracle_inputs(inp))
        of = out_to_f64(o).reshape(4, n, d)
        gf = out_to_f64(d_o).reshape(4, n, d)
        refs = [oracle.attention_backward_head(qf[u], kf[u], vf[u], of[u], gf[u], causal=causal,
                                               scale=oracle.default_scale(d)) for u in range(4)]
        sc = oracle.default_scale(d)
        atols = (_atol(d, sc, kf, gf, vf), _atol(d, sc, qf, gf, vf), 0.0)
        for i, name in enumerate(("dq", "dk", "dv")):
            ref = np.stack([r[i] for r in refs])
            rel = _check(out_to_f64(grads[i]).reshape(4, n, d), ref, f"{name} n={n}", atols[i])
            _print(f"backward d={d} causal={causal} n={n} {name}: rel max {rel[0]:.2e} "
                   f"rel mean {rel[1]:.2e}")


@pytest.mark.parametrize("causal", [False, True])
def test_backward_d128_many_blocks(lib, causal):
    """d = 128 over many key and query blocks with a ragged end (N = 1000):
    the kernels' masked first blocks, unmasked middle blocks and masked last
    block all run."""
    import precision_numerics_amd as pna
    n, d = 1000, 128
    cfg = synth.small(synth.CONFIGS["c3"], batch=1, heads=2, seq_len=n, head_dim=d,
                      causal=causal)
    inp = synth.make_inputs(cfg, seed=77)
    q, k, v = device_inputs(inp)
    o, d_o, grads = _grads(pna, q, k, v, causal, seed=7)
    qf, kf, vf = (x.reshape(2, n, d) for x in oracle_inputs(inp))
    of = out_to_f64(o).reshape(2, n, d)
    gf = out_to_f64(d_o).reshape(2, n, d)
    sc = oracle.default_scale(d)
    for u in range(2):
        ref = oracle.attention_backward_head(qf[u], kf[u], vf[u], of[u], gf[u], causal=causal,
                                             scale=sc)
        atols = (_atol(d, sc, kf[u], gf[u], vf[u]), _atol(d, sc, qf[u], gf[u], vf[u]), 0.0)
        for i, name in enumerate(("dq", "dk", "dv")):
            rel = _check(out_to_f64(grads[i]).reshape(2, n, d)[u], ref[i], f"{name} u={u}",
                         atols[i])
            _print(f"backward d=128 n=1000 causal={causal} unit {u} {name}: rel max {rel[0]:.2e} "
                   f"rel mean {rel[1]:.2e}")


@pytest.mark.parametrize("causal", [False, True])
def test_backward_head_groups(lib, causal):
    """Nine (batch, head) units: the kernels take heads in groups of eight
    (one per XCD) and the ninth on its own, so both branches of the
    workgroup-to-tile map run in one launch; every head is checked."""
    import precision_numerics_amd as pna
    n, d, units = 300, 64, 9
    cfg = synth.small(synth.CONFIGS["c2"], batch=3, heads=3, seq_len=n, head_dim=d,
                      causal=causal)
    inp = synth.make_inputs(cfg, seed=55)
    q, k, v = device_inputs(inp)
    o, d_o, grads = _grads(pna, q, k, v, causal, seed=5)
    qf, kf, vf = (x.reshape(units, n, d) for x in oracle_inputs(inp))
    of = out_to_f64(o).reshape(units, n, d)
    gf = out_to_f64(d_o).reshape(units, n, d)
    sc = oracle.default_scale(d)
    for u in range(units):
        ref = oracle.attention_backward_head(qf[u], kf[u], vf[u], of[u], gf[u], causal=causal,
                                             scale=sc)
        atols = (_atol(d, sc, kf[u], gf[u], vf[u]), _atol(d, sc, qf[u], gf[u], vf[u]), 0.0)
        for i, name in enumerate(("dq", "dk", "dv")):
            _check(out_to_f64(grads[i]).reshape(units, n, d)[u], ref[i], f"{name} u={u}", atols[i])
    _print(f"backward 9 heads causal={causal}: all units within tolerance")


def test_backward_workload_shape(lib):
    """The GPT-2-small workload's shape (B8 H12 N1024 d64, causal), sampled
    heads against the oracle, and bitwise reproducible run to run."""
    import precision_numerics_amd as pna
    cfg = synth.CONFIGS["c2"]
    inp = synth.make_inputs(cfg)
    q, k, v = device_inputs(inp)
    o, d_o, grads = _grads(pna, q, k, v, cfg.causal, seed=2)
    _, _, grads2 = _grads(pna, q, k, v, cfg.causal, seed=2)
    for a, b in zip(grads, grads2):
        assert torch.equal(a, b)
    b_, h, n, d = cfg.shape
    qf, kf, vf = (x.reshape(b_ * h, n, d) for x in oracle_inputs(inp))
    of = out_to_f64(o).reshape(b_ * h, n, d)
    gf = out_to_f64(d_o).reshape(b_ * h, n, d)
    for u in (0, 37, b_ * h - 1):
        ref = oracle.attention_backward_head(qf[u], kf[u], vf[u], of[u], gf[u], causal=True,
                                             scale=oracle.default_scale(d))
        sc = oracle.default_scale(d)
        atols = (_atol(d, sc, kf[u], gf[u], vf[u]), _atol(d, sc, qf[u], gf[u], vf[u]), 0.0)
        for i, name in enumerate(("dq", "dk", "dv")):
            rel = _check(out_to_f64(grads[i]).reshape(b_ * h, n, d)[u], ref[i], f"{name} u={u}",
                         atols[i])
            _print(f"backward c2 unit {u} {name}: rel max {rel[0]:.2e} rel mean {rel[1]:.2e}")


def test_backward_c3_shape_sampled(lib):
    """The backward at the shape and in the launch configuration the bench
    times (B4 H32 N4096 d128, causal): three sampled heads against the
    oracle, and bitwise reproducible run to run."""
    import precision_numerics_amd as pna
    cfg = synth.CONFIGS["c3"]
    inp = synth.make_inputs(cfg)
    q, k, v = device_inputs(inp)
    o, d_o, grads = _grads(pna, q, k, v, cfg.causal, seed=3)
    _, _, grads2 = _grads(pna, q, k, v, cfg.causal, seed=3)
    for a, b in zip(grads, grads2):
        assert torch.equal(a, b)
    b_, h, n, d = cfg.shape
    qf, kf, vf = (x.reshape(b_ * h, n, d) for x in oracle_inputs(inp))
    sc = oracle.default_scale(d)
    for u in (0, 77, b_ * h - 1):
        of = out_to_f64(o.reshape(b_ * h, n, d)[u])
        gf = out_to_f64(d_o.reshape(b_ * h, n, d)[u])
        ref = oracle.attention_backward_head(qf[u], kf[u], vf[u], of, gf, causal=True, scale=sc)
        atols = (_atol(d, sc, kf[u], gf, vf[u]), _atol(d, sc, qf[u], gf, vf[u]), 0.0)
        for i, name in enumerate(("dq", "dk", "dv")):
            rel = _check(out_to_f64(grads[i].reshape(b_ * h, n, d)[u]), ref[i], f"{name} u={u}",
                         atols[i])
            _print(f"backward c3 unit {u} {name}: rel max {rel[0]:.2e} rel mean {rel[1]:.2e}")
