"""delta = rowsum(dO o O) on the GPU against the FP64 oracle.

The bound: each row is summed in fp32 with one fused multiply-add per element
and a fixed butterfly over at most 32 partial sums, so
|delta - delta_ref| <= (d + 5) * 2^-24 * sum_c |dO_c O_c| (bf16 products are
exact in fp32, fp32 products contribute one more rounding each).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from helpers import torch_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _print(*a):
    print(*a, flush=True)


def _pair(shape, dtype, seed):
    rng = np.random.default_rng(seed)
    o = rng.standard_normal(shape, dtype=np.float32)
    g = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.01)
    if dtype == "bf16":
        ob, gb = synth.f32_to_bf16_bits(o), synth.f32_to_bf16_bits(g)
        return (torch_bf16(ob), torch_bf16(gb), synth.bf16_bits_to_f32(ob),
                synth.bf16_bits_to_f32(gb))
    return torch.from_numpy(o).cuda(), torch.from_numpy(g).cuda(), o, g


def _check(delta, o, g, rows=None):
    o64 = o.astype(np.float64).reshape(-1, o.shape[-1])
    g64 = g.astype(np.float64).reshape(-1, o.shape[-1])
    got = delta.cpu().numpy().astype(np.float64).reshape(-1)
    if rows is not None:
        o64, g64, got = o64[rows], g64[rows], got[rows]
    ref = oracle.attention_delta(o64, g64)
    bound = (o.shape[-1] + 5) * 2.0 ** -24 * np.abs(o64 * g64).sum(-1) + 1e-30
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"worst {float((err / bound).max()):.3f} of the bound"
    return float(err.max())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_delta_matches_oracle(lib, dtype, d):
    import precision_numerics_amd as pna
    for n in (1, 3, 17, 257, 1000):
        to, tg, o, g = _pair((2, 3, n, d), dtype, 10 + n)
        delta = pna.attn_bwd_delta(to, tg)
        torch.cuda.synchronize()
        err = _check(delta, o, g)
        _print(f"delta {dtype} d={d} n={n}: max err {err:.3e}")


def test_delta_of_flash_output(lib):
    """delta from the forward kernel's own bf16 output, as the backward pass
    would form it."""
    import precision_numerics_amd as pna
    cfg = synth.small(synth.CONFIGS["c2"], batch=2, heads=4, seq_len=300)
    inp = synth.make_inputs(cfg)
    q, k, v = (torch_bf16(x) for x in (inp.q, inp.k, inp.v))
    o = pna.attn_fwd_flash(q, k, v, causal=True)
    rng = np.random.default_rng(3)
    gb = synth.f32_to_bf16_bits(rng.standard_normal(o.shape, dtype=np.float32))
    g = torch_bf16(gb)
    delta = pna.attn_bwd_delta(o, g)
    torch.cuda.synchronize()
    _check(delta, o.float().cpu().numpy(), synth.bf16_bits_to_f32(gb))


def test_delta_full_size_and_deterministic(lib):
    """The bench workload's shape (B4 H32 N4096 d128): more rows than one
    grid pass covers, checked on sampled rows; two calls agree bitwise."""
    import precision_numerics_amd as pna
    to, tg, o, g = _pair((4, 32, 4096, 128), "bf16", 99)
    d1 = pna.attn_bwd_delta(to, tg)
    d2 = pna.attn_bwd_delta(to, tg)
    torch.cuda.synchronize()
    assert torch.equal(d1, d2)
    rows = np.random.default_rng(5).choice(4 * 32 * 4096, size=4096, replace=False)
    rows = np.concatenate([rows, [0, 4 * 32 * 4096 - 1]])
    _check(d1, o, g, rows)


def test_delta_closed_forms(lib):
    import precision_numerics_amd as pna
    to, _, o, _ = _pair((1, 2, 33, 64), "bf16", 4)
    sq = pna.attn_bwd_delta(to, to)                     # dO = O: squared row norms
    zero = pna.attn_bwd_delta(to, torch.zeros_like(to))
    torch.cuda.synchronize()
    _check(sq, o, o)
    assert torch.count_nonzero(zero).item() == 0
