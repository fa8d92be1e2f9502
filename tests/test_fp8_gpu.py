"""E4M3 fp8 Q/K attention on the GPU against the FP64 oracle.

Q and K are quantised per row to E4M3 codes ("FP8 Formats for Deep
Learning", in the reference list of "Why Low-Precision Transformer Training
Fails"; the per-row absmax/448 scale is this library's reading, as for the
INT8 path of "INT-FlashAttention"); the scores are scale * sq_i * sk_j times
the dot products of the decoded codes.

* The quantiser is bit-exact: codes and scales equal the oracle's.
* The fp8 matrix cores sum each 16-term product with less than fp32
  precision; the baseline's stored products (unscaled) are checked against
  the exact dot products within 2^-12 of the sum of the terms' magnitudes.
* Outputs meet the bf16 tolerances of the other paths against the oracle's
  exact fp8 attention, for both kernels, head_dim 64 and 128, causal or not,
  P in bf16 or fp32, on ragged shapes and on the full int8 workload shape.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from helpers import assert_close, out_to_f64, torch_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _print(*a):
    print(*a, flush=True)


def _inputs(b, h, n, d, seed):
    """fp32 Q, K draws and bf16 V of the int8 workload's recipe."""
    cfg = synth.small(synth.CONFIGS["c5"], batch=b, heads=h, seq_len=n, head_dim=d)
    return cfg, synth.make_inputs(cfg, seed=seed)


def _quantised(pna, inp):
    q = torch.from_numpy(inp.q).cuda()
    k = torch.from_numpy(inp.k).cuda()
    qc, qs = pna.attn_quantize_fp8(q)
    kc, ks = pna.attn_quantize_fp8(k)
    return qc, qs, kc, ks


def _oracle(inp, causal, units=None):
    b, h, n, d = inp.q.shape
    qc, qs = oracle.quantize_fp8(inp.q)
    kc, ks = oracle.quantize_fp8(inp.k)
    v = synth.bf16_bits_to_f32(inp.v).astype(np.float64).reshape(b * h, n, d)
    qc, kc = qc.reshape(b * h, n, d), kc.reshape(b * h, n, d)
    qs, ks = qs.reshape(b * h, n), ks.reshape(b * h, n)
    units = range(b * h) if units is None else units
    res = [oracle.attention_fp8_head(qc[u], qs[u], kc[u], ks[u], v[u], causal=causal,
                                     scale=oracle.default_scale(d)) for u in units]
    return np.stack([r[0] for r in res]), np.stack([r[1] for r in res])


@pytest.mark.parametrize("rows,d", [(1, 1), (7, 64), (333, 128), (5, 1000), (64, 3)])
def test_fp8_quantiser_bit_exact(lib, rows, d):
    import precision_numerics_amd as pna
    rng = np.random.default_rng(rows * 131 + d)
    x = (rng.standard_normal((rows, d)) * np.exp(rng.standard_normal((rows, 1)) * 4)
         ).astype(np.float32)
    if rows > 3:
        x[1] = 0.0
        x[2, : d // 2] = -0.0
        x[3] = rng.standard_normal(d).astype(np.float32) * np.float32(1e-30)
    codes, scales = pna.attn_quantize_fp8(torch.from_numpy(x).cuda())
    oc, osc = oracle.quantize_fp8(x)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(scales.cpu().numpy(), osc)


@pytest.mark.parametrize("kernel", ["flash", "baseline"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p_bf16", [True, False])
def test_fp8_attention_tiny_shapes(lib, kernel, d, causal, p_bf16):
    import precision_numerics_amd as pna
    for n in (1, 3, 65, 200, 300):
        cfg, inp = _inputs(2, 2, n, d, seed=700 + n)
        qc, qs, kc, ks = _quantised(pna, inp)
        v = torch_bf16(inp.v)
        _print(f"fp8 {kernel} d={d} causal={causal} p_bf16={p_bf16} n={n}")
        if kernel == "flash":
            lse = torch.empty(qc.shape[:-1], dtype=torch.float32, device="cuda")
            o = pna.attn_fwd_flash(qc, kc, v, causal=causal, p_bf16=p_bf16, q_scale=qs,
                                   k_scale=ks, lse=lse)
        else:
            o, ws = pna.attn_fwd_baseline(qc, kc, v, causal=causal, p_bf16=p_bf16, q_scale=qs,
                                          k_scale=ks)
        torch.cuda.synchronize()
        ref, lse_ref = _oracle(inp, causal)
        assert_close(out_to_f64(o).reshape(ref.shape), ref, "bf16", f"fp8 n={n}")
        if kernel == "flash":
            err = np.abs(lse.cpu().numpy().astype(np.float64).reshape(lse_ref.shape) - lse_ref)
            assert err.max() <= 1e-3 * max(1.0, np.abs(lse_ref).max()), err.max()
        else:
            # the stored products against the exact dot products of the codes
            b, h = 2, 2
            s = ws[: 4 * b * h * n * n].view(torch.float32).view(b * h, n, n).cpu().numpy()
            oqc, _ = oracle.quantize_fp8(inp.q)
            okc, _ = oracle.quantize_fp8(inp.k)
            qd = oracle.e4m3_decode(oqc.reshape(b * h, n, d))
            kd = oracle.e4m3_decode(okc.reshape(b * h, n, d))
            exact = qd @ np.swapaxes(kd, -1, -2)
            mag = np.abs(qd) @ np.swapaxes(np.abs(kd), -1, -2)
            dev = np.abs(s.astype(np.float64) - exact)
            assert np.all(dev <= mag * 2.0 ** -12), (dev / np.maximum(mag, 1e-300)).max()


def test_fp8_full_int8_workload_shape(lib):
    """The int8 workload's shape (B4 H32 N2048 d128, non-causal) with E4M3
    codes, flash kernel in the benchmark's launch configuration, sampled
    heads against the oracle."""
    import precision_numerics_amd as pna
    cfg = synth.CONFIGS["c5"]
    inp = synth.make_inputs(cfg)
    qc, qs, kc, ks = _quantised(pna, inp)
    v = torch_bf16(inp.v)
    o = pna.attn_fwd_flash(qc, kc, v, causal=cfg.causal, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    b, h, n, d = cfg.shape
    units = [0, 37, b * h - 1]
    ref, _ = _oracle(inp, cfg.causal, units)
    st = assert_close(out_to_f64(o).reshape(b * h, n, d)[units], ref, "bf16", "fp8 c5 shape")
    _print(f"fp8 full shape: {st}")
