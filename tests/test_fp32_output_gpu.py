"""O in fp32 for bf16, int8 and fp8 inputs (attn_problem_t.o_f32).

The kernels form O = acc / l in fp32 and round it to bf16 only at the
store, so the fp32 output is that value unrounded: rounding it to bf16 (RNE)
must give the default bf16 output bit for bit, for every kernel, variant and
mode.  Against the FP64 oracle the fp32 output is held to the bf16-class
tolerances (P is still rounded upstream) and must not be further from it on
average than the bf16 output, whose error includes the rounding of O.  This
is what the rounding-bias experiment needs to separate the rounding of O
from the rounding of P ("Why Low-Precision Transformer Training Fails",
Figures 5 and 7)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from helpers import assert_close, device_inputs, error_stats, oracle_inputs, out_to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _run(pna, kernel, q, k, v, causal, p_bf16, qs, ks, beta, out_f32):
    if kernel == "flash":
        return pna.attn_fwd_flash(q, k, v, causal=causal, p_bf16=p_bf16, q_scale=qs, k_scale=ks,
                                  beta=beta, out_f32=out_f32)
    return pna.attn_fwd_baseline(q, k, v, causal=causal, p_bf16=p_bf16, q_scale=qs, k_scale=ks,
                                 out_f32=out_f32)[0]


@pytest.mark.parametrize("kernel,variant", [("flash", "standard"), ("flash", "stabilized"),
                                            ("baseline", "standard")])
@pytest.mark.parametrize("dtype", ["bf16", "int8"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p_bf16", [True, False])
def test_fp32_output_is_the_unrounded_bf16_output(lib, kernel, variant, dtype, d, causal, p_bf16):
    import precision_numerics_amd as pna
    if variant == "stabilized" and dtype != "bf16":
        pytest.skip("the stabilised variant is built for bf16 inputs")
    beta = 2.0 if variant == "stabilized" else None
    for n in (17, 300):
        cfg = synth.small(synth.CONFIGS["c5" if dtype == "int8" else "c2"], batch=2, heads=3,
                          seq_len=n, head_dim=d, causal=causal)
        inp = synth.make_inputs(cfg, seed=900 + n + d)
        q, k, v = device_inputs(inp)
        qs = ks = None
        if dtype == "int8":
            q, qs = pna.attn_quantize_int8(q)
            k, ks = pna.attn_quantize_int8(k)
        print(f"fp32 O {kernel} {variant} {dtype} d={d} causal={causal} p_bf16={p_bf16} n={n}",
              flush=True)
        o16 = _run(pna, kernel, q, k, v, causal, p_bf16, qs, ks, beta, False)
        o32 = _run(pna, kernel, q, k, v, causal, p_bf16, qs, ks, beta, True)
        torch.cuda.synchronize()
        assert o32.dtype == torch.float32 and o16.dtype == torch.bfloat16
        assert torch.equal(o32.to(torch.bfloat16).view(torch.int16), o16.view(torch.int16))
        if dtype == "int8":
            qc, qsc = oracle.quantize_int8(inp.q)
            kc, ksc = oracle.quantize_int8(inp.k)
            ref, _ = oracle.attention_int8(qc, qsc, kc, ksc,
                                           synth.bf16_bits_to_f32(inp.v).astype(np.float64),
                                           causal=causal)
        else:
            ref, _ = oracle.attention(*oracle_inputs(inp), causal=causal)
        st32 = assert_close(out_to_f64(o32), ref, "bf16", "fp32 output")
        st16 = error_stats(out_to_f64(o16), ref)
        assert st32["mean_abs"] <= st16["mean_abs"]


def test_fp32_output_full_workload_sample(lib):
    """Llama-shaped causal workload (the bench's): fp32 O of sampled heads
    against the oracle, and its bf16 rounding equals the bf16 output."""
    import precision_numerics_amd as pna
    cfg = synth.CONFIGS["c3"]
    inp = synth.make_inputs(cfg)
    q, k, v = device_inputs(inp)
    o16 = pna.attn_fwd_flash(q, k, v, causal=True)
    o32 = pna.attn_fwd_flash(q, k, v, causal=True, out_f32=True)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16).view(torch.int16), o16.view(torch.int16))
    b, h, n, dd = cfg.shape
    units = [0, 77, b * h - 1]
    qq, kk, vv = (x.reshape(b * h, n, dd) for x in oracle_inputs(inp))
    ref = np.stack([oracle.attention_head(qq[u], kk[u], vv[u], causal=True,
                                          scale=oracle.default_scale(dd))[0] for u in units])
    got = out_to_f64(o32.view(b * h, n, dd)[units])
    st = assert_close(got, ref, "bf16", "c3 fp32 output")
    st16 = error_stats(out_to_f64(o16.view(b * h, n, dd)[units]), ref)
    print(f"c3 fp32 O: {st}; bf16 O: {st16}", flush=True)
    assert st["mean_abs"] < st16["mean_abs"]
