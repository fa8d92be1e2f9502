"""The int32 products Qc Kc^T of the int8 flash kernel are exact at full size.

"INT-FlashAttention" (abstract) runs Q and K through the FlashAttention
forward as int8; the products of int8 codes are integers that an int32
accumulator holds exactly (|sum| <= 128 * 127^2 < 2^31).  The flash kernel
never stores its score tiles, so attn_fwd_flash_debug_s, a debug instance of
the same kernel template, writes every int32 tile it forms into s_out.  Here
it runs at the int8 workload's full shape (batch 4, 32 heads, seq 2048,
d 128: 1024 query tiles on the persistent schedule, four heads per XCD at a
time) and on a ragged causal shape with more tiles than compute units, and

* the dumped products of sampled heads equal the oracle's integer dot
  products bit for bit, and
* the debug instance's output O is bitwise the production instance's, so
  both form the same scores.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from helpers import device_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SENTINEL = np.iinfo(np.int32).min


def _run(pna, cfg, inp):
    q, k, v = device_inputs(inp)
    qc, qs = pna.attn_quantize_int8(q)
    kc, ks = pna.attn_quantize_int8(k)
    b, h, n, _ = cfg.shape
    s_out = torch.full((b, h, n, n), SENTINEL, dtype=torch.int32, device="cuda")
    o_dbg, _ = pna.attn_fwd_flash_debug_s(qc, kc, v, causal=cfg.causal, q_scale=qs, k_scale=ks,
                                          s_out=s_out)
    o_prod = pna.attn_fwd_flash(qc, kc, v, causal=cfg.causal, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    return s_out, o_dbg, o_prod


def _check_units(cfg, inp, s_out, units):
    b, h, n, d = cfg.shape
    qc, _ = oracle.quantize_int8(inp.q)
    kc, _ = oracle.quantize_int8(inp.k)
    qc, kc = qc.reshape(b * h, n, d), kc.reshape(b * h, n, d)
    s_all = s_out.view(b * h, n, n)
    visible = np.tril(np.ones((n, n), bool)) if cfg.causal else np.ones((n, n), bool)
    for u in units:
        got = s_all[u].cpu().numpy().astype(np.int64)
        want = oracle.int8_scores(qc[u], kc[u])
        written = got != SENTINEL
        assert written[visible].all(), f"unit {u}: visible products not written"
        assert np.array_equal(got[written], want[written]), f"unit {u}"
        print(f"unit {u}: {int(written.sum())} products bit-exact", flush=True)


def test_int8_scores_bit_exact_full_workload(lib):
    import precision_numerics_amd as pna
    cfg = synth.CONFIGS["c5"]
    print(f"int8 debug dump at {cfg.shape}, causal={cfg.causal}", flush=True)
    inp = synth.make_inputs(cfg)
    s_out, o_dbg, o_prod = _run(pna, cfg, inp)
    assert torch.equal(o_dbg, o_prod)
    b, h = cfg.batch, cfg.heads
    rng = np.random.default_rng(cfg.seed)
    units = sorted({0, 5, b * h - 1, *rng.choice(b * h, 3, replace=False).tolist()})
    _check_units(cfg, inp, s_out, units)


def test_int8_scores_bit_exact_persistent_causal(lib):
    """64 heads of 1100 queries: 320 query tiles of 256 rows (the last one
    ragged) on the persistent schedule, causal; every head is checked."""
    import precision_numerics_amd as pna
    cfg = synth.small(synth.CONFIGS["c5"], batch=2, heads=32, seq_len=1100, causal=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert cfg.batch * cfg.heads * -(-cfg.seq_len // 256) > cus
    inp = synth.make_inputs(cfg, seed=4242)
    s_out, o_dbg, o_prod = _run(pna, cfg, inp)
    assert torch.equal(o_dbg, o_prod)
    _check_units(cfg, inp, s_out, range(cfg.batch * cfg.heads))
