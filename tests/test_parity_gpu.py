"""Parity of the HIP path (through the C ABI) with the FP64 oracle.

Tiny and ragged shapes are compared element by element; the five workloads
run at full size in the launch configuration the benchmark times, compared
in full where the oracle is quick (c1, c2) and on sampled heads otherwise.
Integer work is bit-exact: the int8 codes and scales, and the int32 score
products Qc Kc^T of both kernels.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from helpers import (assert_close, device_inputs, error_stats, oracle_inputs, out_to_f64,
                     torch_bf16)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu(lib):
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    yield


def _print(*a):
    print(*a, flush=True)


def gpu_forward(pna, cfg, inp, kernel="flash", p_bf16=None, lse=False):
    """Run the HIP path on the workload; returns (O float64 host, extras)."""
    p_bf16 = cfg.p_bf16 if p_bf16 is None else p_bf16
    q, k, v = device_inputs(inp)
    extras = {}
    qs = ks = None
    if cfg.dtype == "int8":
        q, qs = pna.attn_quantize_int8(q)
        k, ks = pna.attn_quantize_int8(k)
        extras["codes"] = (q, qs, k, ks)
    if kernel == "flash":
        lse_t = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda") if lse else None
        o = pna.attn_fwd_flash(q, k, v, causal=cfg.causal, p_bf16=p_bf16, q_scale=qs,
                               k_scale=ks, lse=lse_t)
        extras["lse"] = lse_t
    else:
        o, ws = pna.attn_fwd_baseline(q, k, v, causal=cfg.causal, p_bf16=p_bf16, q_scale=qs,
                                      k_scale=ks)
        extras["workspace"] = ws
    torch.cuda.synchronize()
    extras["o_dev"] = o
    return out_to_f64(o), extras


def oracle_forward(cfg, inp, units=None):
    """Oracle O (and lse) for all (b, h) units, or for the listed ones."""
    b, h, n, d = cfg.shape
    units = list(range(b * h)) if units is None else list(units)
    if cfg.dtype == "int8":
        qc, qs = oracle.quantize_int8(inp.q)
        kc, ks = oracle.quantize_int8(inp.k)
        v = synth.bf16_bits_to_f32(inp.v).astype(np.float64)
        qc, kc = qc.reshape(b * h, n, d), kc.reshape(b * h, n, d)
        qs, ks, v = qs.reshape(b * h, n), ks.reshape(b * h, n), v.reshape(b * h, n, d)
        res = [oracle.attention_int8_head(qc[u], qs[u], kc[u], ks[u], v[u], causal=cfg.causal,
                                          scale=oracle.default_scale(d)) for u in units]
    else:
        q, k, v = (x.reshape(b * h, n, d) for x in oracle_inputs(inp))
        res = [oracle.attention_head(q[u], k[u], v[u], causal=cfg.causal,
                                     scale=oracle.default_scale(d)) for u in units]
    return np.stack([r[0] for r in res]), np.stack([r[1] for r in res]), units


# ---------------------------------------------------------------------------
# tiny and ragged shapes, every kernel and mode, compared in full
# ---------------------------------------------------------------------------

TINY_N = [1, 2, 3, 17, 64, 65, 200, 257]


@pytest.mark.parametrize("kernel", ["flash", "baseline"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "int8"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p_bf16", [True, False])
def test_tiny_shapes(lib, kernel, dtype, d, causal, p_bf16):
    import precision_numerics_amd as pna
    base = {"f32": "c1", "bf16": "c2", "int8": "c5"}[dtype]
    for n in TINY_N:
        cfg = synth.small(synth.CONFIGS[base], batch=2, heads=3, seq_len=n, head_dim=d,
                          causal=causal)
        inp = synth.make_inputs(cfg, seed=1000 + n)
        _print(f"tiny {kernel} {dtype} d={d} causal={causal} p_bf16={p_bf16} n={n}")
        o, ex = gpu_forward(pna, cfg, inp, kernel, p_bf16=p_bf16, lse=(kernel == "flash"))
        ref, lse_ref, _ = oracle_forward(cfg, inp)
        # fp32 I/O is held to the fp32 bound only when P stays fp32; rounding
        # P to bf16 puts it in the bf16 class
        cls = "f32" if (dtype == "f32" and not p_bf16) else "bf16"
        assert_close(o, ref.reshape(o.shape), cls, f"{kernel} {dtype} d={d} causal={causal} n={n}")
        if kernel == "flash":
            lse = ex["lse"].cpu().numpy().astype(np.float64).reshape(lse_ref.shape)
            assert np.abs(lse - lse_ref).max() <= 1e-4 * max(1.0, np.abs(lse_ref).max())


# ---------------------------------------------------------------------------
# int8: the quantiser and the int32 score products are bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows,d", [(1, 1), (7, 64), (333, 128), (5, 1000), (64, 3)])
def test_quantiser_bit_exact(lib, rows, d):
    import precision_numerics_amd as pna
    rng = np.random.default_rng(rows * 1000 + d)
    x = rng.standard_normal((rows, d)).astype(np.float32) * rng.uniform(0.01, 50, (rows, 1)).astype(np.float32)
    x[0, :] = 0.0                              # absmax = 0 row
    if d >= 8:
        x[-1, :8] = np.array([127, 0.5, 1.5, 2.5, -2.5, -0.5, 3.5, -126.5], np.float32)
        x[-1, 8:] = 0.25
    codes, scales = pna.attn_quantize_int8(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_int8(x)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [17, 65, 200])
def test_int8_scores_bit_exact(lib, d, causal, n):
    import precision_numerics_amd as pna
    cfg = synth.small(synth.CONFIGS["c5"], batch=2, heads=2, seq_len=n, head_dim=d, causal=causal)
    inp = synth.make_inputs(cfg, seed=77 + n)
    q, k, v = device_inputs(inp)
    qc, qs = pna.attn_quantize_int8(q)
    kc, ks = pna.attn_quantize_int8(k)
    sentinel = np.iinfo(np.int32).min
    s_out = torch.full((2, 2, n, n), sentinel, dtype=torch.int32, device="cuda")
    pna.attn_fwd_flash_debug_s(qc, kc, v, causal=causal, q_scale=qs, k_scale=ks, s_out=s_out)
    _, ws = pna.attn_fwd_baseline(qc, kc, v, causal=causal, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    ocq, _ = oracle.quantize_int8(inp.q)
    ock, _ = oracle.quantize_int8(inp.k)
    dots = oracle.int8_scores(ocq, ock)                        # [2,2,n,n] int64
    flash_s = s_out.cpu().numpy().astype(np.int64)
    written = flash_s != sentinel
    visible = np.tril(np.ones((n, n), bool)) if causal else np.ones((n, n), bool)
    assert written[..., visible].all()
    assert np.array_equal(flash_s[written], dots[written])
    base_s = ws[: 4 * 4 * n * n].view(torch.int32).cpu().numpy().reshape(2, 2, n, n)
    assert np.array_equal(base_s.astype(np.int64), dots)


# ---------------------------------------------------------------------------
# invariants on the GPU outputs
# ---------------------------------------------------------------------------

def _bf16_tensor(x):
    return torch_bf16(synth.f32_to_bf16_bits(np.ascontiguousarray(x, np.float32)))


@pytest.mark.parametrize("kernel", ["flash", "baseline"])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_values(lib, kernel, causal):
    import precision_numerics_amd as pna
    rng = np.random.default_rng(5)
    b, h, n, d = 1, 2, 300, 128
    k = rng.standard_normal((b, h, n, d)).astype(np.float32)
    v = rng.standard_normal((b, h, n, d)).astype(np.float32)
    qt, kt, vt = _bf16_tensor(np.zeros_like(k)), _bf16_tensor(k), _bf16_tensor(v)
    if kernel == "flash":
        o = pna.attn_fwd_flash(qt, kt, vt, causal=causal)
    else:
        o, _ = pna.attn_fwd_baseline(qt, kt, vt, causal=causal)
    torch.cuda.synchronize()
    o = out_to_f64(o)
    vv = out_to_f64(vt)
    if causal:
        ref = np.cumsum(vv, axis=2) / np.arange(1, n + 1)[None, None, :, None]
        assert np.array_equal(o[:, :, 0], vv[:, :, 0])         # row 0 is V_0 exactly
    else:
        ref = np.broadcast_to(vv.mean(axis=2, keepdims=True), vv.shape)
    st = error_stats(o, ref)
    assert st["max_abs"] <= 2e-2 and st["mean_abs"] <= 2e-3, st


@pytest.mark.parametrize("kernel", ["flash", "baseline"])
def test_key_value_permutation_invariance(lib, kernel):
    import precision_numerics_amd as pna
    cfg = synth.CONFIGS["c5"].scaled(batch=1, heads=2, seq_len=500, dtype="bf16", causal=False)
    inp = synth.make_inputs(cfg, seed=9)
    perm = np.random.default_rng(1).permutation(cfg.seq_len)
    inp2 = synth.Inputs(cfg, inp.q, np.ascontiguousarray(inp.k[:, :, perm]),
                        np.ascontiguousarray(inp.v[:, :, perm]))
    o1, _ = gpu_forward(pna, cfg, inp, kernel)
    o2, _ = gpu_forward(pna, cfg, inp2, kernel)
    st = error_stats(o1, o2)
    assert st["max_abs"] <= 2e-2 and st["mean_abs"] <= 2e-3, st


def test_single_key_returns_value_exactly(lib):
    import precision_numerics_amd as pna
    for dtype in ("bf16", "f32"):
        cfg = synth.small(synth.CONFIGS["c2" if dtype == "bf16" else "c1"], batch=3, heads=2,
                          seq_len=1, head_dim=128)
        inp = synth.make_inputs(cfg)
        o, _ = gpu_forward(pna, cfg, inp)
        assert np.array_equal(o, oracle_inputs(inp)[2])


@pytest.mark.parametrize("name", ["c2", "c5"])
def test_flash_is_deterministic(lib, name):
    import precision_numerics_amd as pna
    cfg = synth.small(synth.CONFIGS[name], batch=1, heads=4, seq_len=777)
    inp = synth.make_inputs(cfg)
    a, exa = gpu_forward(pna, cfg, inp)
    b, exb = gpu_forward(pna, cfg, inp)
    assert torch.equal(exa["o_dev"], exb["o_dev"])


# ---------------------------------------------------------------------------
# the deviation reduction
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 1000, 1 << 20, 3_000_001])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_deviation_matches_oracle(lib, n, dtype):
    import precision_numerics_amd as pna
    rng = np.random.default_rng(n)
    ref = rng.standard_normal(n)
    test32 = (ref + rng.standard_normal(n) * 1e-3).astype(np.float32)
    if n > 10:
        test32[n // 3] = np.nan
        test32[n // 2] = np.inf
        test32[7] = np.float32(ref[7] + 0.5)
        test32[n - 1] = np.float32(ref[n - 1] - 0.5)
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(test32)
        t = torch_bf16(bits)
        test = synth.bf16_bits_to_f32(bits).astype(np.float64)
    else:
        t = torch.from_numpy(test32).cuda()
        test = test32.astype(np.float64)
    got = pna.attn_deviation(t, torch.from_numpy(ref).cuda())
    want = oracle.deviation(test, ref)
    assert got["n"] == want["n"] and got["n_nonfinite"] == want["n_nonfinite"]
    assert got["argmax"] == want["argmax"]
    assert got["max_abs"] == want["max_abs"] and got["max_ref_abs"] == want["max_ref_abs"]
    for key in ("mean_abs", "mean_signed", "rms", "rel_normwise"):
        assert abs(got[key] - want[key]) <= 1e-12 * max(1e-300, abs(want[key])) + 1e-300, key
    again = pna.attn_deviation(t, torch.from_numpy(ref).cuda())
    assert again == got                                   # bitwise reproducible



@pytest.mark.parametrize("n", [1, 4095, 70001])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_deviation_unaligned_views(lib, n, dtype):
    """Operands one element past a 16-byte boundary take the element-wise
    first pass: same oracle agreement, and the same result as aligned copies
    of the same values."""
    import precision_numerics_amd as pna
    rng = np.random.default_rng(100 + n)
    ref = rng.standard_normal(n + 1)
    test32 = (ref + rng.standard_normal(n + 1) * 1e-3).astype(np.float32)
    if n >= 3:
        test32[1 + n // 2] = np.nan
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(test32)
        t_all = torch_bf16(bits)
        test = synth.bf16_bits_to_f32(bits).astype(np.float64)[1:]
    else:
        t_all = torch.from_numpy(test32).cuda()
        test = test32.astype(np.float64)[1:]
    r_all = torch.from_numpy(ref).cuda()
    t_view, r_view = t_all[1:], r_all[1:]          # 2 or 4 and 8 bytes past the allocation start
    assert t_view.data_ptr() % 16 != 0 and r_view.data_ptr() % 16 != 0
    got = pna.attn_deviation(t_view, r_view)
    want = oracle.deviation(test, ref[1:])
    assert got["n"] == want["n"] and got["n_nonfinite"] == want["n_nonfinite"]
    assert got["argmax"] == want["argmax"] and got["max_abs"] == want["max_abs"]
    for key in ("mean_abs", "mean_signed", "rms", "rel_normwise"):
        assert abs(got[key] - want[key]) <= 1e-12 * max(1e-300, abs(want[key])) + 1e-300, key
    aligned = pna.attn_deviation(t_view.clone(), r_view.clone())
    assert aligned["argmax"] == got["argmax"] and aligned["max_abs"] == got["max_abs"]
    assert aligned["n_nonfinite"] == got["n_nonfinite"]

# ---------------------------------------------------------------------------
# the five workloads at full size (bench launch configuration)
# ---------------------------------------------------------------------------

def _sample_units(cfg, count):
    b, h = cfg.batch, cfg.heads
    rng = np.random.default_rng(cfg.seed)
    units = sorted(set([0, b * h - 1] + list(rng.choice(b * h, size=min(count, b * h),
                                                        replace=False))))
    return units[:count + 2]


@pytest.mark.parametrize("name,kernel,p_bf16,count", [
    ("c1", "flash", False, None), ("c1", "baseline", False, None),
    ("c2", "flash", True, None), ("c2", "baseline", True, None),
    ("c3", "flash", True, 3), ("c3", "baseline", True, 2),
    ("c4", "flash", True, 1), ("c4", "flash", False, 1),
    ("c5", "flash", True, 3), ("c5", "baseline", True, 2),
])
def test_full_workloads(lib, name, kernel, p_bf16, count):
    import precision_numerics_amd as pna
    cfg = synth.CONFIGS[name]
    _print(f"workload {name} {kernel} p_bf16={p_bf16}: generating inputs")
    inp = synth.make_inputs(cfg)
    o, ex = gpu_forward(pna, cfg, inp, kernel, p_bf16=p_bf16)
    b, h, n, d = cfg.shape
    o = o.reshape(b * h, n, d)
    units = None if count is None else _sample_units(cfg, count)
    _print(f"workload {name} {kernel}: oracle on units {units if units else 'all'}")
    ref, _, units = oracle_forward(cfg, inp, units)
    st = assert_close(o[units], ref, "f32" if cfg.dtype == "f32" else "bf16", f"{name} {kernel}")
    _print(f"workload {name} {kernel} p_bf16={p_bf16}: {st}")
    if cfg.dtype == "int8":
        qc, qs, kc, ks = ex["codes"]
        oq, osc = oracle.quantize_int8(inp.q)
        assert np.array_equal(qc.cpu().numpy(), oq) and np.array_equal(qs.cpu().numpy(), osc)
        if kernel == "baseline":
            okc, _ = oracle.quantize_int8(inp.k)
            s_all = ex["workspace"][: 4 * b * h * n * n].view(torch.int32).view(b * h, n, n)
            for u in units:
                dots = oracle.int8_scores(oq.reshape(b * h, n, d)[u], okc.reshape(b * h, n, d)[u])
                assert np.array_equal(s_all[u].cpu().numpy().astype(np.int64), dots)


@pytest.mark.parametrize("tile_rows", [1, 7, 64, 256, 10 ** 6])
def test_int8_tile_quantiser_and_attention(lib, tile_rows):
    """Per-tile int8 scales: codes and per-row scales bit-exact with the
    oracle's tile quantiser; flash and baseline on them match the oracle's
    int8 attention (ragged n, both causal modes)."""
    import precision_numerics_amd as pna
    cfg = synth.small(synth.CONFIGS["c5"], batch=2, heads=3, seq_len=333, head_dim=64)
    inp = synth.make_inputs(cfg, seed=88 + tile_rows % 97)
    q32 = torch.from_numpy(inp.q).cuda()
    k32 = torch.from_numpy(inp.k).cuda()
    qc, qs = pna.attn_quantize_int8_tiles(q32, tile_rows)
    kc, ks = pna.attn_quantize_int8_tiles(k32, tile_rows)
    oqc, oqs = oracle.quantize_int8_tiles(inp.q, tile_rows)
    okc, oks = oracle.quantize_int8_tiles(inp.k, tile_rows)
    assert np.array_equal(qc.cpu().numpy(), oqc) and np.array_equal(qs.cpu().numpy(), oqs)
    assert np.array_equal(kc.cpu().numpy(), okc) and np.array_equal(ks.cpu().numpy(), oks)
    v = torch_bf16(inp.v)
    vf = synth.bf16_bits_to_f32(inp.v).astype(np.float64)
    for causal in (False, True):
        ref, _ = oracle.attention_int8(oqc, oqs, okc, oks, vf, causal=causal)
        o = pna.attn_fwd_flash(qc, kc, v, causal=causal, q_scale=qs, k_scale=ks)
        ob, _ = pna.attn_fwd_baseline(qc, kc, v, causal=causal, q_scale=qs, k_scale=ks)
        torch.cuda.synchronize()
        _print(f"int8 tiles={tile_rows} causal={causal}")
        assert_close(out_to_f64(o), ref, "bf16", f"flash tiles={tile_rows}")
        assert_close(out_to_f64(ob), ref, "bf16", f"baseline tiles={tile_rows}")
