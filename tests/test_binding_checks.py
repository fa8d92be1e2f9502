"""The Python binding rejects tensors whose shape, dtype or device differs
from what the problem (built from q) implies, before it calls the C ABI:
the ABI sees only pointers, so such a tensor would make a kernel read or
write past its allocation.  CPU only: every case raises before any launch."""
import pytest

torch = pytest.importorskip("torch")

import precision_numerics_amd as pna  # noqa: E402

B, H, N, D = 2, 3, 17, 64
bf16, f32 = torch.bfloat16, torch.float32


def t(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def qkv(dtype=bf16):
    vt = f32 if dtype == f32 else bf16
    return t((B, H, N, D), dtype), t((B, H, N, D), dtype), t((B, H, N, D), vt)


def test_well_formed_cpu_tensors_reach_the_device_check():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="CUDA"):
        pna.attn_fwd_flash(q, k, v, causal=True)


@pytest.mark.parametrize("case", [
    "k_shape", "k_dtype", "v_dtype", "v_shape", "out_dtype", "out_shape", "lse_shape",
    "lse_dtype", "q_3d", "scale_for_bf16",
])
def test_flash_rejects(case):
    q, k, v = qkv()
    kw = {}
    err = ValueError
    if case == "k_shape":
        k = t((B, H, N + 1, D), bf16)
    elif case == "k_dtype":
        k, err = t((B, H, N, D), f32), TypeError
    elif case == "v_dtype":
        v, err = t((B, H, N, D), f32), TypeError
    elif case == "v_shape":
        v = t((B, H, N, 2 * D), bf16)
    elif case == "out_dtype":
        kw["out"], err = t((B, H, N, D), f32), TypeError
    elif case == "out_shape":
        kw["out"] = t((B, H, N - 1, D), bf16)
    elif case == "lse_shape":
        kw["lse"] = t((B, H, N + 3), f32)
    elif case == "lse_dtype":
        kw["lse"], err = t((B, H, N), bf16), TypeError
    elif case == "q_3d":
        q = t((B * H, N, D), bf16)
    elif case == "scale_for_bf16":
        kw["q_scale"] = t((B, H, N), f32)
    with pytest.raises(err) as exc:
        pna.attn_fwd_flash(q, k, v, causal=False, **kw)
    assert "CUDA" not in str(exc.value)


@pytest.mark.parametrize("code_dtype", [torch.int8, torch.uint8])
def test_flash_scaled_qk_needs_matching_scales(code_dtype):
    q, k = t((B, H, N, D), code_dtype), t((B, H, N, D), code_dtype)
    v = t((B, H, N, D), bf16)
    good = t((B, H, N), f32)
    with pytest.raises(ValueError, match="q_scale is required"):
        pna.attn_fwd_flash(q, k, v, causal=False, k_scale=good)
    with pytest.raises(ValueError, match="k_scale has shape"):
        pna.attn_fwd_flash(q, k, v, causal=False, q_scale=good, k_scale=t((B, H, N - 1), f32))
    with pytest.raises(TypeError, match="k_scale has dtype"):
        pna.attn_fwd_flash(q, k, v, causal=False, q_scale=good, k_scale=t((B, H, N), bf16))
    with pytest.raises(TypeError, match="v has dtype"):
        pna.attn_fwd_flash(q, k, t((B, H, N, D), f32), causal=False, q_scale=good,
                           k_scale=good)
    with pytest.raises(ValueError, match="CUDA"):
        pna.attn_fwd_flash(q, k, v, causal=False, q_scale=good, k_scale=good)


def test_debug_s_rejects_a_short_score_buffer():
    q, k = t((B, H, N, D), torch.int8), t((B, H, N, D), torch.int8)
    v, sc = t((B, H, N, D), bf16), t((B, H, N), f32)
    with pytest.raises(ValueError, match="s_out has shape"):
        pna.attn_fwd_flash_debug_s(q, k, v, causal=False, q_scale=sc, k_scale=sc,
                                   s_out=t((B, H, N, N - 1), torch.int32))
    with pytest.raises(TypeError, match="s_out has dtype"):
        pna.attn_fwd_flash_debug_s(q, k, v, causal=False, q_scale=sc, k_scale=sc,
                                   s_out=t((B, H, N, N), torch.int64))


def test_baseline_checks_like_flash():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="out has shape"):
        pna.attn_fwd_baseline(q, k, v, causal=True, out=t((B, H, N, D + 1), bf16))
    q32, k32, v32 = qkv(f32)
    with pytest.raises(TypeError, match="v has dtype"):
        pna.attn_fwd_baseline(q32, k32, t((B, H, N, D), bf16), causal=True)


def test_deviation_checks():
    with pytest.raises(TypeError, match="o_ref"):
        pna.attn_deviation(t(10, f32), t(10, f32))
    with pytest.raises(ValueError, match="size"):
        pna.attn_deviation(t(10, f32), t(11, torch.float64))
    with pytest.raises(TypeError, match="o_test"):
        pna.attn_deviation(t(10, torch.float64), t(10, torch.float64))


@pytest.mark.parametrize("fn,code", [(pna.attn_quantize_int8, torch.int8),
                                     (pna.attn_quantize_fp8, torch.uint8)])
def test_quantiser_checks(fn, code):
    x = t((5, 64), f32)
    with pytest.raises(TypeError, match="x has dtype"):
        fn(t((5, 64), bf16))
    with pytest.raises(ValueError, match="codes has shape"):
        fn(x, codes=t((5, 63), code))
    with pytest.raises(TypeError, match="codes has dtype"):
        fn(x, codes=t((5, 64), torch.int32))
    with pytest.raises(ValueError, match="scales has shape"):
        fn(x, scales=t((6,), f32))


def test_tile_quantiser_checks():
    with pytest.raises(ValueError, match=r"\[\.\.\., n, d\]"):
        pna.attn_quantize_int8_tiles(t((64,), f32), 4)
    with pytest.raises(ValueError, match="scales has shape"):
        pna.attn_quantize_int8_tiles(t((3, 8, 64), f32), 4, scales=t((3, 8, 1), f32))


def test_delta_checks():
    o = t((B, H, N, D), bf16)
    with pytest.raises(TypeError, match="d_o has dtype"):
        pna.attn_bwd_delta(o, t((B, H, N, D), f32))
    with pytest.raises(ValueError, match="delta has shape"):
        pna.attn_bwd_delta(o, o.clone(), delta=t((B, H), f32))
    with pytest.raises(TypeError, match="o has dtype"):
        pna.attn_bwd_delta(t((B, H, N, D), torch.int8), t((B, H, N, D), torch.int8))


def test_backward_checks():
    q, k, v = qkv()
    o, d_o, lse = t((B, H, N, D), bf16), t((B, H, N, D), bf16), t((B, H, N), f32)
    with pytest.raises(ValueError, match="lse has shape"):
        pna.attn_bwd_flash(q, k, v, o, d_o, t((B, H, N + 1), f32), causal=True)
    with pytest.raises(TypeError, match="d_o has dtype"):
        pna.attn_bwd_flash(q, k, v, o, t((B, H, N, D), f32), lse, causal=True)
    with pytest.raises(ValueError, match="dk has shape"):
        pna.attn_bwd_flash(q, k, v, o, d_o, lse, causal=True, dk=t((B, H, N, D // 2), bf16))
    with pytest.raises(TypeError, match="bfloat16"):
        pna.attn_bwd_flash(*qkv(f32), t((B, H, N, D), f32), t((B, H, N, D), f32), lse,
                           causal=True)


def test_wasserstein_checks():
    with pytest.raises(ValueError, match="size"):
        pna.attn_wasserstein(t(10, f32), t(9, f32))
    with pytest.raises(TypeError):
        pna.attn_wasserstein(t(10, torch.int8), t(10, f32))


@pytest.mark.parametrize("call", ["wasserstein", "deviation", "deviation_noalloc", "delta",
                                  "quant", "tiles", "fp8", "baseline", "backward", "debug_s"])
def test_well_formed_calls_reach_the_device_check(call):
    """Every binding function runs its checks to the end on well-formed CPU
    tensors and stops at the device check (no Python error on the way)."""
    q, k, v = qkv()
    i8, sc = t((B, H, N, D), torch.int8), t((B, H, N), f32)
    calls = {
        "wasserstein": lambda: pna.attn_wasserstein(t(10, f32), t(10, torch.float64)),
        "deviation": lambda: pna.attn_deviation(t(10, f32), t(10, torch.float64)),
        "deviation_noalloc": lambda: pna.attn_deviation_noalloc(t(10, bf16),
                                                                t(10, torch.float64)),
        "delta": lambda: pna.attn_bwd_delta(q, q.clone()),
        "quant": lambda: pna.attn_quantize_int8(t((5, 64), f32)),
        "tiles": lambda: pna.attn_quantize_int8_tiles(t((2, 5, 64), f32), 2),
        "fp8": lambda: pna.attn_quantize_fp8(t((5, 64), f32)),
        "baseline": lambda: pna.attn_fwd_baseline(q, k, v, causal=True),
        "backward": lambda: pna.attn_bwd_flash(q, k, v, q.clone(), q.clone(),
                                               t((B, H, N), f32), causal=True),
        "debug_s": lambda: pna.attn_fwd_flash_debug_s(i8, i8.clone(), v, causal=False,
                                                      q_scale=sc, k_scale=sc,
                                                      s_out=t((B, H, N, N), torch.int32)),
    }
    with pytest.raises(ValueError, match="CUDA"):
        calls[call]()


def test_out_f32_needs_an_fp32_buffer():
    q, k, v = qkv()
    with pytest.raises(TypeError, match="out has dtype"):
        pna.attn_fwd_flash(q, k, v, causal=True, out_f32=True, out=t((B, H, N, D), bf16))
    with pytest.raises(ValueError, match="CUDA"):
        pna.attn_fwd_flash(q, k, v, causal=True, out_f32=True, out=t((B, H, N, D), f32))
