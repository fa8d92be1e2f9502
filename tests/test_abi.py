"""The C-ABI library: it loads, exports every declared entry point, and its
host-side validation rejects bad arguments before any HIP call (CPU only:
no computation is launched)."""
import ctypes
import os
import re

import pytest

import precision_numerics_amd as pna
from precision_numerics_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for fname in os.listdir(os.path.join(ROOT, "include")):
        if fname.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fname)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def clib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libpnattn.so is not built: run __graft_entry__.build()")
    return pna.load()


def test_exports_every_declared_symbol(clib):
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(clib, name), name
    assert set(names) == set(B._SIGNATURES), "binding and header disagree"


def _prob(**kw):
    base = dict(batch=1, heads=2, seq_len=16, head_dim=64, causal=0, dtype=B.ATTN_BF16,
                p_bf16=1, softmax_scale=0.0, stabilized=0, beta=0.0)
    base.update(kw)
    return B.AttnProblem(**base)


FAKE = 0x1000  # never dereferenced: every case below fails validation first


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), B.ATTN_ERR_UNSUPPORTED),
    (dict(head_dim=0), B.ATTN_ERR_INVALID_ARG),
    (dict(batch=-1), B.ATTN_ERR_INVALID_ARG),
    (dict(seq_len=(1 << 22) + 1), B.ATTN_ERR_UNSUPPORTED),
    (dict(batch=1 << 16, heads=1 << 8, seq_len=1 << 22), B.ATTN_ERR_UNSUPPORTED),  # tiles
    (dict(causal=2), B.ATTN_ERR_INVALID_ARG),
    (dict(p_bf16=7), B.ATTN_ERR_INVALID_ARG),
    (dict(dtype=9), B.ATTN_ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), B.ATTN_ERR_INVALID_ARG),
    (dict(stabilized=1), B.ATTN_ERR_INVALID_ARG),            # beta missing
    (dict(stabilized=1, beta=1.0), B.ATTN_ERR_INVALID_ARG),  # beta must exceed 1
    (dict(stabilized=1, beta=float("inf")), B.ATTN_ERR_INVALID_ARG),
    (dict(stabilized=2, beta=2.0), B.ATTN_ERR_INVALID_ARG),
    (dict(stabilized=0, beta=2.0), B.ATTN_ERR_INVALID_ARG),  # beta without the variant
    (dict(stabilized=1, beta=2.0, dtype=B.ATTN_F32), B.ATTN_ERR_UNSUPPORTED),
    (dict(dtype=B.ATTN_INT8), B.ATTN_ERR_INVALID_ARG),       # scales missing
    (dict(o_f32=2), B.ATTN_ERR_INVALID_ARG),
])
def test_flash_validation(clib, kw, status):
    p = _prob(**kw)
    rc = clib.attn_fwd_flash(ctypes.byref(p), FAKE, FAKE, FAKE, None, None, FAKE, None, None)
    assert rc == status
    assert clib.attn_last_error().decode()


def test_baseline_rejects_stabilized(clib):
    p = _prob(stabilized=1, beta=2.0)
    rc = clib.attn_fwd_baseline(ctypes.byref(p), FAKE, FAKE, FAKE, None, None, FAKE, 1 << 20,
                                FAKE, None)
    assert rc == B.ATTN_ERR_UNSUPPORTED
    assert "flash" in clib.attn_last_error().decode()


def test_delta_validation(clib):
    p = _prob()
    assert clib.attn_bwd_delta(None, FAKE, FAKE, FAKE, None) == B.ATTN_ERR_INVALID_ARG
    assert clib.attn_bwd_delta(ctypes.byref(p), None, FAKE, FAKE, None) == B.ATTN_ERR_INVALID_ARG
    assert clib.attn_bwd_delta(ctypes.byref(p), FAKE, FAKE, None, None) == B.ATTN_ERR_INVALID_ARG
    bad = _prob(head_dim=80)
    assert clib.attn_bwd_delta(ctypes.byref(bad), FAKE, FAKE, FAKE, None) == B.ATTN_ERR_UNSUPPORTED
    bad = _prob(dtype=5)
    assert clib.attn_bwd_delta(ctypes.byref(bad), FAKE, FAKE, FAKE, None) == B.ATTN_ERR_INVALID_ARG
    empty = _prob(seq_len=0)
    assert clib.attn_bwd_delta(ctypes.byref(empty), None, None, None, None) == B.ATTN_OK


def test_null_pointers_rejected(clib):
    p = _prob()
    assert clib.attn_fwd_flash(None, FAKE, FAKE, FAKE, None, None, FAKE, None, None) == 1
    assert clib.attn_fwd_flash(ctypes.byref(p), None, FAKE, FAKE, None, None, FAKE, None, None) == 1
    assert clib.attn_fwd_flash(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None) == 1


def test_empty_problem_is_a_noop(clib):
    for kw in (dict(batch=0), dict(heads=0), dict(seq_len=0)):
        p = _prob(**kw)
        assert clib.attn_fwd_flash(ctypes.byref(p), None, None, None, None, None, None, None,
                                   None) == 0
        assert clib.attn_last_error().decode() == ""
        assert clib.attn_fwd_baseline(ctypes.byref(p), None, None, None, None, None, None, 0,
                                      None, None) == 0


def test_baseline_workspace_checks(clib):
    p = _prob(seq_len=100)
    n = ctypes.c_size_t(0)
    assert clib.attn_baseline_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
    assert n.value == 1 * 2 * 100 * 100 * (4 + 2) + 256   # S, P, tail padding
    p32 = _prob(seq_len=100, p_bf16=0)
    assert clib.attn_baseline_workspace_size(ctypes.byref(p32), ctypes.byref(n)) == 0
    assert n.value == 1 * 2 * 100 * 100 * 8 + 256
    rc = clib.attn_fwd_baseline(ctypes.byref(p), FAKE, FAKE, FAKE, None, None, FAKE, 100, FAKE,
                                None)
    assert rc == B.ATTN_ERR_WORKSPACE


def test_debug_s_requires_int8(clib):
    p = _prob()
    rc = clib.attn_fwd_flash_debug_s(ctypes.byref(p), FAKE, FAKE, FAKE, None, None, FAKE, FAKE,
                                     None)
    assert rc == B.ATTN_ERR_UNSUPPORTED


def test_deviation_validation(clib):
    out = B.AttnDeviation()
    assert clib.attn_deviation(FAKE, 5, FAKE, 10, FAKE, 1 << 20, ctypes.byref(out), None) == 1
    assert clib.attn_deviation(FAKE, 1, FAKE, 10, FAKE, 8, ctypes.byref(out), None) == 3
    assert clib.attn_deviation(None, 1, None, 0, None, 0, ctypes.byref(out), None) == 0
    assert out.n == 0 and out.argmax == -1
    b = ctypes.c_size_t(0)
    assert clib.attn_deviation_scratch_size(-1, ctypes.byref(b)) == 1


def test_quantize_validation(clib):
    assert clib.attn_quantize_int8(FAKE, 4, 0, FAKE, FAKE, None) == 1
    assert clib.attn_quantize_int8(FAKE, 4, 2000, FAKE, FAKE, None) == 1
    assert clib.attn_quantize_int8(None, 0, 64, None, None, None) == 0


def test_status_strings(clib):
    for s in range(5):
        assert clib.attn_status_string(s).decode()
    assert "gfx950" in clib.attn_version().decode()


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        B.load(str(tmp_path / "libpnattn.so"))


def test_wasserstein_validation(clib):
    out = B.AttnWasserstein()
    n = ctypes.c_size_t(0)
    W = clib.attn_wasserstein
    assert W(FAKE, B.ATTN_BF16, FAKE, B.ATTN_F64, 10, FAKE, 1 << 30, None, None) == 1
    assert W(FAKE, B.ATTN_INT8, FAKE, B.ATTN_F64, 10, FAKE, 1 << 30, ctypes.byref(out), None) == 1
    assert W(FAKE, B.ATTN_BF16, FAKE, 7, 10, FAKE, 1 << 30, ctypes.byref(out), None) == 1
    assert W(FAKE, B.ATTN_BF16, FAKE, B.ATTN_F64, -1, FAKE, 1 << 30, ctypes.byref(out), None) == 1
    assert W(FAKE, B.ATTN_BF16, FAKE, B.ATTN_F64, 1 << 31, FAKE, 1 << 40, ctypes.byref(out),
             None) == 1
    assert W(None, B.ATTN_BF16, FAKE, B.ATTN_F64, 10, FAKE, 1 << 30, ctypes.byref(out), None) == 1
    assert W(FAKE, B.ATTN_BF16, FAKE, B.ATTN_F64, 10, FAKE, 16, ctypes.byref(out), None) == 3
    assert W(None, B.ATTN_BF16, None, B.ATTN_F64, 0, None, 0, ctypes.byref(out), None) == 0
    assert out.n == 0 and out.w1 != out.w1          # NaN: no distribution
    assert clib.attn_wasserstein_scratch_size(100, B.ATTN_BF16, B.ATTN_F64, ctypes.byref(n)) == 0
    assert n.value >= 100 * 2 * (2 + 8)
    assert clib.attn_wasserstein_scratch_size(100, B.ATTN_INT8, B.ATTN_F64, ctypes.byref(n)) == 1


def test_f64_is_not_an_attention_dtype(clib):
    p = _prob(dtype=B.ATTN_F64)
    assert clib.attn_fwd_flash(ctypes.byref(p), FAKE, FAKE, FAKE, None, None, FAKE, None,
                               None) == B.ATTN_ERR_INVALID_ARG
    out = B.AttnDeviation()
    assert clib.attn_deviation(FAKE, B.ATTN_F64, FAKE, 10, FAKE, 1 << 20, ctypes.byref(out),
                               None) == B.ATTN_ERR_INVALID_ARG


def test_fp8_validation(clib):
    p = _prob(dtype=B.ATTN_FP8)
    assert clib.attn_fwd_flash(ctypes.byref(p), FAKE, FAKE, FAKE, None, None, FAKE, None,
                               None) == B.ATTN_ERR_INVALID_ARG          # scales missing
    assert "ATTN_FP8" in clib.attn_last_error().decode()
    p = _prob(dtype=B.ATTN_FP8, stabilized=1, beta=2.0)
    assert clib.attn_fwd_flash(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                               None) == B.ATTN_ERR_UNSUPPORTED
    p = _prob(dtype=B.ATTN_FP8)
    assert clib.attn_fwd_flash_debug_s(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       None) == B.ATTN_ERR_UNSUPPORTED
    assert clib.attn_quantize_fp8(FAKE, 4, 0, FAKE, FAKE, None) == 1
    assert clib.attn_quantize_fp8(FAKE, 4, 2000, FAKE, FAKE, None) == 1
    assert clib.attn_quantize_fp8(None, 0, 64, None, None, None) == 0


def test_tile_quantiser_validation(clib):
    Q = clib.attn_quantize_int8_tiles
    assert Q(FAKE, 2, 16, 0, 4, FAKE, FAKE, None) == 1
    assert Q(FAKE, 2, 16, 64, 0, FAKE, FAKE, None) == 1
    assert Q(FAKE, -1, 16, 64, 4, FAKE, FAKE, None) == 1
    assert Q(None, 2, 16, 64, 4, FAKE, FAKE, None) == 1
    assert Q(None, 0, 16, 64, 4, None, None, None) == 0
    assert Q(None, 2, 0, 64, 4, None, None, None) == 0


def test_backward_validation(clib):
    p = _prob()
    n = ctypes.c_size_t(0)
    assert clib.attn_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
    assert n.value == 1 * 2 * 16 * 4
    BW = clib.attn_bwd_flash
    args = [FAKE] * 10       # q, k, v, o, d_o, lse, dq, dk, dv, workspace
    assert BW(ctypes.byref(p), *args[:5], None, *args[6:], 1 << 20, None) == 1       # lse NULL
    assert BW(ctypes.byref(p), *args[:9], None, 1 << 20, None) == 1                   # workspace NULL
    assert BW(ctypes.byref(p), *args, 8, None) == 3                                   # too small
    p8 = _prob(dtype=B.ATTN_INT8)
    assert BW(ctypes.byref(p8), *args, 1 << 20, None) == 1                            # scales
    pf = _prob(dtype=B.ATTN_F32)
    assert BW(ctypes.byref(pf), *args, 1 << 20, None) == 2
    ps = _prob(stabilized=1, beta=2.0)
    assert BW(ctypes.byref(ps), *args, 1 << 20, None) == 2
    empty = _prob(seq_len=0)
    assert BW(ctypes.byref(empty), *([None] * 10), 0, None) == 0


def test_backward_takes_bf16_output(clib):
    p = _prob(o_f32=1)
    rc = clib.attn_bwd_flash(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, FAKE, 1 << 20, None)
    assert rc == B.ATTN_ERR_UNSUPPORTED
    assert "bf16" in clib.attn_last_error().decode()
