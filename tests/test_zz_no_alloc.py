"""attn_deviation_noalloc (the library's own scratch array, no allocation)
gives bitwise the statistics of attn_deviation with a caller-provided
scratch buffer, on two calls in a row, the second with a smaller input (so
the array still holds the first call's partials when the second starts)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from helpers import torch_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _case(n, dtype, seed):
    rng = np.random.default_rng(seed)
    ref = rng.standard_normal(n)
    test32 = (ref + rng.standard_normal(n) * 1e-3).astype(np.float32)
    if n > 10:
        test32[n // 3] = np.nan
        test32[5] = np.float32(ref[5] + 0.25)
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(test32)
        return torch_bf16(bits), synth.bf16_bits_to_f32(bits).astype(np.float64), ref
    return torch.from_numpy(test32).cuda(), test32.astype(np.float64), ref


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_scratch_entry_point(lib, dtype):
    import precision_numerics_amd as pna
    for n, seed in ((3_000_001, 1), (4097, 2), (1, 3)):
        print(f"noalloc deviation {dtype} n={n}", flush=True)
        t, test64, ref = _case(n, dtype, seed)
        ref_t = torch.from_numpy(ref).cuda()
        got = pna.attn_deviation_noalloc(t, ref_t)
        want = pna.attn_deviation(t, ref_t)
        assert got == want
        orc = oracle.deviation(test64, ref)
        assert got["n_nonfinite"] == orc["n_nonfinite"] and got["argmax"] == orc["argmax"]
        assert got["max_abs"] == orc["max_abs"]


def test_noalloc_empty_and_errors(lib):
    import precision_numerics_amd as pna
    e = torch.empty(0, dtype=torch.float32, device="cuda")
    r = torch.empty(0, dtype=torch.float64, device="cuda")
    got = pna.attn_deviation_noalloc(e, r)
    assert got["n"] == 0 and got["argmax"] == -1
    with pytest.raises(TypeError):
        pna.attn_deviation_noalloc(e, e)
