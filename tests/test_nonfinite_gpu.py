"""Non-finite inputs reach the output, and the deviation harness counts them.

A NaN or an infinity in Q, K or V has a defined effect on the plain
definition S = scale QK^T, P = softmax(S), O = PV ("Is Flash Attention
Stable?", abstract: the forward pass whose deviation is measured): a NaN in
query row i makes row i of O NaN; a NaN in key row j makes every row that
sees key j NaN (all rows, or rows i >= j under the causal mask) and leaves
the others alone, since masked keys are dropped before the exponentials; an
infinity in V row 0 (seen by every row) makes that column of O non-finite
everywhere; an infinity in a query row makes its row max +inf and the row
NaN.  Both kernels must reproduce the FP64 oracle's pattern of non-finite
elements exactly, agree with it at the bf16 tolerances everywhere else, and
attn_deviation must count the non-finite elements.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from helpers import BF16_MAX_ABS, BF16_MEAN_ABS, out_to_f64, torch_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

B, H, N, D = 1, 2, 300, 64


def _inputs(case, seed=11):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, H, N, D)).astype(np.float32) for _ in range(3))
    if case == "q_nan":
        q[0, 1, 37, 5] = np.nan
    elif case == "k_nan":
        k[0, 0, 100, 3] = np.nan
    elif case == "v_inf":
        v[0, 1, 0, 7] = np.inf
    elif case == "q_inf":
        q[0, 0, 50, 9] = np.inf
    elif case == "k_neg_inf":
        k[0, 1, 260, 0] = -np.inf
    bits = [synth.f32_to_bf16_bits(x) for x in (q, k, v)]
    wide = [synth.bf16_bits_to_f32(b).astype(np.float64) for b in bits]
    return bits, wide


@pytest.mark.parametrize("kernel", ["flash", "baseline"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", ["q_nan", "k_nan", "v_inf", "q_inf", "k_neg_inf"])
def test_nonfinite_inputs_propagate(lib, kernel, causal, case):
    import precision_numerics_amd as pna
    bits, wide = _inputs(case)
    q, k, v = (torch_bf16(b) for b in bits)
    print(f"nonfinite {kernel} causal={causal} case={case}", flush=True)
    if kernel == "flash":
        o = pna.attn_fwd_flash(q, k, v, causal=causal)
    else:
        o, _ = pna.attn_fwd_baseline(q, k, v, causal=causal)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):
        ref, _ = oracle.attention(*wide, causal=causal)
    got = out_to_f64(o)
    bad_ref = ~np.isfinite(ref)
    bad_got = ~np.isfinite(got)
    assert bad_ref.any(), "the case must produce non-finite output"
    assert np.array_equal(bad_got, bad_ref), (
        f"{int(bad_got.sum())} non-finite on the GPU, {int(bad_ref.sum())} in the oracle")
    fin = ~bad_ref
    err = np.abs(got[fin] - ref[fin])
    assert err.max() <= BF16_MAX_ABS and err.mean() <= BF16_MEAN_ABS
    dev = pna.attn_deviation(o, torch.from_numpy(ref).cuda())
    assert dev["n_nonfinite"] == int(bad_ref.sum())
    assert dev["n"] == ref.size
    assert dev["max_abs"] == float(err.max())
