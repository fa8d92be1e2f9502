"""Seeded input generators: encodings and reproducibility (CPU only)."""
import numpy as np
import pytest
import torch

import synth


def test_bf16_encoding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),     # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-45], np.float32),
        # exact ties: lower 16 bits 0x8000, both parities of the kept lsb
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x7F7F8000], np.uint32).view(np.float32),
    ])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16)
                          .to(torch.float32).numpy())


def test_bf16_nan_stays_nan():
    x = np.array([np.nan, -np.nan], np.float32)
    b = synth.f32_to_bf16_bits(x)
    assert np.isnan(synth.bf16_bits_to_f32(b)).all()


@pytest.mark.parametrize("name", ["c1", "c2", "c5"])
def test_inputs_are_reproducible(name):
    cfg = synth.small(synth.CONFIGS[name], batch=1, heads=2, seq_len=64)
    a = synth.make_inputs(cfg)
    b = synth.make_inputs(cfg)
    assert a.digest() == b.digest()
    c = synth.make_inputs(cfg, seed=cfg.seed + 100)
    assert a.digest() != c.digest()


def test_lowrank_inputs_share_a_rank4_component():
    cfg = synth.small(synth.CONFIGS["c4"], heads=2, seq_len=512)
    inp = synth.make_inputs(cfg)
    q = synth.bf16_bits_to_f32(inp.q).astype(np.float64)
    k = synth.bf16_bits_to_f32(inp.k).astype(np.float64)
    # Q and K are 0.9 * (same rank-4 component) + 0.1 * noise: their difference
    # is noise of std 0.1*sqrt(2), and Q has 4 dominant singular values
    diff = (q - k).std()
    assert 0.12 < diff < 0.16
    sv = np.linalg.svd(q[0, 0], compute_uv=False)
    assert sv[3] > 10 * sv[4]
    v = synth.bf16_bits_to_f32(inp.v)
    assert abs(v.std() - 1.0) < 0.02


def test_config_flop_counts():
    c3 = synth.CONFIGS["c3"]
    assert c3.flops() == 2.0 * 4 * 32 * 128 * 4096 * 4097
    c5 = synth.CONFIGS["c5"]
    assert c5.flops() == 4.0 * 4 * 32 * 2048 * 2048 * 128
