"""The seeded generators: determinism, bf16 rounding, weight distributions and
the congested layer's calibrated router bias."""
import math

import numpy as np
import torch

import workloads
from oracle.switch_oracle import router_logits, softmax_top1, capacity


def test_bf16_rounding_matches_torch():
    a = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    a[:4] = [0.0, -0.0, 1e-40, -3.0e38]
    ours = workloads.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = workloads.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_deterministic_and_per_expert_streams():
    cfg = workloads.CONFIGS[1]
    a = workloads.make_layer_inputs(cfg)
    b = workloads.make_layer_inputs(cfg)
    np.testing.assert_array_equal(a.x_bits, b.x_bits)
    np.testing.assert_array_equal(a.w1_bits, b.w1_bits)
    np.testing.assert_array_equal(a.w2_bits[3], workloads.expert_w2_bits(cfg, 3))
    assert a.x_bits.shape == (512, 64) and a.w1_bits.shape == (4, 128, 64) and a.w2_bits.shape == (4, 64, 128)
    assert a.b_r[0] == 2.0 and np.all(a.b_r[1:] == 0)


def test_weight_distributions():
    cfg = workloads.CONFIGS[2]
    w1 = workloads.bf16_bits_to_f32(workloads.expert_w1_bits(cfg, 0))
    sigma = 0.1 / math.sqrt(cfg.d)
    assert np.abs(w1).max() <= 2 * sigma * (1 + 2 ** -8)
    # truncated at 2 sigma: std = sigma * 0.8796
    assert abs(w1.std() / sigma - 0.8796) < 0.01
    inp = workloads.make_router_inputs(cfg)
    assert abs(inp.w_r.std() - math.sqrt(0.1 / cfg.d)) < 0.01 * math.sqrt(0.1 / cfg.d)
    x = inp.x
    assert abs(x.std() - 1) < 0.01


def test_tiny_layer_forces_congestion():
    cfg = workloads.CONFIGS[1]
    inp = workloads.make_router_inputs(cfg)
    r = softmax_top1(router_logits(inp.x, inp.w_r, inp.b_r))
    C = capacity(cfg.T, cfg.E, cfg.c)
    counts = np.bincount(r.expert, minlength=cfg.E)
    assert C == 160 and counts[0] > C


def test_congested_bias_gives_fifteen_percent():
    cfg = workloads.CONFIGS[3]
    inp = workloads.make_router_inputs(cfg)
    share = np.mean(np.argmax(router_logits(inp.x, inp.w_r, inp.b_r), axis=1) == 0)
    assert abs(share - 0.15) <= 0.005, share


def test_tie_heavy_logits():
    z = workloads.tie_heavy_logits(1000, 8, 3)
    assert set(np.unique(z * 4).astype(int)) <= set(range(-3, 4))
    ties = np.sum((z == z.max(axis=1, keepdims=True)).sum(axis=1) > 1)
    assert ties > 300
