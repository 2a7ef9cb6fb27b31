"""The seeded input generators: determinism, independence of keys, shapes and
distribution moments (CPU only)."""
import math

import numpy as np
import torch

from synthetic import CONFIGS, make_layer, make_expert, make_tokens, host_array, seed_of
from synthetic.gen import make_centroids


def test_same_key_same_values():
    cfg = CONFIGS["tiny_fp32"]
    a = make_layer(cfg)
    b = make_layer(cfg)
    assert torch.equal(a.h, b.h) and torch.equal(a.e, b.e) and torch.equal(a.w_down, b.w_down)


def test_single_expert_redraw_matches_stack():
    cfg = CONFIGS["tiny_fp32"]
    lay = make_layer(cfg)
    wg, wu, wd = make_expert(cfg, 5)
    assert torch.equal(wg, lay.w_gate[5]) and torch.equal(wu, lay.w_up[5])
    assert torch.equal(wd, lay.w_down[5])


def test_keys_distinct():
    keys = {seed_of(0, c, t, i) for c in range(5) for t in ("h", "e", "w_gate", "w_up")
            for i in range(50)}
    assert len(keys) == 5 * 4 * 50


def test_moments_and_shapes():
    cfg = CONFIGS["tiny_fp32"].with_tokens(4096)
    lay = make_layer(cfg)
    assert lay.h.shape == (4096, 128) and lay.w_gate.shape == (8, 256, 128)
    assert lay.w_down.shape == (8, 128, 256)
    assert abs(lay.h.std().item() - 1.0) < 0.01
    assert abs(lay.w_gate.std().item() * math.sqrt(128) - 1.0) < 0.02
    assert abs(lay.w_down.std().item() * math.sqrt(256) - 1.0) < 0.02
    assert abs(lay.e.std().item() * math.sqrt(128) - 1.0) < 0.05
    assert torch.all(lay.b == 0)


def test_bf16_host_view_is_bit_exact():
    cfg = CONFIGS["dsv3_decode"].with_tokens(8)
    h = make_tokens(cfg)
    bits = host_array(h)
    assert bits.dtype == np.uint16
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, h.float().numpy())


def test_mixture_tokens_and_hot_centroids():
    cfg = CONFIGS["dsv3_skewed"].with_tokens(64)
    h = make_tokens(cfg).float()
    assert h.shape == (64, 7168)
    # the mixture shift has norm a = 4 on top of unit-variance noise
    assert abs(h.pow(2).sum(1).mean().item() - (7168 + 16)) < 400
    e0 = make_centroids(cfg, beta=0.0)
    e1 = make_centroids(cfg, beta=2.0)
    assert torch.equal(e0[8:], e1[8:])
    assert abs((e1[:8] - e0[:8]).norm(dim=1).mean().item() - 2.0) < 1e-3
