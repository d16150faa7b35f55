"""The seeded input generator: shapes, tree bounds, bf16 rounding, determinism."""

import numpy as np
import pytest
import torch

from workloads import (CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_custom, make_workload,
                       tree_bounded, tree_depths, tree_uniform)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -3.4e38], np.float32)])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("max_depth,max_fanout", [(5, 4), (6, None), (8, None), (1, None), (2, 2)])
def test_bounded_trees_respect_bounds(max_depth, max_fanout):
    rng = np.random.default_rng(1)
    for _ in range(50):
        T = 7 if (max_depth, max_fanout) == (2, 2) else 64
        p = tree_bounded(T, rng, max_depth, max_fanout)
        assert p[0] == -1 and all(-1 <= p[i] < i for i in range(1, T))
        assert all(p[i] >= 0 for i in range(1, T))
        assert tree_depths(p).max() <= max_depth
        if max_fanout is not None:
            assert np.bincount(p[1:], minlength=T).max() <= max_fanout


def test_uniform_trees_are_topological():
    rng = np.random.default_rng(2)
    for _ in range(20):
        p = tree_uniform(32, rng)
        assert p[0] == -1 and all(0 <= p[i] < i for i in range(1, 32))


def test_small_workloads_are_deterministic_and_shaped():
    for key in (1, 2):
        a, b = make_workload(key), make_workload(key)
        c = CONFIGS[key]
        assert a.q.shape == (c.B, c.Hq, c.T, c.D)
        assert a.k_cache.shape == (c.B, c.Hkv, c.Lcap, c.D)
        assert a.k_tree.shape == (c.B, c.Hkv, c.T, c.D)
        assert a.parent.shape == (c.B, c.T)
        for name in ("q", "k_cache", "v_cache", "k_tree", "v_tree", "parent", "prefix_len"):
            assert np.array_equal(getattr(a, name), getattr(b, name))
        assert a.q.dtype == (np.float32 if c.dtype == "f32" else np.uint16)


def test_ragged_tail_is_zero_or_poison():
    w = make_custom(B=2, Hq=2, Hkv=1, D=8, Lcap=20, T=3, prefix_len=[13, 20], seed=3)
    assert np.all(w.k_cache[0, :, 13:] == 0) and np.any(w.k_cache[0, :, :13] != 0)
    p = make_custom(B=2, Hq=2, Hkv=1, D=8, Lcap=20, T=3, prefix_len=[13, 20], seed=3, poison_tail=True)
    assert np.all(np.isnan(bf16_bits_to_f32(p.v_cache[0, :, 13:])))
    assert np.array_equal(p.k_cache[1], w.k_cache[1])
