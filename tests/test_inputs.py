"""Checks of the seeded input generator (shapes, trees, page tables, bf16 rounding)."""
import numpy as np
import pytest
import torch

from gen import CONFIGS, get_config, make_inputs, make_tree_parents
from gen.inputs import round_to_bf16


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32) * 7
    # include exact ties (low half = 0x8000) to check ties-to-even
    x[:8] = np.array([1.00390625, 1.01171875, -3.0078125, 0.0, 1.0, -2.5, 1e-3, 65504.0], np.float32)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(round_to_bf16(x.copy()), ref)


@pytest.mark.parametrize("kind", ["uniform", "bounded", "chain"])
def test_tree_parents_are_topological(kind):
    rng = np.random.default_rng(1)
    for n in (1, 2, 16, 64):
        p = make_tree_parents(rng, n, kind)
        assert p[0] == -1
        assert all(0 <= p[i] < i for i in range(1, n))


def test_bounded_tree_limits():
    rng = np.random.default_rng(2)
    for _ in range(20):
        p = make_tree_parents(rng, 64, "bounded", max_depth=8, max_branch=4)
        depth = np.zeros(64, int)
        depth[0] = 1
        for i in range(1, 64):
            depth[i] = depth[p[i]] + 1
        assert depth.max() <= 8
        assert np.bincount(p[1:], minlength=64).max() <= 4


def test_tiny_config_shapes_and_determinism():
    cfg = get_config("tiny_f32_b1_h16_p256_t8")
    a, b = make_inputs(cfg), make_inputs(cfg)
    assert a.q_nope.shape == (8, 16, 512) and a.q_pe.shape == (8, 16, 64)
    assert a.kv_c.shape == (264, 512) and a.k_pe.shape == (264, 64)
    assert list(a.kv_indptr) == [0, 264]
    np.testing.assert_array_equal(a.kv_indices, np.arange(264))
    for k in ("q_nope", "q_pe", "kv_c", "k_pe", "parents"):
        np.testing.assert_array_equal(getattr(a, k), getattr(b, k))
    assert a.scale == pytest.approx(1 / np.sqrt(192))


def test_bf16_config_values_are_bf16_exact():
    cfg = get_config("b1_h64_p4096_t16_bf16", prefix=64)
    x = make_inputs(cfg)
    for arr in (x.q_nope, x.q_pe, x.kv_c, x.k_pe):
        assert (arr.view(np.uint32) & 0xFFFF).max() == 0
    assert 0.4 < x.q_nope.std() < 0.6
    assert 0.9 < x.kv_c.std() < 1.1


def test_paged_config_small_pool():
    cfg = get_config("b8_h64_paged600k_t16_bf16", prefix_range=(5, 40), pool_slots=1000, heads=2)
    x = make_inputs(cfg, poison_unused=True)
    lens = x.kv_lens
    assert (lens >= 5 + 16).all() and (lens <= 40 + 16).all()
    idx = x.kv_indices
    assert len(np.unique(idx)) == len(idx) == lens.sum()
    used = np.zeros(1000, bool)
    used[idx] = True
    assert np.isnan(x.kv_c[~used]).all() and not np.isnan(x.kv_c[used]).any()


def test_named_configs_exist():
    assert len(CONFIGS) == 5
    big = get_config("b1_h64_p200000_t32_bf16_s256")
    assert big.num_splits == 256 and big.rows == 2048


def test_ragged_trees_are_packed():
    cfg = get_config("b4_h64_p32768_t64_bf16", prefix=10, heads=2, tree_nodes=256,
                     tree_range=(0, 256), tree_kind="uniform")
    x = make_inputs(cfg)
    Tb = x.tree_lens
    assert len(Tb) == 4 and (Tb >= 0).all() and (Tb <= 256).all()
    assert x.parents.shape == (Tb.sum(),) and x.q_nope.shape == (Tb.sum(), 2, 512)
    assert x.rows == Tb.sum() * 2
    np.testing.assert_array_equal(x.kv_lens, 10 + Tb)
    for b in range(4):
        p = x.parents[x.tree_indptr[b]:x.tree_indptr[b + 1]]
        assert all(-1 <= p[i] < i for i in range(len(p)))
        if len(p):
            assert p[0] == -1
    y = make_inputs(cfg, tree_lens=[3, 0, 70, 1])
    assert list(y.tree_indptr) == [0, 3, 3, 73, 74]


def test_uniform_workloads_keep_their_draws():
    """The tree-size draw happens only for ragged workloads: a uniform workload
    draws exactly as before (first values fixed here)."""
    x = make_inputs(get_config("tiny_f32_b1_h16_p256_t8"))
    assert list(x.tree_indptr) == [0, 8] and x.parents.shape == (1, 8)
    rng = np.random.default_rng(0)
    parents = make_tree_parents(rng, 8, "uniform")
    np.testing.assert_array_equal(x.parents[0], parents)
    np.testing.assert_array_equal(x.q_nope.reshape(-1)[:5], rng.standard_normal(8 * 16 * 512, dtype=np.float32)[:5])
