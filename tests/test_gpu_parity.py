"""GPU parity: libmlaverify (HIP, gfx950) against the float64 oracle.

Small cases compare every output element. The three large workloads are
compared in full (every node, head and feature) and on sampled tree nodes
that the oracle computes one by one, plus size-independent properties (split
invariance, determinism).
"""
import numpy as np
import pytest

from gen import get_config, make_inputs, make_tree_parents
from gpu_util import compare, log, node_rows, run_hip, run_oracle
from oracle import tree_ancestors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_absorbed_tree_amd.binding  # noqa: F401  (fails loudly if the library is missing)


def _full_case(cfg, num_splits=0, min_group=1, **gen_kw):
    x = make_inputs(cfg, **gen_kw)
    log("case %s splits=%d" % (cfg, num_splits))
    o, lse, info = run_hip(x, num_splits)
    assert info["splits_per_workgroup"] >= min_group, info
    o_ref, lse_ref = run_oracle(x)
    compare(o, lse, o_ref, lse_ref, cfg.dtype, "plan=%s" % info)
    return x, o, lse


# --------------------------------------------------------------------------
# named small workloads, every element
# --------------------------------------------------------------------------

def test_tiny_fp32_workload():
    _full_case(get_config("tiny_f32_b1_h16_p256_t8"))


@pytest.mark.parametrize("splits", [0, 1, 5])
def test_p4096_bf16_workload(splits):
    _full_case(get_config("b1_h64_p4096_t16_bf16"), splits)


# --------------------------------------------------------------------------
# ragged shapes, several tiles, forced splits
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("splits", [1, 2, 3, 7])
def test_ragged_rows_and_tail(dtype, splits):
    # 7 nodes x 5 heads = 35 rows (a partial row block); P = 70 leaves a partial last tile.
    cfg = get_config("b1_h64_p4096_t16_bf16", batch=3, heads=5, tree_nodes=7, prefix=70,
                     dtype=dtype, seed=21)
    _full_case(cfg, splits)


@pytest.mark.parametrize("splits", [0, 1, 2])
def test_empty_prefix_full_tree(splits):
    cfg = get_config("b4_h64_p32768_t64_bf16", batch=2, prefix=0, seed=22)
    _full_case(cfg, splits)


def test_single_node_tree_decode():
    cfg = get_config("b1_h64_p4096_t16_bf16", batch=4, tree_nodes=1, prefix=1000, seed=23)
    _full_case(cfg)


def test_chain_tree_64_nodes():
    cfg = get_config("b1_h64_p4096_t16_bf16", heads=8, tree_nodes=64, prefix=31, tree_kind="chain",
                     seed=24)
    _full_case(cfg, 2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_paged_pool_with_nan_poison(dtype):
    cfg = get_config("b8_h64_paged600k_t16_bf16", batch=5, heads=16, prefix_range=(1, 300),
                     pool_slots=5000, dtype=dtype, seed=25)
    _full_case(cfg, 0, poison_unused=True)


def test_bf16_many_heads_rows_span_blocks():
    # 16 nodes x 24 heads = 384 rows = 3 row blocks; nodes straddle block edges.
    cfg = get_config("b1_h64_p4096_t16_bf16", batch=2, heads=24, prefix=517, seed=26)
    _full_case(cfg, 3)


# --------------------------------------------------------------------------
# several consecutive splits per workgroup (one partial written per split)
# --------------------------------------------------------------------------

def test_split_groups_with_ragged_ends():
    # 3 sequences of 1336..2773 keys, 43 forced splits (42 for the sequence
    # of 42 tiles): the planner puts 5 splits in a workgroup, so each
    # sequence's last group is short (3 or 2 splits).
    cfg = get_config("b1_h64_p4096_t16_bf16", batch=3, prefix_range=(1000, 3000), seed=32)
    _full_case(cfg, 43, min_group=2)


def test_split_groups_partial_row_block_one_tile_splits():
    # 35 rows (one partial row block); 600 splits of 1-2 tiles, several per
    # workgroup (7: the last group of each sequence is short).
    cfg = get_config("b1_h64_p4096_t16_bf16", batch=2, heads=5, tree_nodes=7, prefix=20000, seed=33)
    _full_case(cfg, 600, min_group=4)


def test_split_groups_paged_nan_poison():
    # page_size=1 pool with NaN in every unused slot; 16 forced splits per
    # sequence, several per workgroup (4).
    cfg = get_config("b8_h64_paged600k_t16_bf16", batch=5, prefix_range=(600, 2000), pool_slots=20000,
                     seed=36)
    _full_case(cfg, 16, min_group=2, poison_unused=True)


def test_split_groups_tree64_tail_spans_tiles():
    # 64-node tree (its tail spans two key tiles), 32 row blocks, 16 splits,
    # 2 per workgroup: the last split of each group holds the masked tail.
    cfg = get_config("b4_h64_p32768_t64_bf16", batch=1, prefix=2000, seed=37)
    _full_case(cfg, 16, min_group=2)


def test_split_groups_late_spike_redo():
    """A prefix key near the end scores ~100 (log2 units) above the rest: the
    workgroup that meets it late in its group repeats the group with the exact
    max, rewriting every partial it already wrote."""
    cfg = get_config("b1_h64_p4096_t16_bf16", batch=2, prefix=4000, seed=34)
    x = make_inputs(cfg)
    rng = np.random.default_rng(35)
    direction = rng.standard_normal(576).astype(np.float32)
    direction /= np.linalg.norm(direction)
    x.q_nope[:] = 5.0 * direction[:512]
    x.q_pe[:] = 5.0 * direction[512:]
    spike = int(x.kv_indices[int(x.kv_indptr[0]) + 3500])  # slot of prefix position 3500
    x.kv_c[spike] = 200.0 * direction[:512]
    x.k_pe[spike] = 200.0 * direction[512:]
    from gen.inputs import round_to_bf16
    for a in (x.q_nope, x.q_pe, x.kv_c, x.k_pe):
        round_to_bf16(a)
    o, lse, info = run_hip(x, 100)
    assert info["splits_per_workgroup"] >= 2, info
    o_ref, lse_ref = run_oracle(x)
    compare(o, lse, o_ref, lse_ref, "bf16", "plan=%s" % info)
    assert np.abs(o[:cfg.tree_nodes] - x.kv_c[spike]).max() < 0.05  # sequence 0


@pytest.mark.parametrize("dtype,splits", [("bf16", 4), ("bf16", 8), ("f32", 6), ("bf16", 12), ("f32", 20)])
def test_plan_for_longer_kv_leaves_empty_split_groups(dtype, splits):
    """A plan built for 4000-key sequences runs on much shorter ones (plan
    reuse across decode steps): the run divides each sequence's actual tiles
    among the planned splits, so the later split groups get no key and write
    empty partials (m = -inf). Up to 8 groups per row the one-wave-per-row
    combine merges them, above that the lane-group combine; both must weigh
    the empty ones to nothing."""
    import torch
    from mla_absorbed_tree_amd.verify import MlaVerify, device_inputs
    base = "b1_h64_p4096_t16_bf16" if dtype == "bf16" else "tiny_f32_b1_h16_p256_t8"
    cfg = get_config(base, batch=3, heads=16, tree_nodes=8, prefix=None, prefix_range=(1, 70), seed=77)
    x = make_inputs(cfg)
    d = device_inputs(x)
    mv = MlaVerify(cfg.batch, cfg.heads, cfg.tree_nodes, cfg.dtype, np.full(cfg.batch, 4000), splits)
    assert mv.info["total_groups"] == cfg.batch * splits and mv.info["uses_combine"] == 1, mv.info
    o, lse = mv(d["q_nope"], d["q_pe"], d["kv_c"], d["k_pe"], d["kv_indptr"], d["kv_indices"], d["tree_parents"],
                x.scale)
    torch.cuda.synchronize()
    mv.close()
    log("  kv lens %s, plan %s" % (list(x.kv_lens), mv.info))
    o_ref, lse_ref = run_oracle(x)
    compare(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, dtype, "(%d splits)" % splits)


def test_interleaved_576_wide_cache():
    """kv_c and k_pe inside one [slots, 576] buffer via row strides."""
    import torch
    from mla_absorbed_tree_amd.verify import device_inputs
    cfg = get_config("b8_h64_paged600k_t16_bf16", batch=3, heads=16, prefix_range=(40, 200),
                     pool_slots=2000, seed=27)
    x = make_inputs(cfg)
    d = device_inputs(x)
    kv = torch.cat([d["kv_c"], d["k_pe"]], dim=1).contiguous()
    o, lse, _ = run_hip(x, 0, kv_c=kv, k_pe=kv[:, 512:], strides=(576, 576), device_tensors=d)
    o_ref, lse_ref = run_oracle(x)
    compare(o, lse, o_ref, lse_ref, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_planted_spike_mask(dtype):
    """One tail key dominates: only its descendants (and itself) may lock onto it."""
    cfg = get_config("b1_h64_p4096_t16_bf16", heads=8, tree_nodes=16, prefix=4, dtype=dtype,
                     seed=28)
    x = make_inputs(cfg)
    T, P = cfg.tree_nodes, 4
    rng = np.random.default_rng(29)
    direction = rng.standard_normal(576).astype(np.float32)
    direction /= np.linalg.norm(direction)
    x.q_nope[:] = 5.0 * direction[:512]
    x.q_pe[:] = 5.0 * direction[512:]
    u = 3  # planted tail node: score 250 * scale ~ 18 above the others
    x.kv_c[P + u] = 50.0 * direction[:512]
    x.k_pe[P + u] = 50.0 * direction[512:]
    if dtype == "bf16":
        from gen.inputs import round_to_bf16
        for a in (x.q_nope, x.q_pe, x.kv_c, x.k_pe):
            round_to_bf16(a)
    o, lse, _ = run_hip(x, 0)
    o_ref, lse_ref = run_oracle(x)
    compare(o, lse, o_ref, lse_ref, dtype)
    anc = tree_ancestors(x.parents[0])
    for t in range(T):
        near = np.abs(o[t] - x.kv_c[P + u]).max()
        assert (near < 0.05) == (u in anc[t]), (t, near)


# --------------------------------------------------------------------------
# full-size workloads, sampled nodes
# --------------------------------------------------------------------------

def _sampled(cfg_name, nodes, splits=0, **kw):
    cfg = get_config(cfg_name)
    x = make_inputs(cfg, **kw)
    log("case %s (sampled %d nodes)" % (cfg_name, len(nodes)))
    o, lse, info = run_hip(x, splits)
    o_ref, lse_ref = run_oracle(x, nodes=nodes)
    rows = node_rows(x, nodes)
    compare(o[rows], lse[rows], o_ref, lse_ref, cfg.dtype, "plan=%s" % info)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    return x, o, lse


def test_b4_p32768_t64_sampled():
    _sampled("b4_h64_p32768_t64_bf16", [(0, 0), (0, 63), (1, 17), (2, 40), (3, 5), (3, 62)])


def test_b1_p200000_t32_s256_sampled():
    _sampled("b1_h64_p200000_t32_bf16_s256", [(0, 0), (0, 13), (0, 31)])


def test_b8_paged600k_sampled():
    _sampled("b8_h64_paged600k_t16_bf16", [(0, 3), (2, 15), (4, 0), (5, 9), (7, 12)],
             poison_unused=True)


@pytest.mark.parametrize("name", ["b4_h64_p32768_t64_bf16", "b1_h64_p200000_t32_bf16_s256",
                                  "b8_h64_paged600k_t16_bf16", "b4_h64_p32768_t1to256_ragged_bf16"])
def test_full_size_every_node(name):
    """The large workloads at full size in the benchmark's launch configuration
    (the workload's own split setting), every output element against the
    oracle; the paged pool's unused slots hold NaN."""
    cfg = get_config(name)
    x = make_inputs(cfg, poison_unused=cfg.layout == "paged")
    log("case %s (every node)" % name)
    o, lse, info = run_hip(x, cfg.num_splits)
    o_ref, lse_ref = run_oracle(x)
    compare(o, lse, o_ref, lse_ref, cfg.dtype, "plan=%s" % info)


def test_split_invariance_at_full_size():
    cfg = get_config("b4_h64_p32768_t64_bf16")
    x = make_inputs(cfg)
    o1, l1, _ = run_hip(x, 1)
    o2, l2, info = run_hip(x, 0)
    o3, l3, _ = run_hip(x, 16)
    for o, l in ((o2, l2), (o3, l3)):
        assert np.abs(o - o1).max() < 2e-3
        assert np.abs(l - l1).max() < 1e-4


@pytest.mark.parametrize("name,splits,combine", [("b1_h64_p4096_t16_bf16", 1, "none"),
                                                ("b1_h64_p4096_t16_bf16", 4, "one wave per row"),
                                                ("b1_h64_p4096_t16_bf16", 40, "lane groups"),
                                                ("tiny_f32_b1_h16_p256_t8", 3, "one wave per row")])
def test_attend_then_combine_equals_run(name, splits, combine):
    """mla_verify_attend followed by mla_verify_combine on one stream is
    mla_verify_run, bit for bit: without a combine, and through both combine
    kernels (up to 8 split groups per row one wave per row, else lane groups)."""
    import torch
    from mla_absorbed_tree_amd import binding as B
    from mla_absorbed_tree_amd.verify import MlaVerify, device_inputs
    cfg = get_config(name, heads=8 if name.startswith("b1") else 16)
    x = make_inputs(cfg)
    d = device_inputs(x)
    mv = MlaVerify(cfg.batch, cfg.heads, cfg.tree_nodes, cfg.dtype, x.kv_lens, splits)
    groups = mv.info["total_groups"] // cfg.batch
    assert (combine == "none") == (groups == 1) and (combine == "lane groups") == (groups > 8), mv.info
    args = (d["q_nope"], d["q_pe"], d["kv_c"], d["k_pe"], d["kv_indptr"], d["kv_indices"], d["tree_parents"],
            x.scale)
    o1, l1 = mv(*args)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    B.mla_verify_attend(mv.plan, *args, o2, l2, mv.workspace)
    B.mla_verify_combine(mv.plan, o2, l2, mv.workspace)
    torch.cuda.synchronize()
    mv.close()
    log("  %s splits=%d groups=%d (%s)" % (name, splits, groups, combine))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, lse_ref = run_oracle(x)
    compare(o1.cpu().numpy(), l1.cpu().numpy(), o_ref, lse_ref, cfg.dtype)


def test_repeat_runs_are_bitwise_identical():
    cfg = get_config("b1_h64_p4096_t16_bf16")
    x = make_inputs(cfg)
    from mla_absorbed_tree_amd.verify import device_inputs
    d = device_inputs(x)
    a = run_hip(x, 0, device_tensors=d)
    b = run_hip(x, 0, device_tensors=d)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("name,reps", [("b4_h64_p32768_t64_bf16", 24), ("b1_h64_p200000_t32_bf16_s256", 16),
                                       ("b4_h64_p32768_t1to256_ragged_bf16", 8)])
def test_stress_back_to_back_runs_are_bitwise_stable(name, reps):
    """Many runs of one plan enqueued back to back on one stream, with no
    synchronisation between them (each run's workgroups overlap the previous
    run's tail), at full size in the benchmark's launch configuration: every
    run's out and lse equal the first run's bit for bit. The LDS ring, the
    barrier per tile, the weight exchange between paired waves and the split
    groups must not let any data race show through."""
    import torch
    from mla_absorbed_tree_amd.verify import MlaVerify, device_inputs
    cfg = get_config(name)
    x = make_inputs(cfg)
    d = device_inputs(x)
    ragged = x.parents.ndim == 1
    mv = MlaVerify(cfg.batch, cfg.heads, cfg.tree_nodes, cfg.dtype, x.kv_lens, cfg.num_splits,
                   tree_lens=x.tree_lens if ragged else None)
    rows = int(x.tree_indptr[-1])
    outs = [torch.empty((rows, cfg.heads, 512), dtype=torch.float32, device="cuda") for _ in range(2)]
    lses = [torch.empty((rows, cfg.heads), dtype=torch.float32, device="cuda") for _ in range(2)]
    args = (d["q_nope"], d["q_pe"], d["kv_c"], d["k_pe"], d["kv_indptr"], d["kv_indices"], d["tree_parents"],
            x.scale)
    log("  %s: %d runs back to back, plan %s" % (name, reps, mv.info))
    mv(*args, out=outs[0], lse=lses[0])
    mismatches = torch.zeros((), dtype=torch.int64, device="cuda")
    for _ in range(reps - 1):
        mv(*args, out=outs[1], lse=lses[1])
        # compared on the stream, so no run waits for the host
        mismatches += (outs[1] != outs[0]).sum() + (lses[1] != lses[0]).sum()
    torch.cuda.synchronize()
    mv.close()
    assert torch.isfinite(outs[0]).all() and torch.isfinite(lses[0]).all()
    assert int(mismatches) == 0


# --------------------------------------------------------------------------
# tree masks and invalid trees
# --------------------------------------------------------------------------

def test_tree_masks_bit_exact():
    import torch
    from mla_absorbed_tree_amd import binding as B
    rng = np.random.default_rng(30)
    for T in (1, 2, 5, 31, 32, 33, 63, 64):
        for kind in ("uniform", "bounded", "chain"):
            par = np.stack([make_tree_parents(rng, T, kind) for _ in range(3)]).astype(np.int32)
            masks = torch.zeros(3 * T, dtype=torch.int64, device="cuda")
            B.mla_verify_tree_masks(torch.from_numpy(par).cuda(), 3, T, masks)
            got = masks.cpu().numpy().view(np.uint64).reshape(3, T)
            for b in range(3):
                for t, anc in enumerate(tree_ancestors(par[b])):
                    want = 0
                    for u in anc:
                        want |= 1 << u
                    assert int(got[b, t]) == want, (T, kind, b, t)
    # invalid parents: node 2 points forward; it and its descendants get mask 0
    par = np.array([[-1, 0, 3, 0, 2, 1]], dtype=np.int32)
    masks = torch.zeros(6, dtype=torch.int64, device="cuda")
    B.mla_verify_tree_masks(torch.from_numpy(par).cuda(), 1, 6, masks)
    got = masks.cpu().numpy().view(np.uint64)
    assert list(got) == [0b1, 0b11, 0, 0b1001, 0, 0b100011]


def test_invalid_tree_rows_are_nan():
    cfg = get_config("b1_h64_p4096_t16_bf16", batch=2, heads=4, tree_nodes=6, prefix=40, seed=31)
    x = make_inputs(cfg)
    x.parents[1] = [-1, 0, 5, 0, 2, 1]   # node 2 of sequence 1 points forward
    o, lse, _ = run_hip(x, 0)
    bad = {(1, 2), (1, 4)}
    for b in range(2):
        for t in range(6):
            r = b * 6 + t
            assert np.isnan(o[r]).all() == ((b, t) in bad)
            assert np.isnan(lse[r]).all() == ((b, t) in bad)
    good = [(b, t) for b in range(2) for t in range(6) if (b, t) not in bad]
    x.parents[1] = [-1, 0, 0, 0, 2, 1]   # the oracle rejects invalid trees; valid rows match anyway
    o_ref, lse_ref = run_oracle(x, nodes=good)
    rows = node_rows(x, good)
    compare(o[rows], lse[rows], o_ref, lse_ref, "bf16")
