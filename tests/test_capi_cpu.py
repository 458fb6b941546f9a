"""Host-side checks of libmlaverify: it loads, exports what the header declares,
and its planner validates problems and sizes workspaces (no device work)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


@pytest.fixture(scope="module")
def B():
    lib = os.path.join(ROOT, "mla_absorbed_tree_amd", "libmlaverify.so")
    if not os.path.exists(lib):
        from mla_absorbed_tree_amd.build_lib import build
        build()
    from mla_absorbed_tree_amd import binding
    return binding


def declared_functions():
    names = set()
    for header in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
        names |= set(re.findall(r"\b(mla_\w+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_binding_symbols(B):
    assert declared_functions() == sorted(B.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(B):
    lib = ctypes.CDLL(B.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(B):
    assert B.mla_verify_status_string(0) == "MLA_OK"
    assert B.mla_verify_status_string(-3) == "MLA_ERR_WORKSPACE"


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), -1), (dict(batch=65537), -1), (dict(num_heads=0), -1),
    (dict(tree_nodes=0), -1), (dict(tree_nodes=257), -2), (dict(d_latent=256), -2),
    (dict(d_rope=32), -2), (dict(dtype=7), -1), (dict(kv_c_row_stride=500), -1),
    (dict(kv_c_row_stride=516), -1), (dict(k_pe_row_stride=60), -1), (dict(num_splits=-1), -1),
    (dict(kv_len_host=[10, 3]), -1), (dict(tree_len_host=[3, 9]), -1),
    (dict(tree_len_host=[-1, 2]), -1), (dict(tree_len_host=[8, 8], kv_len_host=[100, 7]), -1)])
def test_plan_rejects_bad_problems(B, kw, status):
    args = dict(batch=2, num_heads=4, tree_nodes=8, dtype=1, kv_len_host=[100, 50])
    args.update(kw)
    if "batch" in kw and kw["batch"] > 0:
        args["kv_len_host"] = [100] * kw["batch"]
    with pytest.raises(B.MlaVerifyError) as e:
        B.mla_verify_plan(**args)
    assert e.value.status == status
    assert B.mla_verify_last_error() != ""


def test_forced_and_auto_split_schedules(B):
    p, ws = B.mla_verify_plan(1, 64, 32, 1, [200032], num_splits=256)
    info = B.mla_verify_plan_get_info(p)
    assert info["total_splits"] == 256 and info["uses_combine"] == 1
    rows = 32 * 64
    # 256 splits x 16 row blocks: each workgroup runs 16 consecutive splits,
    # one workgroup per compute unit
    assert info["splits_per_workgroup"] == 16
    assert info["grid_blocks"] == 256 // 16 * (rows // info["rows_per_block"])
    # one partial per workgroup's group of 16 splits (their merge is a sum
    # in the accumulators): per (group, row) an fp32 (m, l, s0, s1) record
    # and the output in scaled fp16
    assert 16 * rows * (4 * 4 + 512 * 2) <= ws < 17 * rows * (4 * 4 + 512 * 2)
    B.mla_verify_plan_destroy(p)
    # groups that do not divide the split counts: 64, 32 and 48 splits (the
    # last two capped at the key tiles) of 8 row blocks each; the estimate
    # takes 6 splits per workgroup, ceil(64/6) + ceil(32/6) + ceil(48/6) =
    # 11 + 6 + 8 = 25 groups (200 workgroups, one round), padded to 4 per XCD
    p, _ = B.mla_verify_plan(3, 64, 16, 1, [3016, 1016, 1516], num_splits=64)
    info = B.mla_verify_plan_get_info(p)
    assert info["total_splits"] == 64 + 32 + 48 and info["splits_per_workgroup"] == 6
    assert info["total_groups"] == 25 and info["grid_blocks"] == 4 * 8 * 8
    B.mla_verify_plan_destroy(p)
    # forced splits on the ragged batch (T_b = 172, 207, 6, 207 at 64 heads:
    # 86, 104, 3 and 104 row blocks of 32,800-odd keys). A rule that aimed at
    # one workgroup per compute unit merged every forced count into one group
    # per sequence there: 4 groups for 8 XCDs, 104 row blocks queued on one
    # XCD's 32 units, 6.3 ms against 2.3 ms measured. The estimate keeps every
    # XCD busy: one split per group up to 8 per sequence, then 32 groups.
    tl = [172, 207, 6, 207]
    for ns, groups in ((2, 8), (4, 16), (8, 32), (16, 32), (64, 32)):
        p, _ = B.mla_verify_plan(4, 64, 256, 1, [32768 + t for t in tl], num_splits=ns, tree_len_host=tl)
        info = B.mla_verify_plan_get_info(p)
        assert info["total_splits"] == 4 * ns and info["total_groups"] == groups, (ns, info)
        B.mla_verify_plan_destroy(p)
    # fp32 problems run one split per workgroup
    p, _ = B.mla_verify_plan(1, 64, 32, 0, [200032], num_splits=256)
    assert B.mla_verify_plan_get_info(p)["splits_per_workgroup"] == 1
    B.mla_verify_plan_destroy(p)
    # more splits than key tiles are capped at the tile count
    p, _ = B.mla_verify_plan(2, 4, 4, 1, [40, 100], num_splits=50)
    info = B.mla_verify_plan_get_info(p)
    assert info["total_splits"] == 2 + 4
    B.mla_verify_plan_destroy(p)
    # a problem with many row blocks needs no split: no combine, no partials
    p, ws = B.mla_verify_plan(16, 64, 64, 1, [5000] * 16)
    info = B.mla_verify_plan_get_info(p)
    assert info["total_splits"] == 16 and info["uses_combine"] == 0 and ws == 256
    B.mla_verify_plan_destroy(p)
    # ... but at least one chunk per XCD: 4 long sequences get 2 splits each
    p, ws = B.mla_verify_plan(4, 64, 64, 1, [32832] * 4)
    info = B.mla_verify_plan_get_info(p)
    assert info["total_splits"] == 8 and info["uses_combine"] == 1
    B.mla_verify_plan_destroy(p)
    # fp32 uses 32-row blocks
    p, _ = B.mla_verify_plan(1, 16, 8, 0, [264], num_splits=1)
    assert B.mla_verify_plan_get_info(p)["rows_per_block"] == 32
    B.mla_verify_plan_destroy(p)


def test_run_argument_checks_happen_before_any_launch(B):
    p, ws = B.mla_verify_plan(1, 64, 16, 1, [4112], num_splits=4)
    fake = 1 << 20  # never dereferenced: every call below fails validation first
    args = [fake] * 7
    with pytest.raises(B.MlaVerifyError) as e:
        B.mla_verify_run(p, *args, 0.1, fake, fake, fake, ws - 1, stream=0)
    assert e.value.status == B.MLA_ERR_WORKSPACE
    with pytest.raises(B.MlaVerifyError) as e:
        B.mla_verify_run(p, *args, 0.1, fake, fake, fake + 64, ws, stream=0)
    assert e.value.status == B.MLA_ERR_WORKSPACE   # misaligned workspace
    with pytest.raises(B.MlaVerifyError) as e:
        B.mla_verify_run(p, fake, 0, *args[2:], 0.1, fake, fake, fake, ws, stream=0)
    assert e.value.status == B.MLA_ERR_INVALID_ARG
    with pytest.raises(B.MlaVerifyError) as e:
        B.mla_verify_run(p, fake + 4, *args[1:], 0.1, fake, fake, fake, ws, stream=0)
    assert e.value.status == B.MLA_ERR_INVALID_ARG  # misaligned q_nope
    with pytest.raises(B.MlaVerifyError) as e:
        B.mla_verify_run(p, *args, float("nan"), fake, fake, fake, ws, stream=0)
    assert e.value.status == B.MLA_ERR_INVALID_ARG
    for bad in (0.0, -0.5, float("inf"), 2.5e38):  # the last overflows scale * log2(e)
        with pytest.raises(B.MlaVerifyError) as e:
            B.mla_verify_run(p, *args, bad, fake, fake, fake, ws, stream=0)
        assert e.value.status == B.MLA_ERR_INVALID_ARG
    with pytest.raises(B.MlaVerifyError) as e:
        B.mla_verify_tree_masks(fake, 1, 257, fake, stream=0)
    assert e.value.status == B.MLA_ERR_INVALID_ARG
    B.mla_verify_plan_destroy(p)


def test_ragged_tree_plans(B):
    # Row blocks are counted for the largest tree (200 nodes x 8 heads = 13
    # blocks of 128 rows); the sequence without nodes gets no split, and
    # splits are sized by the work each sequence really has.
    p, ws = B.mla_verify_plan(3, 8, 256, 1, [5000, 300, 9000], tree_len_host=[200, 0, 1])
    info = B.mla_verify_plan_get_info(p)
    assert info["rows_per_block"] == 128
    assert info["grid_blocks"] % 13 == 0
    # 157 and 282 tiles, one chunk length for both (10 tiles: 16 and 29
    # splits), none for the empty tree.
    assert info["total_splits"] == 16 + 29 and info["uses_combine"] == 1
    B.mla_verify_plan_destroy(p)
    # every tree empty: a valid plan with nothing to launch
    p, ws = B.mla_verify_plan(2, 64, 16, 1, [100, 100], tree_len_host=[0, 0])
    info = B.mla_verify_plan_get_info(p)
    assert info["grid_blocks"] == 0 and info["total_splits"] == 0 and info["uses_combine"] == 0
    B.mla_verify_plan_destroy(p)
    # equal tree sizes given explicitly plan exactly like tree_len_host = NULL
    for kw in (dict(), dict(num_splits=256)):
        a, wa = B.mla_verify_plan(4, 64, 64, 1, [32832] * 4, **kw)
        b, wb = B.mla_verify_plan(4, 64, 64, 1, [32832] * 4, tree_len_host=[64] * 4, **kw)
        assert B.mla_verify_plan_get_info(a) == B.mla_verify_plan_get_info(b) and wa == wb
        B.mla_verify_plan_destroy(a)
        B.mla_verify_plan_destroy(b)


def test_planning_large_batches_is_fast(B):
    """The automatic split search stays cheap for big batches of long sequences."""
    import time
    for b, h, t, n in ((256, 64, 64, 200000), (256, 1, 1, 200000), (1, 64, 256, 200256),
                       (B.MLA_VERIFY_MAX_BATCH, 8, 4, 40000)):
        t0 = time.perf_counter()
        p, _ = B.mla_verify_plan(b, h, t, 1, [n] * b)
        assert time.perf_counter() - t0 < 0.5, (b, h, t, n)
        B.mla_verify_plan_destroy(p)


def test_plans_of_the_named_workloads(B):
    """The planner's choices for the measured workloads (a change here changes
    what the benchmark measures, so it should be deliberate)."""
    from gen import get_config
    want = {"tiny_f32_b1_h16_p256_t8": (2, 32, 1), "b1_h64_p4096_t16_bf16": (17, 192, 1),
            "b4_h64_p32768_t64_bf16": (8, 256, 1), "b1_h64_p200000_t32_bf16_s256": (256, 256, 16),
            "b8_h64_paged600k_t16_bf16": (64, 512, 1), "b4_h64_p32768_t1to256_ragged_bf16": (32, 3328, 1)}
    for name, (splits, grid, group) in want.items():
        cfg = get_config(name)
        rng = np.random.default_rng(cfg.seed)  # only the lengths and tree sizes are needed
        P = (rng.integers(*cfg.prefix_range, size=cfg.batch, endpoint=True) if cfg.prefix_range
             else np.full(cfg.batch, cfg.prefix))
        Tb = rng.integers(*cfg.tree_range, size=cfg.batch, endpoint=True) if cfg.tree_range else None
        kv = P + (Tb if Tb is not None else cfg.tree_nodes)
        p, _ = B.mla_verify_plan(cfg.batch, cfg.heads, cfg.tree_nodes, 1 if cfg.dtype == "bf16" else 0, kv,
                                 cfg.num_splits, tree_len_host=Tb)
        info = B.mla_verify_plan_get_info(p)
        B.mla_verify_plan_destroy(p)
        assert (info["total_splits"], info["grid_blocks"], info["splits_per_workgroup"]) == (splits, grid, group), name
        # A workgroup merges `group` consecutive splits into one partial:
        # groups per sequence = ceil(S_b / group). With equal splits per
        # sequence (every workload here but the paged and ragged ones, which
        # run one split per group), partial_rows = sum of G_b * T_b * H over
        # the sequences with more than one group.
        if group == 1:
            assert info["total_groups"] == info["total_splits"], name
        if info["total_splits"] % cfg.batch == 0 and info["max_splits"] * cfg.batch == info["total_splits"]:
            g = -(-info["max_splits"] // group)
            assert info["total_groups"] == g * cfg.batch, name
            T = Tb if Tb is not None else np.full(cfg.batch, cfg.tree_nodes)
            assert info["partial_rows"] == (g * int(np.sum(T)) * cfg.heads if g > 1 else 0), name
            assert info["uses_combine"] == int(g > 1), name


def test_large_batch_needs_staged_tables(B):
    """Above MLA_VERIFY_ARG_TABLE_BATCH sequences a plan's tables go to device
    memory: the plan reports their size, runs fail until they are staged, and
    staging checks the buffer (all before any device work)."""
    p, ws = B.mla_verify_plan(1000, 4, 8, 1, [100] * 1000)
    info = B.mla_verify_plan_get_info(p)
    assert info["table_bytes"] == 12 * 1001
    fake = 1 << 20  # never dereferenced: the calls fail validation first
    with pytest.raises(B.MlaVerifyError) as e:
        B.mla_verify_run(p, fake, fake, fake, fake, fake, fake, fake, 0.1, fake, fake, 1 << 21, ws, stream=0)
    assert e.value.status == B.MLA_ERR_INVALID_ARG and "mla_verify_plan_stage_tables" in str(e.value)
    with pytest.raises(B.MlaVerifyError):
        B.mla_verify_plan_stage_tables(p, fake, info["table_bytes"] - 4, stream=0)
    with pytest.raises(B.MlaVerifyError):
        B.mla_verify_plan_stage_tables(p, fake + 2, info["table_bytes"], stream=0)
    B.mla_verify_plan_destroy(p)
    # at the argument-table bound nothing is staged and staging is a no-op
    p, _ = B.mla_verify_plan(B.MLA_VERIFY_ARG_TABLE_BATCH, 4, 8, 1, [100] * B.MLA_VERIFY_ARG_TABLE_BATCH)
    assert B.mla_verify_plan_get_info(p)["table_bytes"] == 0
    B.mla_verify_plan_stage_tables(p, None, 0, stream=0)
    B.mla_verify_plan_destroy(p)


def test_varlen_run_requires_tree_indptr(B):
    p, ws = B.mla_verify_plan(2, 4, 8, 1, [100, 50], tree_len_host=[8, 3])
    fake = 1 << 20  # never dereferenced: the call fails validation first
    with pytest.raises(B.MlaVerifyError) as e:
        B.mla_verify_run_varlen(p, fake, fake, fake, fake, fake, fake, 0, fake, 0.1, fake, fake, fake, ws,
                                stream=0)
    assert e.value.status == B.MLA_ERR_INVALID_ARG
    B.mla_verify_plan_destroy(p)


def test_noalloc_rejects_plans_beyond_its_buffer(B):
    """mla_verify_run_noalloc checks the plan's workspace against its built-in
    buffer before any device work (so this runs without a GPU)."""
    # fp32, 8 sequences x 64 nodes x 64 heads, 64 forced splits of 64k keys:
    # the fp32 kernel writes one partial per split, about 4 GB, far beyond the
    # 64 MiB buffer. (The bf16 kernel merges a workgroup's splits in its
    # accumulators, so the same bf16 plan needs no partials at all.)
    plan, ws = B.mla_verify_plan(8, 64, 64, B.MLA_DTYPE_F32, [65536] * 8, num_splits=64)
    try:
        assert ws > B.NOALLOC_WORKSPACE_BYTES
        with pytest.raises(B.MlaVerifyError) as e:
            B.mla_verify_run_noalloc(plan, None, None, None, None, None, None, None, 0.07, None, None,
                                     stream=0)
        assert e.value.status == B.MLA_ERR_WORKSPACE
        assert "built-in buffer" in str(e.value)
    finally:
        B.mla_verify_plan_destroy(plan)
