"""GPU test of mla_verify_run_noalloc, the entry point whose workspace is the
library's built-in device buffer (for callers that cannot allocate): two calls
in a row, the second on a smaller problem, each compared with mla_verify_run
(caller-owned workspace) on the same inputs and with the float64 oracle."""
import numpy as np
import pytest

from gpu_util import compare, log, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_absorbed_tree_amd.binding  # noqa: F401  (fails loudly if the library is missing)


def _run_pair(B, cfg, num_splits):
    import torch
    from gen import make_inputs
    from mla_absorbed_tree_amd.verify import device_inputs

    x = make_inputs(cfg)
    d = device_inputs(x)
    dtype = B.MLA_DTYPE_BF16 if cfg.dtype == "bf16" else B.MLA_DTYPE_F32
    plan, ws_bytes = B.mla_verify_plan(cfg.batch, cfg.heads, cfg.tree_nodes, dtype, x.kv_lens, num_splits)
    try:
        info = B.mla_verify_plan_get_info(plan)
        assert ws_bytes <= B.NOALLOC_WORKSPACE_BYTES
        rows = cfg.batch * cfg.tree_nodes
        args = (d["q_nope"], d["q_pe"], d["kv_c"], d["k_pe"], d["kv_indptr"], d["kv_indices"],
                d["tree_parents"], x.scale)
        # NaN-filled outputs: a row the call fails to write cannot pass.
        out_a = torch.full((rows, cfg.heads, 512), float("nan"), device="cuda")
        lse_a = torch.full((rows, cfg.heads), float("nan"), device="cuda")
        out_b = torch.full_like(out_a, float("nan"))
        lse_b = torch.full_like(lse_a, float("nan"))
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        B.mla_verify_run(plan, *args, out_a, lse_a, ws)
        B.mla_verify_run_noalloc(plan, *args, out_b, lse_b)
        torch.cuda.synchronize()
        oa, la = out_a.cpu().numpy(), lse_a.cpu().numpy()
        ob, lb = out_b.cpu().numpy(), lse_b.cpu().numpy()
    finally:
        B.mla_verify_plan_destroy(plan)
    log("  %s splits=%d uses_combine=%d workspace=%d B" % (cfg.name, num_splits, info["uses_combine"], ws_bytes))
    # Same kernels on the same inputs: the two entry points agree bit for bit,
    # and both meet the oracle's tolerance.
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)
    o_ref, lse_ref = run_oracle(x)
    compare(ob.reshape(o_ref.shape), lb.reshape(lse_ref.shape), o_ref, lse_ref, cfg.dtype, "(noalloc)")
    return info


def test_noalloc_matches_run_on_two_calls_in_a_row():
    from gen import get_config
    from mla_absorbed_tree_amd import binding as B

    # First call: 4k prefix, 64 heads, 16 nodes, 8 forced splits (partials and
    # combine in the built-in buffer). Second call: a smaller problem (two
    # sequences, 16 heads, 8 nodes, 3 splits) that reuses the same buffer.
    info1 = _run_pair(B, get_config("b1_h64_p4096_t16_bf16"), 8)
    info2 = _run_pair(B, get_config("b1_h64_p4096_t16_bf16", batch=2, heads=16, tree_nodes=8, prefix=700), 3)
    assert info1["uses_combine"] == 1 and info2["uses_combine"] == 1


def test_noalloc_rejects_a_plan_beyond_the_buffer():
    from mla_absorbed_tree_amd import binding as B

    # fp32 writes one partial per split: about 4 GB here
    plan, ws = B.mla_verify_plan(8, 64, 64, B.MLA_DTYPE_F32, [65536] * 8, num_splits=64)
    try:
        assert ws > B.NOALLOC_WORKSPACE_BYTES
        with pytest.raises(B.MlaVerifyError) as e:
            B.mla_verify_run_noalloc(plan, None, None, None, None, None, None, None, 0.07, None, None)
        assert e.value.status == B.MLA_ERR_WORKSPACE
    finally:
        B.mla_verify_plan_destroy(plan)
