"""GPU parity of the KV-cache compaction kernel (mla_kv_compact) against the
oracle: the copy and the rewritten page table are compared bit for bit, and
attention over the compacted pool must equal attention over the scattered one
bit for bit (same kernel, same values, same order)."""
import numpy as np
import pytest
import torch

from gen import get_config, make_inputs
from gpu_util import log
from oracle import kv_compact

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mla_absorbed_tree_amd import binding
    return binding


def _dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt)


def _compact(B, x, dtype, dst_base, src_strides=(512, 64), dst_strides=(512, 64), total=None,
             kv_c=None, k_pe=None):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    code = B.MLA_DTYPE_BF16 if dtype == "bf16" else B.MLA_DTYPE_F32
    n = int(x.kv_indptr[-1])
    if kv_c is None:
        kv_c, k_pe = _dev(x.kv_c, dt), _dev(x.k_pe, dt)
    indptr = _dev(x.kv_indptr, torch.int32)
    idx = _dev(x.kv_indices, torch.int32)
    rows = dst_base + n + 8
    if dst_strides == (576, 576):
        dpool = torch.full((rows, 576), float("nan"), dtype=dt, device="cuda")
        dc, dp = dpool, dpool[:, 512:]
    else:
        dc = torch.full((rows, 512), float("nan"), dtype=dt, device="cuda")
        dp = torch.full((rows, 64), float("nan"), dtype=dt, device="cuda")
    new = torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda")
    B.mla_kv_compact(code, x.cfg.batch, n if total is None else total, kv_c, k_pe, src_strides[0],
                     src_strides[1], indptr, idx, dc, dp, dst_strides[0], dst_strides[1], dst_base, new)
    torch.cuda.synchronize()
    return dc, dp, new


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bit_exact_against_oracle(B, dtype):
    cfg = get_config("b8_h64_paged600k_t16_bf16", batch=6, heads=4, prefix_range=(0, 700),
                     pool_slots=6000, dtype=dtype, seed=60)
    x = make_inputs(cfg, poison_unused=True)
    dst_base = 1234
    dc, dp, new = _compact(B, x, dtype, dst_base)
    rc, rp, rn = kv_compact(x.kv_c, x.k_pe, x.kv_indptr, x.kv_indices, dst_base)
    n = len(rn)
    got_c = dc[dst_base:dst_base + n].float().cpu().numpy()
    got_p = dp[dst_base:dst_base + n].float().cpu().numpy()
    np.testing.assert_array_equal(got_c, rc)
    np.testing.assert_array_equal(got_p, rp)
    np.testing.assert_array_equal(new.cpu().numpy()[:n], rn)
    # nothing outside the destination run is touched
    assert torch.isnan(dc[:dst_base]).all() and torch.isnan(dc[dst_base + n:]).all()


def test_interleaved_576_wide_pools_and_empty_sequences(B):
    cfg = get_config("b8_h64_paged600k_t16_bf16", batch=4, heads=4, prefix_range=(0, 300),
                     pool_slots=3000, seed=61)
    x = make_inputs(cfg)
    # one sequence with no tokens at all (compaction does not need T of them)
    lens = np.diff(x.kv_indptr).astype(np.int64)
    lens[2] = 0
    x.kv_indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x.kv_indices = x.kv_indices[:x.kv_indptr[-1]]
    src = torch.cat([_dev(x.kv_c, torch.bfloat16), _dev(x.k_pe, torch.bfloat16)], dim=1).contiguous()
    dc, dp, new = _compact(B, x, "bf16", 5, src_strides=(576, 576), dst_strides=(576, 576),
                           kv_c=src, k_pe=src[:, 512:])
    rc, rp, rn = kv_compact(x.kv_c, x.k_pe, x.kv_indptr, x.kv_indices, 5)
    n = len(rn)
    np.testing.assert_array_equal(dc[5:5 + n, :512].float().cpu().numpy(), rc)
    np.testing.assert_array_equal(dp[5:5 + n].float().cpu().numpy(), rp)
    np.testing.assert_array_equal(new.cpu().numpy()[:n], rn)


def test_device_length_bounds_the_copy(B):
    """total_tokens above the device kv_indptr[batch]: only the device count is copied."""
    cfg = get_config("b8_h64_paged600k_t16_bf16", batch=2, heads=4, prefix_range=(50, 90),
                     pool_slots=1000, seed=62)
    x = make_inputs(cfg)
    n = int(x.kv_indptr[-1])
    dc, dp, new = _compact(B, x, "bf16", 0, total=n + 5)
    rc, _, rn = kv_compact(x.kv_c, x.k_pe, x.kv_indptr, x.kv_indices, 0)
    np.testing.assert_array_equal(dc[:n].float().cpu().numpy(), rc)
    assert torch.isnan(dc[n:]).all()
    assert (new[:n].cpu().numpy() == rn).all()


def test_full_pool_compaction_then_attention_is_unchanged(B):
    """The 8-sequence paged workload at full size (page_size=1 pool of 600k
    slots): compaction matches the oracle bit for bit, and verify attention over
    the compacted pool equals attention over the scattered pool bit for bit."""
    from mla_absorbed_tree_amd.verify import MlaVerify, device_inputs
    cfg = get_config("b8_h64_paged600k_t16_bf16")
    x = make_inputs(cfg)
    log("compaction of %d tokens" % int(x.kv_indptr[-1]))
    d = device_inputs(x)
    n = int(x.kv_indptr[-1])
    dc = torch.empty((n, 512), dtype=torch.bfloat16, device="cuda")
    dp = torch.empty((n, 64), dtype=torch.bfloat16, device="cuda")
    new = torch.empty(n, dtype=torch.int32, device="cuda")
    B.mla_kv_compact(B.MLA_DTYPE_BF16, cfg.batch, n, d["kv_c"], d["k_pe"], 512, 64, d["kv_indptr"],
                     d["kv_indices"], dc, dp, 512, 64, 0, new)
    torch.cuda.synchronize()
    rc, rp, rn = kv_compact(x.kv_c, x.k_pe, x.kv_indptr, x.kv_indices, 0)
    np.testing.assert_array_equal(dc.float().cpu().numpy(), rc)
    np.testing.assert_array_equal(dp.float().cpu().numpy(), rp)
    np.testing.assert_array_equal(new.cpu().numpy(), rn)
    del rc, rp
    mv = MlaVerify(cfg.batch, cfg.heads, cfg.tree_nodes, cfg.dtype, x.kv_lens, 0)
    o0, l0 = mv(d["q_nope"], d["q_pe"], d["kv_c"], d["k_pe"], d["kv_indptr"], d["kv_indices"],
                d["tree_parents"], x.scale)
    o1, l1 = mv(d["q_nope"], d["q_pe"], dc, dp, d["kv_indptr"], new, d["tree_parents"], x.scale)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    mv.close()
