"""KV-cache compaction on the CPU: the oracle against a hand-worked example and
against the verify oracle (compaction must not change any attention result),
plus the C-ABI argument checks (no device work)."""
import json
import os

import numpy as np
import pytest

from gen import get_config, make_inputs
from oracle import kv_compact, verify_attention

HERE = os.path.dirname(os.path.abspath(__file__))


def test_hand_worked_example():
    g = json.load(open(os.path.join(HERE, "golden", "kv_compact_small.json")))
    pool = np.array(g["pool_rows"], dtype=np.float64)
    rows_c, rows_p, new = kv_compact(pool, pool[:, :1], np.array(g["kv_indptr"]),
                                     np.array(g["kv_indices"]), g["dst_base"])
    np.testing.assert_array_equal(rows_c, np.array(g["expected_rows"], dtype=np.float64))
    np.testing.assert_array_equal(rows_p[:, 0], np.array(g["expected_rows"], dtype=np.float64)[:, 0])
    assert list(new) == g["expected_new_indices"]


@pytest.mark.parametrize("seed", [0, 1])
def test_compaction_leaves_attention_unchanged(seed):
    """Attention over the compacted pool (contiguous runs, rewritten page table)
    equals attention over the scattered pool, bit for bit."""
    cfg = get_config("b8_h64_paged600k_t16_bf16", batch=3, heads=2, prefix_range=(5, 40),
                     pool_slots=400, dtype="f32", seed=50 + seed)
    x = make_inputs(cfg)
    dst_base = 37
    rows_c, rows_p, new = kv_compact(x.kv_c, x.k_pe, x.kv_indptr, x.kv_indices, dst_base)
    n = len(new)
    pool_c = np.full((dst_base + n, x.kv_c.shape[1]), np.nan, dtype=x.kv_c.dtype)
    pool_p = np.full((dst_base + n, x.k_pe.shape[1]), np.nan, dtype=x.k_pe.dtype)
    pool_c[new] = rows_c
    pool_p[new] = rows_p
    o0, l0 = verify_attention(x.q_nope, x.q_pe, x.kv_c, x.k_pe, x.kv_indptr, x.kv_indices, x.parents, x.scale)
    o1, l1 = verify_attention(x.q_nope, x.q_pe, pool_c, pool_p, x.kv_indptr, new, x.parents, x.scale)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)


def test_runs_are_contiguous_and_disjoint():
    rng = np.random.default_rng(3)
    lens = np.array([5, 0, 9, 1])
    indptr = np.concatenate([[0], np.cumsum(lens)])
    idx = rng.permutation(100)[:indptr[-1]].astype(np.int32)
    pool = rng.standard_normal((100, 4))
    _, _, new = kv_compact(pool, pool, indptr, idx, dst_base=11)
    for b in range(len(lens)):
        run = new[indptr[b]:indptr[b + 1]]
        assert list(run) == list(range(11 + indptr[b], 11 + indptr[b + 1]))
    assert len(set(new.tolist())) == len(new)


@pytest.fixture(scope="module")
def B():
    from mla_absorbed_tree_amd import binding
    return binding


def test_capi_argument_checks(B):
    fake = 1 << 20  # never dereferenced: every call below fails validation first
    good = dict(dtype=B.MLA_DTYPE_BF16, batch=2, total_tokens=10, kv_c=fake, k_pe=fake,
                kv_c_row_stride=512, k_pe_row_stride=64, kv_indptr=fake, kv_indices=fake,
                dst_kv_c=fake, dst_k_pe=fake, dst_kv_c_row_stride=512, dst_k_pe_row_stride=64,
                dst_base=0, new_kv_indices=fake + 4096, stream=0)
    bad_cases = [dict(dtype=7), dict(batch=0), dict(batch=B.MLA_VERIFY_MAX_BATCH + 1),
                 dict(total_tokens=-1), dict(dst_base=-1), dict(dst_base=2**31 - 5),
                 dict(kv_c_row_stride=500), dict(k_pe_row_stride=60), dict(dst_kv_c_row_stride=516),
                 dict(kv_c=0), dict(new_kv_indices=0), dict(kv_c=fake + 8),
                 dict(dst_k_pe=fake + 4), dict(new_kv_indices=fake)]
    for over in bad_cases:
        with pytest.raises(B.MlaVerifyError) as e:
            B.mla_kv_compact(**{**good, **over})
        assert e.value.status == B.MLA_ERR_INVALID_ARG, over
        assert B.mla_verify_last_error() != ""
    B.mla_kv_compact(**{**good, "total_tokens": 0})  # nothing to copy: no launch, no error
