"""Pins of the oracle's packed ("ragged") trees and of trees above 64 nodes.

Every node of the draft tree is a query of the verify step, and the pages put
no limit on how many there are ("Ground Truth in Silicon" page, "Input
Knowledge Required", item 3). Each test ties the oracle to
something other than itself: separate single-sequence runs on hand-sliced
inputs, the scalar brute force (its own visibility walk), torch SDPA in float64
with a causal mask, a boolean transitive closure, and a planted dominant key.
"""
import numpy as np
import pytest

from gen import make_tree_parents
from oracle import brute_force_verify, tree_mask_words, verify_attention
from test_oracle_pins import closure_mask, sdpa_reference


def ragged_inputs(P_list, T_list, H, Dl, Dr, seed, kind="uniform", q_std=0.7, paged=True):
    rng = np.random.default_rng(seed)
    B = len(P_list)
    parents = np.concatenate([make_tree_parents(rng, T, kind) for T in T_list] or
                             [np.zeros(0, np.int32)]).astype(np.int32)
    tree_indptr = np.concatenate([[0], np.cumsum(T_list)]).astype(np.int32)
    N = np.asarray(P_list) + np.asarray(T_list)
    rows = int(tree_indptr[-1])
    qn = rng.standard_normal((rows, H, Dl)) * q_std
    qp = rng.standard_normal((rows, H, Dr)) * q_std
    total = int(N.sum())
    slots = total + (5 if paged else 0)
    kv_c = rng.standard_normal((slots, Dl))
    k_pe = rng.standard_normal((slots, Dr))
    indices = (rng.permutation(slots)[:total] if paged else np.arange(total)).astype(np.int32)
    indptr = np.concatenate([[0], np.cumsum(N)]).astype(np.int32)
    assert len(indptr) == B + 1
    return dict(q_nope=qn, q_pe=qp, kv_c=kv_c, k_pe=k_pe, kv_indptr=indptr, kv_indices=indices,
                parents=parents, tree_indptr=tree_indptr)


def test_ragged_batch_equals_separate_sequences():
    """Packed rows of sequence b == a B=1 run on that sequence's hand-sliced data."""
    P_list, T_list = [7, 0, 30, 12], [5, 3, 0, 70]
    x = ragged_inputs(P_list, T_list, H=3, Dl=16, Dr=8, seed=11)
    o, lse = verify_attention(x["q_nope"], x["q_pe"], x["kv_c"], x["k_pe"], x["kv_indptr"],
                              x["kv_indices"], x["parents"], 0.4, tree_indptr=x["tree_indptr"])
    assert o.shape[0] == sum(T_list)
    row = 0
    for b, (P, T) in enumerate(zip(P_list, T_list)):
        if T == 0:
            continue
        k0, k1 = x["kv_indptr"][b], x["kv_indptr"][b + 1]
        slots = x["kv_indices"][k0:k1]
        ob, lb = verify_attention(x["q_nope"][row:row + T], x["q_pe"][row:row + T],
                                  x["kv_c"][slots], x["k_pe"][slots],
                                  np.array([0, P + T]), np.arange(P + T),
                                  x["parents"][row:row + T][None], 0.4)
        np.testing.assert_array_equal(o[row:row + T], ob)
        np.testing.assert_array_equal(lse[row:row + T], lb)
        row += T


@pytest.mark.parametrize("P_list,T_list,seed", [
    ([3, 0, 5], [4, 2, 0], 0), ([2, 4], [70, 1], 1), ([0], [66], 2)])
def test_ragged_brute_force_agrees(P_list, T_list, seed):
    x = ragged_inputs(P_list, T_list, H=2, Dl=6, Dr=3, seed=seed)
    args = (x["q_nope"], x["q_pe"], x["kv_c"], x["k_pe"], x["kv_indptr"], x["kv_indices"],
            x["parents"], 0.45)
    o, lse = verify_attention(*args, tree_indptr=x["tree_indptr"])
    ob, lb = brute_force_verify(*args, tree_indptr=x["tree_indptr"])
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("P,T", [(3, 100), (0, 65), (40, 256)])
def test_long_chain_equals_causal_attention(P, T):
    """A chain of more than 64 nodes is causal attention over P + T keys."""
    x = ragged_inputs([P], [T], H=2, Dl=8, Dr=4, seed=T, kind="chain")
    o, lse = verify_attention(x["q_nope"], x["q_pe"], x["kv_c"], x["k_pe"], x["kv_indptr"],
                              x["kv_indices"], x["parents"], 0.3, tree_indptr=x["tree_indptr"])
    slots = x["kv_indices"]
    kc, kp = x["kv_c"][slots], x["k_pe"][slots]
    mask = np.arange(P + T)[None, :] <= (P + np.arange(T))[:, None]
    ref = sdpa_reference(x["q_nope"], x["q_pe"], kc, kp, mask, 0.3)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("T,kind,seed", [(200, "uniform", 0), (256, "bounded", 1), (130, "chain", 2),
                                         (64, "uniform", 3), (65, "uniform", 4)])
def test_mask_words_match_closure(T, kind, seed):
    rng = np.random.default_rng(seed)
    parents = make_tree_parents(rng, T, kind, max_depth=40, max_branch=8)
    words = (T + 63) // 64
    m = tree_mask_words(parents, words)
    # Bit u of a row is byte u//8, bit u%8 of its little-endian bytes.
    bits = np.unpackbits(m.astype("<u8").view(np.uint8).reshape(T, -1), axis=1, bitorder="little")
    np.testing.assert_array_equal(bits[:, :T].astype(bool), closure_mask(parents))
    assert not bits[:, T:].any()


def test_mask_words_zero_below_invalid_parent():
    parents = np.array([-1, 0, 1, 7, 3, 0, 5] + [6] * 70, dtype=np.int32)  # node 3 points forward
    m = tree_mask_words(parents, 2)
    bad = {3, 4}  # node 3 and its descendant 4
    for t in range(len(parents)):
        assert (m[t] == 0).all() == (t in bad), t
    assert m[76, 1] == np.uint64(1) << np.uint64(76 - 64) and m[76, 0] == np.uint64(0b1100001)  # 76 -> 6 -> 5 -> 0


def test_planted_key_past_first_mask_word():
    """Tail key u >= 64 made dominant: exactly the rows that have u as an
    ancestor-or-self output (about) that key's kv_c; the others are unchanged."""
    T, P, H, Dl, Dr = 150, 4, 2, 8, 4
    x = ragged_inputs([P], [T], H=H, Dl=Dl, Dr=Dr, seed=5, q_std=0.2, paged=False)
    reach = closure_mask(x["parents"])
    u = 64 + int(np.argmax(reach[:, 64:].sum(axis=0)))  # the node past 64 with most descendants
    assert reach[:, u].sum() > 1
    slot = P + u
    q_dir = np.concatenate([x["q_nope"].mean(axis=(0, 1)), x["q_pe"].mean(axis=(0, 1))])
    x["q_nope"][:] = q_dir[:Dl]
    x["q_pe"][:] = q_dir[Dl:]
    base = verify_attention(x["q_nope"], x["q_pe"], x["kv_c"], x["k_pe"], x["kv_indptr"],
                            x["kv_indices"], x["parents"], 1.0, tree_indptr=x["tree_indptr"])[0]
    spike = 400.0 * q_dir / np.dot(q_dir, q_dir)
    x["kv_c"][slot] = spike[:Dl]
    x["k_pe"][slot] = spike[Dl:]
    o = verify_attention(x["q_nope"], x["q_pe"], x["kv_c"], x["k_pe"], x["kv_indptr"],
                         x["kv_indices"], x["parents"], 1.0, tree_indptr=x["tree_indptr"])[0]
    for t in range(T):
        if reach[t, u]:
            np.testing.assert_allclose(o[t], np.broadcast_to(spike[:Dl], (H, Dl)), rtol=0, atol=1e-6)
        else:
            np.testing.assert_array_equal(o[t], base[t])
