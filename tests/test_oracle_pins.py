"""Pins of the float64 oracle against what the pages and mathematics fix.

Each test ties the oracle to something other than itself: a library routine
(torch scaled_dot_product_attention in float64 on the CPU), an algebraic
identity (absorbed == un-absorbed MLA), closed forms, invariants, a scalar brute
force and a hand-worked example.
"""
import json
import os

import numpy as np
import pytest
import torch

from gen import get_config, make_inputs, make_tree_parents
from oracle import (brute_force_verify, chunk_partial, merge_partials, node_scores,
                    tree_ancestors, verify_attention)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers that are independent of the oracle's own mask construction
# ---------------------------------------------------------------------------

def closure_mask(parents_row):
    """reach[t, u] = u is t or an ancestor of t, by boolean transitive closure."""
    T = len(parents_row)
    adj = np.zeros((T, T), dtype=bool)
    for t, p in enumerate(parents_row):
        if p >= 0:
            adj[t, p] = True
    reach = np.eye(T, dtype=bool)
    for _ in range(T):
        reach = reach | ((reach.astype(np.int64) @ adj.astype(np.int64)) > 0)
    return reach


def small_inputs(B, H, P, T, Dl, Dr, seed, kind="uniform", paged=False, q_std=0.7):
    rng = np.random.default_rng(seed)
    parents = np.stack([make_tree_parents(rng, T, kind) for _ in range(B)]).astype(np.int32)
    N = P + T
    qn = rng.standard_normal((B * T, H, Dl))
    qp = rng.standard_normal((B * T, H, Dr))
    qn *= q_std
    qp *= q_std
    total = B * N
    slots = total + (7 if paged else 0)
    kv_c = rng.standard_normal((slots, Dl))
    k_pe = rng.standard_normal((slots, Dr))
    indices = (rng.permutation(slots)[:total] if paged else np.arange(total)).astype(np.int32)
    indptr = (np.arange(B + 1) * N).astype(np.int32)
    return dict(q_nope=qn, q_pe=qp, kv_c=kv_c, k_pe=k_pe, kv_indptr=indptr,
                kv_indices=indices, parents=parents)


def sdpa_reference(qn, qp, kc, kp, mask, scale):
    """torch SDPA (float64, CPU) over keys [kc | kp] and values kc; one sequence.

    qn [T, H, Dl], qp [T, H, Dr], kc [N, Dl], kp [N, Dr], mask [T, N] bool.
    Returns [T, H, Dl].
    """
    q = torch.from_numpy(np.concatenate([qn, qp], axis=-1)).permute(1, 0, 2)  # H T Dk
    k = torch.from_numpy(np.concatenate([kc, kp], axis=-1))[None].expand(q.shape[0], -1, -1)
    v = torch.from_numpy(kc)[None].expand(q.shape[0], -1, -1)
    m = torch.from_numpy(mask)[None].expand(q.shape[0], -1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(
        q.contiguous(), k.contiguous(), v.contiguous(), attn_mask=m.contiguous(), scale=scale)
    return out.permute(1, 0, 2).numpy()


# ---------------------------------------------------------------------------
# 1. chain tree == causal attention (mask semantics incl. self-visibility)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B,H,P,T,Dl,Dr,seed", [
    (1, 4, 9, 5, 16, 8, 0), (2, 3, 1, 7, 8, 4, 1), (1, 2, 0, 4, 8, 4, 2), (3, 5, 20, 3, 32, 16, 3)])
def test_chain_tree_equals_causal_attention(B, H, P, T, Dl, Dr, seed):
    x = small_inputs(B, H, P, T, Dl, Dr, seed, kind="chain", paged=True)
    scale = 0.3
    o, _ = verify_attention(**x, scale=scale)
    N = P + T
    for b in range(B):
        slots = x["kv_indices"][b * N:(b + 1) * N]
        causal = np.arange(N)[None, :] <= (P + np.arange(T))[:, None]
        ref = sdpa_reference(x["q_nope"][b * T:(b + 1) * T], x["q_pe"][b * T:(b + 1) * T],
                             x["kv_c"][slots], x["k_pe"][slots], causal, scale)
        np.testing.assert_allclose(o[b * T:(b + 1) * T], ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# 2. absorbed form == un-absorbed per-head MLA with random W_UK / W_UV
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_absorbed_equals_unabsorbed(seed):
    B, H, P, T, Dl, Dr, dn, dv = 2, 3, 11, 6, 24, 8, 5, 7
    rng = np.random.default_rng(100 + seed)
    x = small_inputs(B, H, P, T, Dl, Dr, seed, paged=True)
    w_uk = rng.standard_normal((H, dn, Dl)) * 0.4
    w_uv = rng.standard_normal((H, dv, Dl))
    q_raw = rng.standard_normal((B * T, H, dn))
    # absorbed query: qn[h] = W_UK[h]^T q_raw[h]
    x["q_nope"] = np.einsum("hnd,rhn->rhd", w_uk, q_raw)
    scale = 1.0 / np.sqrt(dn + Dr)
    o_lat, lse = verify_attention(**x, scale=scale)
    N = P + T
    for b in range(B):
        slots = x["kv_indices"][b * N:(b + 1) * N]
        kc, kp = x["kv_c"][slots], x["k_pe"][slots]
        mask = np.ones((T, N), dtype=bool)
        mask[:, P:] = closure_mask(x["parents"][b])
        for h in range(H):
            k_nope = kc @ w_uk[h].T          # [N, dn] decompressed keys
            v = kc @ w_uv[h].T               # [N, dv] decompressed values
            q = np.concatenate([q_raw[b * T:(b + 1) * T, h], x["q_pe"][b * T:(b + 1) * T, h]], -1)
            k = np.concatenate([k_nope, kp], -1)
            out = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
                attn_mask=torch.from_numpy(mask)[None], scale=scale)[0].numpy()
            got = o_lat[b * T:(b + 1) * T, h] @ w_uv[h].T
            np.testing.assert_allclose(got, out, rtol=1e-10, atol=1e-12)
            s = scale * (q @ k.T)
            s[~mask] = -np.inf
            ref_lse = torch.logsumexp(torch.from_numpy(s), dim=-1).numpy()
            np.testing.assert_allclose(lse[b * T:(b + 1) * T, h], ref_lse, rtol=0, atol=1e-11)


# ---------------------------------------------------------------------------
# 3. normalisation
# ---------------------------------------------------------------------------

def test_constant_values_reproduce_exactly():
    """If every visible kv_c row is the same vector c, o = c for any scores."""
    x = small_inputs(2, 4, 13, 9, 16, 8, 5, paged=True, q_std=3.0)
    # Keep the scores non-trivial: vary k_pe only, set every kv_c row to c.
    c = np.linspace(-1.0, 2.0, 16)
    x["kv_c"][:] = c
    o, _ = verify_attention(**x, scale=0.9)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-12)


def test_softmax_rows_sum_to_one():
    x = small_inputs(2, 3, 17, 8, 16, 8, 6, paged=True, q_std=2.0)
    _, lse = verify_attention(**x, scale=0.5)
    T = x["parents"].shape[1]
    for b in range(2):
        for t in range(T):
            _, s = node_scores(**x, scale=0.5, b=b, t=t)
            tot = np.exp(s - lse[b * T + t][:, None]).sum(axis=1)
            np.testing.assert_allclose(tot, 1.0, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# 4. position-freeness: paged == contiguous, prefix permutation invariance
# ---------------------------------------------------------------------------

def test_paged_layout_equals_contiguous():
    B, H, P, T, Dl, Dr = 3, 2, 10, 5, 8, 4
    x = small_inputs(B, H, P, T, Dl, Dr, 7)
    o1, l1 = verify_attention(**x, scale=0.4)
    rng = np.random.default_rng(8)
    pool = 100
    perm = rng.permutation(pool)[:B * (P + T)]
    kv_c = rng.standard_normal((pool, Dl))
    k_pe = rng.standard_normal((pool, Dr))
    kv_c[perm] = x["kv_c"]
    k_pe[perm] = x["k_pe"]
    y = dict(x, kv_c=kv_c, k_pe=k_pe, kv_indices=perm.astype(np.int32))
    o2, l2 = verify_attention(**y, scale=0.4)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_prefix_permutation_invariance():
    B, H, P, T, Dl, Dr = 2, 3, 25, 6, 16, 8
    x = small_inputs(B, H, P, T, Dl, Dr, 9, paged=True)
    o1, l1 = verify_attention(**x, scale=0.6)
    rng = np.random.default_rng(10)
    idx = x["kv_indices"].copy()
    N = P + T
    for b in range(B):
        idx[b * N:b * N + P] = idx[b * N:b * N + P][rng.permutation(P)]
    o2, l2 = verify_attention(**dict(x, kv_indices=idx), scale=0.6)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# 5. scalar brute force on tiny shapes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind,seed", [("uniform", 11), ("bounded", 12), ("chain", 13)])
def test_brute_force_agrees(kind, seed):
    x = small_inputs(2, 3, 5, 6, 8, 4, seed, kind=kind, paged=True)
    o1, l1 = verify_attention(**x, scale=0.35)
    o2, l2 = brute_force_verify(**x, scale=0.35)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_brute_force_variable_lengths():
    """Sequences with different prefix lengths, including an empty prefix."""
    rng = np.random.default_rng(14)
    T, H, Dl, Dr = 4, 2, 8, 4
    P = [0, 3, 9]
    B = len(P)
    parents = np.stack([make_tree_parents(rng, T) for _ in range(B)])
    N = [p + T for p in P]
    indptr = np.concatenate([[0], np.cumsum(N)]).astype(np.int32)
    total = indptr[-1]
    x = dict(q_nope=rng.standard_normal((B * T, H, Dl)), q_pe=rng.standard_normal((B * T, H, Dr)),
             kv_c=rng.standard_normal((total + 3, Dl)), k_pe=rng.standard_normal((total + 3, Dr)),
             kv_indptr=indptr, kv_indices=rng.permutation(total + 3)[:total].astype(np.int32),
             parents=parents)
    o1, l1 = verify_attention(**x, scale=0.5)
    o2, l2 = brute_force_verify(**x, scale=0.5)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# 6. closed form at q = 0
# ---------------------------------------------------------------------------

def test_zero_query_closed_form():
    B, H, P, T, Dl, Dr = 2, 3, 7, 8, 8, 4
    x = small_inputs(B, H, P, T, Dl, Dr, 15, paged=True)
    x["q_nope"][:] = 0.0
    x["q_pe"][:] = 0.0
    o, lse = verify_attention(**x, scale=0.7)
    N = P + T
    for b in range(B):
        slots = x["kv_indices"][b * N:(b + 1) * N]
        kc = x["kv_c"][slots]
        reach = closure_mask(x["parents"][b])
        for t in range(T):
            vis = np.concatenate([np.ones(P, bool), reach[t]])
            np.testing.assert_allclose(o[b * T + t], np.broadcast_to(kc[vis].mean(0), (H, Dl)),
                                       rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[b * T + t], np.log(vis.sum()), rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# 7. tail isolation: only ancestors (and self) influence a node
# ---------------------------------------------------------------------------

def test_tail_isolation():
    B, H, P, T, Dl, Dr = 1, 2, 6, 10, 8, 4
    x = small_inputs(B, H, P, T, Dl, Dr, 16, kind="bounded")
    o1, l1 = verify_attention(**x, scale=0.5)
    reach = closure_mask(x["parents"][0])
    for u in range(T):
        y = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in x.items()}
        y["kv_c"][P + u] += 3.0
        y["k_pe"][P + u] -= 2.0
        o2, l2 = verify_attention(**y, scale=0.5)
        for t in range(T):
            if reach[t, u]:
                assert np.abs(o2[t] - o1[t]).max() > 1e-3, (t, u)
            else:
                np.testing.assert_array_equal(o2[t], o1[t])
                np.testing.assert_array_equal(l2[t], l1[t])


# ---------------------------------------------------------------------------
# 8. split-KV partials merged by log-sum-exp == unsplit
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("chunks", [1, 2, 3, 7, 40])
def test_split_merge_equals_unsplit(chunks):
    B, H, P, T, Dl, Dr = 1, 3, 30, 6, 8, 4
    x = small_inputs(B, H, P, T, Dl, Dr, 17, paged=True, q_std=2.0)
    o_ref, l_ref = verify_attention(**x, scale=0.5)
    N = P + T
    slots = x["kv_indices"][:N]
    for t in range(T):
        pos, s = node_scores(**x, scale=0.5, b=0, t=t)
        vals = x["kv_c"][slots[pos]]
        # chunk the logical key range [0, N) evenly; some chunks hold no visible key
        bounds = np.linspace(0, N, chunks + 1).round().astype(int)
        parts = []
        for c in range(chunks):
            sel = (pos >= bounds[c]) & (pos < bounds[c + 1])
            parts.append(chunk_partial(s[:, sel], vals[sel]))
        o, lse = merge_partials(parts)
        np.testing.assert_allclose(o, o_ref[t], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, l_ref[t], rtol=0, atol=1e-13)


def test_merge_with_all_but_one_chunk_empty():
    s = np.array([[0.5, -1.0, 2.0]])
    vals = np.array([[1.0, 0.0], [0.0, 1.0], [2.0, 2.0]])
    empty = chunk_partial(s[:, :0], vals[:0])
    assert np.isneginf(empty[0]).all() and (empty[1] == 0).all()
    o, lse = merge_partials([empty, chunk_partial(s, vals), empty])
    w = np.exp(s[0] - s[0].max())
    np.testing.assert_allclose(o[0], (w / w.sum()) @ vals, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0], s[0].max() + np.log(w.sum()), rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# 9. T = 1 reduces to single-token decode attention
# ---------------------------------------------------------------------------

def test_single_node_is_decode_attention():
    B, H, P, T, Dl, Dr = 2, 4, 33, 1, 16, 8
    x = small_inputs(B, H, P, T, Dl, Dr, 18, paged=True)
    o, _ = verify_attention(**x, scale=0.25)
    N = P + 1
    for b in range(B):
        slots = x["kv_indices"][b * N:(b + 1) * N]
        ref = sdpa_reference(x["q_nope"][b:b + 1], x["q_pe"][b:b + 1], x["kv_c"][slots],
                             x["k_pe"][slots], np.ones((1, N), bool), 0.25)
        np.testing.assert_allclose(o[b:b + 1], ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# 10. hand-worked example
# ---------------------------------------------------------------------------

def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "hand_worked_tree.json")) as f:
        g = json.load(f)
    arr = {k: np.asarray(g[k], dtype=np.float64) for k in ("q_nope", "q_pe", "kv_c", "k_pe")}
    o, lse = verify_attention(**arr, kv_indptr=np.asarray(g["kv_indptr"]),
                              kv_indices=np.asarray(g["kv_indices"]),
                              parents=np.asarray(g["parents"]), scale=g["scale"])
    np.testing.assert_allclose(o, g["expected_o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, g["expected_lse"], rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# tree helpers
# ---------------------------------------------------------------------------

def test_tree_ancestors_match_closure_and_reject_bad_parents():
    rng = np.random.default_rng(19)
    for kind in ("uniform", "bounded", "chain"):
        par = make_tree_parents(rng, 64, kind)
        anc = tree_ancestors(par)
        reach = closure_mask(par)
        for t in range(64):
            assert anc[t] == list(np.nonzero(reach[t])[0])
    with pytest.raises(ValueError):
        tree_ancestors([-1, 1])
    with pytest.raises(ValueError):
        tree_ancestors([-1, -2])


def test_sampled_nodes_match_full_run():
    cfg = get_config("tiny_f32_b1_h16_p256_t8")
    x = make_inputs(cfg)
    args = dict(q_nope=x.q_nope, q_pe=x.q_pe, kv_c=x.kv_c, k_pe=x.k_pe, kv_indptr=x.kv_indptr,
                kv_indices=x.kv_indices, parents=x.parents, scale=x.scale)
    o, lse = verify_attention(**args)
    o2, l2 = verify_attention(**args, nodes=[(0, 5), (0, 2)])
    np.testing.assert_array_equal(o2[0], o[5])
    np.testing.assert_array_equal(l2[1], lse[2])
