"""Float64 CPU oracle for absorbed-MLA tree-verify attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP library.

What is computed (sources are the pages this project follows):

* The cache holds, per token j, a latent ``kv_c[j]`` of width Dl (512) and a
  decoupled RoPE key ``k_pe[j]`` of width Dr (64), both shared by every head;
  the query has been pre-multiplied into latent space ("absorbed"), so head h of
  a query brings ``q_nope[h]`` (Dl wide) and ``q_pe[h]`` (Dr wide).
  -- "Ground Truth in Silicon" page: "The Message in Full" (the oracle's
  docstring) and "Input Knowledge Required", item 2.
* Score of query row (b, t, h) against key j: one scale applied to the sum of
  the latent dot product and the RoPE dot product. The pages' formula is cut off;
  this is the DeepSeek-V3 absorbed form, and the un-absorbed identity test pins it.
* Visibility: the whole prefix, plus the tree-tail tokens of the node itself and
  of its ancestors ("Reading the Reference" page, "Output Knowledge Created by
  This Message": prefix visibility + tree-tail visibility; "Ground Truth in
  Silicon" page, "Input Knowledge Required", item 3). Reading taken: a node sees
  itself (ancestor-or-self), pinned by the chain-tree == causal test.
* Output: softmax over the visible keys, applied to ``kv_c`` (latent-space
  output; the caller applies W_UV), plus the natural-log log-sum-exp of the
  scaled scores ("output aggregation", same page, "Output Knowledge Created").
* Trees of any size, and a different tree size per sequence: every node of the
  draft tree is a query of the verify step, and the pages fix neither how many
  nodes a tree has nor that every sequence has the same number ("Ground Truth
  in Silicon" page, "Input Knowledge Required", item 3). Packed ("ragged") layout: sequence b owns tree nodes
  tree_indptr[b] .. tree_indptr[b+1]-1; its query rows and parent entries are
  stored in that order. With equal sizes T this is the [B*T] / [B, T] layout.
* Split-KV (flash-decode, "The Information-Gathering Pivot" page, "The Context:
  A Multi-Phase Kernel Integration"): per chunk of keys a partial (m, l, O);
  chunks are merged by log-sum-exp.

All inputs are widened exactly to float64 before any arithmetic.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------
# Tree structure
# --------------------------------------------------------------------------

def tree_ancestors(parents: Sequence[int]) -> List[List[int]]:
    """Ancestor-or-self sets of a draft tree given as a parent array.

    A(t) = {t} union A(parent[t]) when parent[t] >= 0, else {t}; parent -1 means
    the node hangs off the last prefix token, which every node sees anyway.
    Returned lists are sorted ascending. Raises on a parent that is not an
    earlier node (the tree is stored in topological order).
    """
    parents = [int(p) for p in parents]
    out: List[List[int]] = []
    for t, p in enumerate(parents):
        if p < -1 or p >= t:
            raise ValueError("parent[%d] = %d is not an earlier node or -1" % (t, p))
        anc = {t}
        if p >= 0:
            anc.update(out[p])
        out.append(sorted(anc))
    return out


def visible_positions(prefix_len: int, ancestors_of_t: Sequence[int]) -> np.ndarray:
    """Logical key positions node t sees: 0..P-1, then P+u for each u in A(t)."""
    tail = prefix_len + np.asarray(ancestors_of_t, dtype=np.int64)
    return np.concatenate([np.arange(prefix_len, dtype=np.int64), tail])


def tree_mask_words(parents: Sequence[int], words: int) -> np.ndarray:
    """Ancestor-or-self sets as bit masks: uint64 [T, words], bit u%64 of word
    u//64 of row t set iff u is in A(t). A node whose parent chain holds an
    invalid parent (not an earlier node and not -1) gets an all-zero row.
    """
    parents = [int(p) for p in parents]
    T = len(parents)
    out = np.zeros((T, words), dtype=np.uint64)
    for t in range(T):
        node, ok, members = t, True, []
        while node >= 0:
            p = parents[node]
            if p < -1 or p >= node:
                ok = False
                break
            members.append(node)
            node = p
        if ok:
            for u in members:
                out[t, u // 64] |= np.uint64(1) << np.uint64(u % 64)
    return out


def _tree_layout(parents, tree_indptr):
    """(per-sequence parent lists, first packed node of each sequence)."""
    if tree_indptr is None:
        parents = np.asarray(parents)
        B, T = parents.shape
        return [parents[b] for b in range(B)], [b * T for b in range(B + 1)]
    ind = [int(v) for v in np.asarray(tree_indptr)]
    flat = np.asarray(parents).reshape(-1)
    if ind[0] != 0 or ind[-1] != len(flat) or any(ind[b + 1] < ind[b] for b in range(len(ind) - 1)):
        raise ValueError("tree_indptr does not describe the packed parent array")
    return [flat[ind[b]:ind[b + 1]] for b in range(len(ind) - 1)], ind


# --------------------------------------------------------------------------
# Vectorised oracle (numpy float64 matmuls)
# --------------------------------------------------------------------------

def _node_scores(qn: np.ndarray, qp: np.ndarray, kc: np.ndarray, kp: np.ndarray,
                 scale: float) -> np.ndarray:
    """s[h, j] = scale * (qn[h] . kc[j] + qp[h] . kp[j]), float64."""
    return scale * (qn @ kc.T + qp @ kp.T)


def verify_attention(q_nope, q_pe, kv_c, k_pe, kv_indptr, kv_indices, parents, scale,
                     nodes: Optional[Iterable[Tuple[int, int]]] = None, tree_indptr=None):
    """Tree-verify attention in float64.

    Shapes: q_nope [B*T, H, Dl], q_pe [B*T, H, Dr], kv_c [slots, Dl],
    k_pe [slots, Dr], kv_indptr [B+1], kv_indices [sum N_b] (page_size = 1,
    logical position j of sequence b lives in slot kv_indices[kv_indptr[b]+j];
    the last T positions are the tree nodes), parents [B, T].
    With ``tree_indptr`` [B+1] the trees are packed: sequence b has
    T_b = tree_indptr[b+1] - tree_indptr[b] nodes (0 allowed), parents is
    [sum T_b] and node (b, t) is query row tree_indptr[b] + t.

    Returns (o, lse): o [rows, H, Dl] and lse [rows, H] in float64, where rows
    is the number of nodes (packed order), or len(nodes) when ``nodes`` lists
    the (b, t) pairs to evaluate.
    """
    trees, first = _tree_layout(parents, tree_indptr)
    B = len(trees)
    H = q_nope.shape[1]
    Dl = q_nope.shape[2]
    want = [(b, t) for b in range(B) for t in range(len(trees[b]))] if nodes is None else list(nodes)
    o = np.zeros((len(want), H, Dl), dtype=np.float64)
    lse = np.zeros((len(want), H), dtype=np.float64)
    by_seq = {}
    for i, (b, t) in enumerate(want):
        by_seq.setdefault(b, []).append((i, t))
    for b, items in by_seq.items():
        T = len(trees[b])
        start, end = int(kv_indptr[b]), int(kv_indptr[b + 1])
        n = end - start
        P = n - T
        if P < 0:
            raise ValueError("sequence %d holds fewer tokens than tree nodes" % b)
        slots = np.asarray(kv_indices[start:end], dtype=np.int64)
        kc = np.asarray(kv_c[slots], dtype=np.float64)
        kp = np.asarray(k_pe[slots], dtype=np.float64)
        anc = tree_ancestors(trees[b])
        for i, t in items:
            qn = np.asarray(q_nope[first[b] + t], dtype=np.float64)
            qp = np.asarray(q_pe[first[b] + t], dtype=np.float64)
            tail = P + np.asarray(anc[t], dtype=np.int64)
            # V(b, t) = prefix (contiguous positions 0..P-1) followed by the tail keys.
            s = np.concatenate([_node_scores(qn, qp, kc[:P], kp[:P], scale),
                                _node_scores(qn, qp, kc[tail], kp[tail], scale)], axis=1)
            m = s.max(axis=1, keepdims=True)
            z = np.exp(s - m).sum(axis=1, keepdims=True)
            row_lse = m + np.log(z)
            w = np.exp(s - row_lse)
            o[i] = w[:, :P] @ kc[:P] + w[:, P:] @ kc[tail]
            lse[i] = row_lse[:, 0]
    return o, lse


def node_scores(q_nope, q_pe, kv_c, k_pe, kv_indptr, kv_indices, parents, scale, b, t,
                tree_indptr=None):
    """Scores of node (b, t) against its visible keys: (positions [V], s [H, V])."""
    trees, first = _tree_layout(parents, tree_indptr)
    T = len(trees[b])
    start, end = int(kv_indptr[b]), int(kv_indptr[b + 1])
    P = end - start - T
    anc = tree_ancestors(trees[b])
    pos = visible_positions(P, anc[t])
    slots = np.asarray(kv_indices[start:end], dtype=np.int64)[pos]
    qn = np.asarray(q_nope[first[b] + t], dtype=np.float64)
    qp = np.asarray(q_pe[first[b] + t], dtype=np.float64)
    s = _node_scores(qn, qp, np.asarray(kv_c[slots], np.float64),
                     np.asarray(k_pe[slots], np.float64), scale)
    return pos, s


# --------------------------------------------------------------------------
# Split-KV partials and their log-sum-exp merge
# --------------------------------------------------------------------------

def chunk_partial(s: np.ndarray, values: np.ndarray):
    """Partial state of one key chunk for each row.

    s [H, n] scores of the chunk's visible keys, values [n, Dl].
    Returns m [H] (chunk max, -inf if empty), l [H] = sum exp(s - m) (0 if
    empty), O [H, Dl] = sum exp(s - m) * values (0 if empty).
    """
    H = s.shape[0]
    Dl = values.shape[1]
    if s.shape[1] == 0:
        return np.full(H, -np.inf), np.zeros(H), np.zeros((H, Dl))
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    return m, e.sum(axis=1), e @ values


def merge_partials(parts):
    """Log-sum-exp merge of chunk partials (m, l, O) into (o, lse).

    M = max m_c; L = sum l_c exp(m_c - M); o = sum exp(m_c - M) O_c / L;
    lse = M + ln L. Empty chunks (m = -inf, l = 0) contribute nothing.
    """
    ms = np.stack([p[0] for p in parts])          # [C, H]
    M = ms.max(axis=0)
    L = np.zeros_like(M)
    O = np.zeros_like(parts[0][2])
    for m, l, Oc in parts:
        live = np.isfinite(m)
        f = np.where(live, np.exp(np.where(live, m - M, 0.0)), 0.0)
        L += f * l
        O += f[:, None] * Oc
    return O / L[:, None], M + np.log(L)


# --------------------------------------------------------------------------
# Scalar brute force (pure Python loops; tiny shapes only)
# --------------------------------------------------------------------------

def brute_force_verify(q_nope, q_pe, kv_c, k_pe, kv_indptr, kv_indices, parents, scale,
                       tree_indptr=None):
    """Same definition as ``verify_attention``, written as scalar Python loops.

    Visibility is decided per key by walking the parent pointers of the query
    node, not by the ancestor lists above. Dimension-generic; use tiny shapes.
    ``tree_indptr`` as in ``verify_attention`` (packed trees).
    """
    if tree_indptr is None:
        rows2d = [[int(x) for x in row] for row in np.asarray(parents)]
        B = len(rows2d)
        T0 = len(rows2d[0]) if B else 0
        ind = [b * T0 for b in range(B + 1)]
        flat = [x for row in rows2d for x in row]
    else:
        ind = [int(v) for v in np.asarray(tree_indptr)]
        B = len(ind) - 1
        flat = [int(x) for x in np.asarray(parents).reshape(-1)]
    rows = ind[-1]
    H = len(q_nope[0]) if len(q_nope) else 0
    Dl = len(kv_c[0])
    Dr = len(k_pe[0])
    o = [[[0.0] * Dl for _ in range(H)] for _ in range(rows)]
    lse = [[0.0] * H for _ in range(rows)]
    for b in range(B):
        par = flat[ind[b]:ind[b + 1]]
        T = len(par)
        start, end = int(kv_indptr[b]), int(kv_indptr[b + 1])
        P = end - start - T
        for t in range(T):
            row = ind[b] + t
            for h in range(H):
                keys = []
                scores = []
                for j in range(end - start):
                    if j >= P:
                        u = j - P
                        node, seen = t, False
                        while node >= 0:
                            if node == u:
                                seen = True
                                break
                            node = par[node]
                        if not seen:
                            continue
                    slot = int(kv_indices[start + j])
                    acc = 0.0
                    for d in range(Dl):
                        acc += float(q_nope[row][h][d]) * float(kv_c[slot][d])
                    for r in range(Dr):
                        acc += float(q_pe[row][h][r]) * float(k_pe[slot][r])
                    keys.append(slot)
                    scores.append(scale * acc)
                mx = max(scores)
                tot = 0.0
                for sc in scores:
                    tot += math.exp(sc - mx)
                row_lse = mx + math.log(tot)
                lse[row][h] = row_lse
                for slot, sc in zip(keys, scores):
                    w = math.exp(sc - row_lse)
                    for d in range(Dl):
                        o[row][h][d] += w * float(kv_c[slot][d])
    return np.array(o, dtype=np.float64).reshape(rows, H, Dl), \
        np.array(lse, dtype=np.float64).reshape(rows, H)
