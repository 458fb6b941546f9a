"""CPU oracle for greedy token acceptance over a verified draft tree.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the tests use it. It shares no code with the HIP
library.

The pages list token acceptance among the speculative-decoding kernels next to
tree-verify attention ("Ground Truth in Silicon" page, "Input Knowledge
Required", item 1) without defining it. Reading taken (greedy acceptance along
the tree): a node is accepted when its draft token equals the target model's
greedy token after its parent (after the last prefix token for a node whose
parent is -1) and its parent is accepted. The result is the deepest accepted
node (ties: smallest index), its root path, and the target's token after it
(the "bonus" token; the token after the prefix when nothing is accepted).
Nodes on an invalid parent chain are never accepted.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np


def _ancestor_sets(parents) -> List[List[int]]:
    """Ancestor-or-self node lists; empty for a node whose root path holds an
    invalid parent (not an earlier node, or below -1)."""
    out: List[List[int]] = []
    for t, p in enumerate(int(v) for v in parents):
        if p < -1 or p >= t or (p >= 0 and not out[p]):
            out.append([])
        else:
            out.append([t] + (out[p] if p >= 0 else []))
    return out


def tree_accept(parents: np.ndarray, draft: np.ndarray, target: np.ndarray,
                root_target: int) -> Tuple[int, List[int], int]:
    """One sequence: (accept_len, path root -> deepest accepted node, bonus token)."""
    T = len(parents)
    anc = _ancestor_sets(parents)
    accepted = [False] * T
    for t in range(T):              # a valid parent precedes its child
        if not anc[t]:
            continue
        p = int(parents[t])
        want = root_target if p < 0 else int(target[p])
        accepted[t] = int(draft[t]) == want and (p < 0 or accepted[p])
    best, best_depth = -1, 0
    for t in range(T):
        if accepted[t] and len(anc[t]) > best_depth:
            best, best_depth = t, len(anc[t])
    if best < 0:
        return 0, [], int(root_target)
    path = sorted(anc[best], key=lambda u: len(anc[u]))
    return best_depth, path, int(target[best])


def tree_accept_batch(parents: np.ndarray, draft: np.ndarray, target: np.ndarray,
                      root_target: np.ndarray):
    """Batched form with the C entry point's output layout:
    (accept_len [B], accept_path [B, T] padded with -1, bonus_token [B])."""
    B, T = parents.shape
    lens = np.zeros(B, np.int32)
    paths = np.full((B, T), -1, np.int32)
    bonus = np.zeros(B, np.int32)
    for b in range(B):
        n, path, tok = tree_accept(parents[b], draft[b], target[b], int(root_target[b]))
        lens[b], bonus[b] = n, tok
        paths[b, :n] = path
    return lens, paths, bonus


def tree_accept_packed(parents: np.ndarray, draft: np.ndarray, target: np.ndarray,
                       root_target: np.ndarray, tree_indptr: np.ndarray):
    """Packed trees: sequence b owns nodes tree_indptr[b] .. tree_indptr[b+1]-1
    of the flat parents / draft / target arrays (parents are node indices of
    the same tree). Returns (accept_len [B], accept_path [sum T_b] where
    sequence b's path starts at tree_indptr[b] and is padded with -1 to T_b,
    bonus_token [B])."""
    ind = [int(v) for v in np.asarray(tree_indptr)]
    B = len(ind) - 1
    lens = np.zeros(B, np.int32)
    paths = np.full(ind[-1], -1, np.int32)
    bonus = np.zeros(B, np.int32)
    for b in range(B):
        lo, hi = ind[b], ind[b + 1]
        n, path, tok = tree_accept(parents[lo:hi], draft[lo:hi], target[lo:hi], int(root_target[b]))
        lens[b], bonus[b] = n, tok
        paths[lo:lo + n] = path
    return lens, paths, bonus
