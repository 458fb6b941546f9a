"""Seeded input generator for the tree-verify workloads.

Draw order, fixed so that a workload is reproducible from its seed:
prefix lengths (only when they are random), tree sizes (only when they are
random), tree parents (sequence by sequence), q_nope, q_pe, kv_c, k_pe, then
the slot permutation (paged layout only).

Layout of what is produced (row-major numpy arrays):
  tree_indptr int32 [B+1] sequence b owns tree nodes tree_indptr[b]..tree_indptr[b+1]-1
                          (b*T for equal tree sizes)
  q_nope   [B*T, H, Dl]   absorbed no-RoPE query, row (b*T + t), head h
                          (packed trees: row tree_indptr[b] + t)
  q_pe     [B*T, H, Dr]   RoPE part of the query
  kv_c     [slots, Dl]    latent cache, one row per cache slot
  k_pe     [slots, Dr]    decoupled RoPE key, one row per cache slot
  kv_indptr  int32 [B+1]  sequence b owns kv_indices[kv_indptr[b]:kv_indptr[b+1]]
  kv_indices int32 [sum N_b]  slot of logical position j (prefix first, then the
                          T tree nodes in node order; page_size = 1)
  parents  int32 [B, T]   parent node of each tree node; -1 = child of the last
                          prefix token; parent[t] < t (packed trees: [sum T_b])
Floating arrays are float32. For bf16 workloads every value is already rounded
to bf16 (round-to-nearest-even), so widening to float64 or narrowing to bf16 is
exact on either side.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from .configs import VerifyConfig


@dataclasses.dataclass
class VerifyInputs:
    cfg: VerifyConfig
    q_nope: np.ndarray
    q_pe: np.ndarray
    kv_c: np.ndarray
    k_pe: np.ndarray
    kv_indptr: np.ndarray
    kv_indices: np.ndarray
    parents: np.ndarray
    prefix_lens: np.ndarray
    scale: float
    tree_indptr: Optional[np.ndarray] = None

    @property
    def tree_lens(self) -> np.ndarray:
        return np.diff(self.tree_indptr).astype(np.int64)

    @property
    def rows(self) -> int:
        return int(self.tree_indptr[-1]) * self.cfg.heads

    @property
    def kv_lens(self) -> np.ndarray:
        return np.diff(self.kv_indptr).astype(np.int64)

    @property
    def total_kv(self) -> int:
        return int(self.kv_indptr[-1])


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even), in place.

    Returns the same float32 array whose low 16 mantissa bits are now zero.
    Inputs here are finite normal draws, so no NaN/overflow handling is needed.
    """
    assert x.dtype == np.float32 and x.flags.c_contiguous
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return x


def make_tree_parents(rng: np.random.Generator, n: int, kind: str = "uniform",
                      max_depth: int = 8, max_branch: int = 4) -> np.ndarray:
    """Draw one draft tree of ``n`` nodes as a parent array (parent[0] = -1).

    "uniform": the parent of node i >= 1 is uniform over 0..i-1.
    "bounded": node 0 has depth 1; the parent of node i >= 1 is uniform over the
    earlier nodes whose depth is below ``max_depth`` and that have fewer than
    ``max_branch`` children.
    """
    parents = np.full(n, -1, dtype=np.int32)
    if kind == "uniform":
        for i in range(1, n):
            parents[i] = rng.integers(0, i)
    elif kind == "bounded":
        depth = np.zeros(n, dtype=np.int64)
        children = np.zeros(n, dtype=np.int64)
        if n:
            depth[0] = 1
        for i in range(1, n):
            eligible = [j for j in range(i) if depth[j] < max_depth and children[j] < max_branch]
            if not eligible:
                raise ValueError("tree bounds leave no room for node %d" % i)
            p = eligible[int(rng.integers(0, len(eligible)))]
            parents[i] = p
            depth[i] = depth[p] + 1
            children[p] += 1
    elif kind == "chain":
        parents[1:] = np.arange(n - 1, dtype=np.int32)
    else:
        raise ValueError(kind)
    return parents


def _normal(rng: np.random.Generator, shape, std: float, bf16: bool) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if bf16:
        round_to_bf16(x)
    return x


def make_inputs(cfg: VerifyConfig, *, poison_unused: bool = False,
                prefix_lens: Optional[np.ndarray] = None,
                tree_lens: Optional[np.ndarray] = None) -> VerifyInputs:
    """Draw the inputs of workload ``cfg`` from ``default_rng(cfg.seed)``.

    ``poison_unused`` fills cache slots that no sequence references with NaN
    (paged layout; the draws are unchanged). ``prefix_lens`` overrides the
    prefix lengths (then no length draw happens). ``tree_lens`` (or
    ``cfg.tree_range``) gives every sequence its own tree size and packs the
    trees; each size must lie in 0..cfg.tree_nodes.
    """
    rng = np.random.default_rng(cfg.seed)
    B, T, H, Dl, Dr = cfg.batch, cfg.tree_nodes, cfg.heads, cfg.d_latent, cfg.d_rope
    bf16 = cfg.dtype == "bf16"
    if cfg.dtype not in ("bf16", "f32"):
        raise ValueError(cfg.dtype)

    if prefix_lens is not None:
        P = np.asarray(prefix_lens, dtype=np.int64)
        assert P.shape == (B,)
    elif cfg.prefix_range is not None:
        lo, hi = cfg.prefix_range
        P = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int64)
    else:
        P = np.full(B, int(cfg.prefix), dtype=np.int64)
    ragged = tree_lens is not None or cfg.tree_range is not None
    if tree_lens is not None:
        Tb = np.asarray(tree_lens, dtype=np.int64)
        assert Tb.shape == (B,)
    elif cfg.tree_range is not None:
        lo, hi = cfg.tree_range
        Tb = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int64)
    else:
        Tb = np.full(B, T, dtype=np.int64)
    if (Tb < 0).any() or (Tb > T).any():
        raise ValueError("tree sizes must lie in 0..%d" % T)
    N = P + Tb
    tree_indptr = np.concatenate([[0], np.cumsum(Tb)]).astype(np.int32)

    trees = [make_tree_parents(rng, int(Tb[b]), cfg.tree_kind, cfg.max_depth, cfg.max_branch)
             for b in range(B)]
    if ragged:
        parents = np.concatenate(trees) if B else np.zeros(0, np.int32)
    else:
        parents = np.stack(trees) if B else np.zeros((0, T), np.int32)
    nodes = int(tree_indptr[-1])

    q_nope = _normal(rng, (nodes, H, Dl), cfg.q_std, bf16)
    q_pe = _normal(rng, (nodes, H, Dr), cfg.q_std, bf16)

    total = int(N.sum())
    slots = cfg.pool_slots if cfg.layout == "paged" else total
    if slots < total:
        raise ValueError("pool of %d slots cannot hold %d tokens" % (slots, total))
    kv_c = _normal(rng, (slots, Dl), cfg.kv_std, bf16)
    k_pe = _normal(rng, (slots, Dr), cfg.kv_std, bf16)

    indptr = np.zeros(B + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(N)
    if cfg.layout == "paged":
        perm = rng.permutation(slots)
        indices = perm[:total].astype(np.int32)
        if poison_unused:
            unused = perm[total:]
            kv_c[unused] = np.nan
            k_pe[unused] = np.nan
    elif cfg.layout == "contiguous":
        indices = np.arange(total, dtype=np.int32)
    else:
        raise ValueError(cfg.layout)

    return VerifyInputs(cfg=cfg, q_nope=q_nope, q_pe=q_pe, kv_c=kv_c, k_pe=k_pe,
                        kv_indptr=indptr.astype(np.int32), kv_indices=indices,
                        parents=parents.astype(np.int32), prefix_lens=P,
                        scale=float(cfg.scale), tree_indptr=tree_indptr)


def make_accept_tokens(rng: np.random.Generator, parents: np.ndarray, vocab: int = 4,
                       p_match: float = 0.8):
    """Synthetic draft and target tokens for one draft tree, for token acceptance.

    The target's token after each node and after the prefix are uniform over
    ``vocab``; a node's draft token copies the target's token after its parent
    (after the prefix for a root) with probability ``p_match``, else it is
    uniform. Returns (draft [T], target [T], root_target) as int32 / int.
    Invalid parents (the generator does not draw them; tests plant them) are
    treated as roots here.
    """
    T = len(parents)
    target = rng.integers(0, vocab, size=T).astype(np.int32)
    root_target = int(rng.integers(0, vocab))
    draft = rng.integers(0, vocab, size=T).astype(np.int32)
    copy = rng.random(T) < p_match
    for t in range(T):
        if copy[t]:
            p = int(parents[t])
            draft[t] = target[p] if 0 <= p < t else root_target
    return draft, target, root_target
