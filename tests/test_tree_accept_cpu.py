"""Token acceptance on the CPU: the oracle against hand-worked cases, the
linear (chain) special case, and a path-enumeration brute force; plus the
C-ABI argument checks (no device work)."""
import json
import os

import numpy as np
import pytest

from gen import make_accept_tokens, make_tree_parents
from oracle import tree_accept

HERE = os.path.dirname(os.path.abspath(__file__))


def test_hand_worked_cases():
    g = json.load(open(os.path.join(HERE, "golden", "tree_accept_small.json")))
    for c in g["cases"]:
        got = tree_accept(np.array(c["parents"]), np.array(c["draft"]), np.array(c["target"]),
                          c["root_target"])
        assert got == (c["accept_len"], c["path"], c["bonus"]), c["name"]


@pytest.mark.parametrize("seed", range(4))
def test_chain_is_linear_speculative_acceptance(seed):
    """On a chain the tree rule is ordinary linear speculative decoding: accept
    the longest draft prefix that matches the target's tokens shifted by one."""
    rng = np.random.default_rng(seed)
    T = 40
    parents = np.arange(-1, T - 1)
    draft, target, root = make_accept_tokens(rng, parents, vocab=3, p_match=0.9)
    want = np.concatenate([[root], target[:-1]])     # token the target emits before each position
    n = 0
    while n < T and draft[n] == want[n]:
        n += 1
    got = tree_accept(parents, draft, target, root)
    assert got == (n, list(range(n)), int(target[n - 1]) if n else root)


def _brute_force(parents, draft, target, root):
    """Every node's root path by walking parent pointers; a path is accepted
    when every step matches; keep the deepest, smallest index first."""
    best = (0, [], int(root))
    for t in range(len(parents)):
        path, u, ok = [], t, True
        while u >= 0:
            p = int(parents[u])
            if p < -1 or p >= u:
                ok = False
                break
            path.append(u)
            u = p
        if not ok:
            continue
        path.reverse()
        prev_tok = root
        for u in path:
            if draft[u] != prev_tok:
                ok = False
                break
            prev_tok = target[u]
        if ok and len(path) > best[0]:
            best = (len(path), path, int(target[t]))
    return best


@pytest.mark.parametrize("kind", ["uniform", "bounded", "chain"])
def test_brute_force_agrees(kind):
    rng = np.random.default_rng({"uniform": 10, "bounded": 11, "chain": 12}[kind])
    for T in (1, 2, 5, 17, 64, 65, 130):
        for _ in range(20):
            parents = make_tree_parents(rng, T, kind)
            if T > 3 and rng.random() < 0.3:      # plant an invalid parent
                k = int(rng.integers(1, T))
                parents = parents.copy()
                parents[k] = k + int(rng.integers(0, 3))
            draft, target, root = make_accept_tokens(rng, parents, vocab=3, p_match=0.8)
            assert tree_accept(parents, draft, target, root) == _brute_force(parents, draft, target, root)


@pytest.fixture(scope="module")
def B():
    from mla_absorbed_tree_amd import binding
    return binding


def test_capi_argument_checks(B):
    fake = 1 << 20  # never dereferenced: every call below fails validation first
    args = dict(tree_parents=fake, draft_tokens=fake, target_tokens=fake, root_targets=fake, batch=2,
                tree_nodes=16, accept_len=fake, accept_path=fake, bonus_token=fake, stream=0)
    for over in (dict(batch=0), dict(tree_nodes=0), dict(tree_nodes=257), dict(draft_tokens=0),
                 dict(accept_path=0)):
        with pytest.raises(B.MlaVerifyError) as e:
            B.mla_tree_accept(**{**args, **over})
        assert e.value.status == B.MLA_ERR_INVALID_ARG, over
    packed = dict(tree_parents=fake, draft_tokens=fake, target_tokens=fake, root_targets=fake,
                  tree_indptr=fake, batch=2, max_tree_nodes=16, accept_len=fake, accept_path=fake,
                  bonus_token=fake, stream=0)
    for over in (dict(batch=0), dict(max_tree_nodes=-1), dict(max_tree_nodes=257), dict(tree_indptr=0),
                 dict(draft_tokens=0), dict(bonus_token=0)):
        with pytest.raises(B.MlaVerifyError) as e:
            B.mla_tree_accept_packed(**{**packed, **over})
        assert e.value.status == B.MLA_ERR_INVALID_ARG, over


def test_packed_trees_match_per_sequence_results():
    """Packed layout: each sequence's slice gives exactly the single-tree
    result (checked by the brute force), including empty trees; with equal
    sizes the packed result is the uniform batch result flattened."""
    from oracle import tree_accept_batch, tree_accept_packed
    rng = np.random.default_rng(77)
    sizes = [5, 0, 70, 1, 130, 0, 17]
    trees = [make_tree_parents(rng, T, "uniform") for T in sizes]
    toks = [make_accept_tokens(rng, p, vocab=3, p_match=0.85) for p in trees]
    ind = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    flat = lambda k: np.concatenate([t[k] for t in toks]).astype(np.int32)
    parents = np.concatenate(trees).astype(np.int32)
    root = np.array([t[2] for t in toks], np.int32)
    lens, paths, bonus = tree_accept_packed(parents, flat(0), flat(1), root, ind)
    for b, T in enumerate(sizes):
        n, path, tok = _brute_force(trees[b], toks[b][0], toks[b][1], toks[b][2])
        assert (lens[b], bonus[b]) == (n, tok), b
        assert list(paths[ind[b]:ind[b] + n]) == path and (paths[ind[b] + n:ind[b + 1]] == -1).all()
    # equal sizes: same as the uniform batch layout
    P = np.stack([make_tree_parents(rng, 9, "bounded") for _ in range(4)]).astype(np.int32)
    tk = [make_accept_tokens(rng, P[b], vocab=3, p_match=0.85) for b in range(4)]
    d, t, r = (np.stack([x[0] for x in tk]), np.stack([x[1] for x in tk]), np.array([x[2] for x in tk]))
    u = tree_accept_batch(P, d, t, r)
    k = tree_accept_packed(P.reshape(-1), d.reshape(-1), t.reshape(-1), r, np.arange(5) * 9)
    for a, c in zip(u, k):
        np.testing.assert_array_equal(a.reshape(-1), c)
