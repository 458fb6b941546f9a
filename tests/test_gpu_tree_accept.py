"""GPU parity of the token-acceptance kernel (mla_tree_accept) against the
oracle: integer outputs, compared exactly."""
import numpy as np
import pytest
import torch

from gen import make_accept_tokens, make_tree_parents
from oracle import tree_accept_batch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mla_absorbed_tree_amd import binding
    return binding


def _run(B, parents, draft, target, root):
    Bn, T = parents.shape
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    lens = torch.full((Bn,), -5, dtype=torch.int32, device="cuda")
    paths = torch.full((Bn, T), -5, dtype=torch.int32, device="cuda")
    bonus = torch.full((Bn,), -5, dtype=torch.int32, device="cuda")
    B.mla_tree_accept(dev(parents), dev(draft), dev(target), dev(root), Bn, T, lens, paths, bonus)
    torch.cuda.synchronize()
    return lens.cpu().numpy(), paths.cpu().numpy(), bonus.cpu().numpy()


@pytest.mark.parametrize("kind", ["uniform", "bounded", "chain"])
@pytest.mark.parametrize("T", [1, 2, 7, 31, 32, 33, 63, 64, 65, 100, 128, 129, 200, 255, 256])
def test_matches_oracle(B, kind, T):
    rng = np.random.default_rng(1000 + T + 100 * ["uniform", "bounded", "chain"].index(kind))
    Bn = 24
    parents = np.stack([make_tree_parents(rng, T, kind) for _ in range(Bn)]).astype(np.int32)
    if T > 3:  # invalid parents in a few sequences
        for b in range(0, Bn, 5):
            k = int(rng.integers(1, T))
            parents[b, k] = k + int(rng.integers(0, 3))
    toks = [make_accept_tokens(rng, parents[b], vocab=3, p_match=0.85) for b in range(Bn)]
    draft = np.stack([t[0] for t in toks])
    target = np.stack([t[1] for t in toks])
    root = np.array([t[2] for t in toks], dtype=np.int32)
    got = _run(B, parents, draft, target, root)
    want = tree_accept_batch(parents, draft, target, root)
    for g, w, name in zip(got, want, ("accept_len", "accept_path", "bonus_token")):
        np.testing.assert_array_equal(g, w, err_msg=name)
    assert want[0].max() >= min(2, T)  # the draw does produce accepted paths


def _run_packed(B, parents, draft, target, root, indptr, max_nodes):
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    Bn = len(indptr) - 1
    lens = torch.full((Bn,), -5, dtype=torch.int32, device="cuda")
    paths = torch.full((max(int(indptr[-1]), 1),), -5, dtype=torch.int32, device="cuda")
    bonus = torch.full((Bn,), -5, dtype=torch.int32, device="cuda")
    B.mla_tree_accept_packed(dev(parents), dev(draft), dev(target), dev(root), dev(indptr), Bn, max_nodes,
                             lens, paths, bonus)
    torch.cuda.synchronize()
    return lens.cpu().numpy(), paths.cpu().numpy()[:int(indptr[-1])], bonus.cpu().numpy()


@pytest.mark.parametrize("max_nodes", [64, 256])
def test_packed_matches_oracle(B, max_nodes):
    from oracle import tree_accept_packed
    rng = np.random.default_rng(2000 + max_nodes)
    sizes = [int(s) for s in rng.integers(0, max_nodes + 1, size=40)] + [0, max_nodes, 1]
    trees = [make_tree_parents(rng, T, ["uniform", "bounded", "chain"][i % 3]) for i, T in enumerate(sizes)]
    for i in range(0, len(trees), 7):  # invalid parents in a few trees
        if sizes[i] > 3:
            k = int(rng.integers(1, sizes[i]))
            trees[i][k] = k + int(rng.integers(0, 3))
    toks = [make_accept_tokens(rng, p, vocab=3, p_match=0.85) for p in trees]
    ind = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    cat = lambda xs: np.concatenate(xs).astype(np.int32)
    parents, draft, target = cat(trees), cat([t[0] for t in toks]), cat([t[1] for t in toks])
    root = np.array([t[2] for t in toks], np.int32)
    got = _run_packed(B, parents, draft, target, root, ind, max_nodes)
    want = tree_accept_packed(parents, draft, target, root, ind)
    for g, w, name in zip(got, want, ("accept_len", "accept_path", "bonus_token")):
        np.testing.assert_array_equal(g, w, err_msg=name)
    assert want[0].max() >= 3


def test_packed_equal_sizes_match_uniform_entry(B):
    rng = np.random.default_rng(2100)
    T, Bn = 100, 9
    parents = np.stack([make_tree_parents(rng, T, "bounded") for _ in range(Bn)]).astype(np.int32)
    toks = [make_accept_tokens(rng, parents[b], vocab=3, p_match=0.85) for b in range(Bn)]
    draft = np.stack([t[0] for t in toks])
    target = np.stack([t[1] for t in toks])
    root = np.array([t[2] for t in toks], dtype=np.int32)
    u = _run(B, parents, draft, target, root)
    k = _run_packed(B, parents.reshape(-1), draft.reshape(-1), target.reshape(-1), root,
                    np.arange(Bn + 1, dtype=np.int32) * T, T)
    for a, c in zip(u, k):
        np.testing.assert_array_equal(a.reshape(-1), c)


def test_packed_size_past_limit_is_flagged(B):
    """A device size above max_tree_nodes gives accept_len -1, the root token as
    bonus and no path writes; the other sequences are unaffected."""
    from oracle import tree_accept
    rng = np.random.default_rng(2200)
    sizes = [10, 65, 5]
    trees = [make_tree_parents(rng, T, "uniform") for T in sizes]
    toks = [make_accept_tokens(rng, p, vocab=3, p_match=0.9) for p in trees]
    ind = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    cat = lambda xs: np.concatenate(xs).astype(np.int32)
    root = np.array([t[2] for t in toks], np.int32)
    lens, paths, bonus = _run_packed(B, cat(trees), cat([t[0] for t in toks]), cat([t[1] for t in toks]),
                                     root, ind, 64)
    assert lens[1] == -1 and bonus[1] == root[1] and (paths[10:75] == -5).all()
    for b in (0, 2):
        n, path, tok = tree_accept(trees[b], toks[b][0], toks[b][1], toks[b][2])
        assert lens[b] == n and bonus[b] == tok
        seg = paths[ind[b]:ind[b + 1]]
        assert list(seg[:n]) == path and (seg[n:] == -1).all()
