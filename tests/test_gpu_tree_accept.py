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
