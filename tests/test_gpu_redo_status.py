"""GPU checks of three run-time rules of libmlaverify against the float64
oracle and against what the header promises:

* the softmax redo: a score more than 64 (log2 units) above the reference max
  that a row fixed on its first tile makes the workgroup repeat its keys with
  the exact max -- for the fp32 kernel, and for the bf16 kernel with a single
  split (the pass that ends in the final epilogue, not in split partials);
* the per-sequence status words at the start of the workspace (bad parent,
  KV shorter than the tree, device tree entries out of range), for sequences
  with and without work, eagerly and inside a captured graph;
* device tree offsets that end past tree_indptr[batch]: the sequence is
  skipped by the attention and the acceptance kernels (sentinel-filled spare
  rows stay untouched).
"""
import numpy as np
import pytest

from gen import get_config, make_inputs
from gen.inputs import round_to_bf16
from gpu_util import compare, log, run_hip, run_oracle

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_absorbed_tree_amd.binding  # noqa: F401  (fails loudly if the library is missing)


def _dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.to(dtype) if dtype is not None else t).cuda()


# --------------------------------------------------------------------------
# softmax redo
# --------------------------------------------------------------------------

def _plant_late_spike(x, seq, pos, seed):
    """Queries along one direction, one prefix key of sequence `seq` (logical
    position `pos`) 40x longer along it: that key outscores the first tile
    by far more than the 64-unit slack."""
    rng = np.random.default_rng(seed)
    direction = rng.standard_normal(576).astype(np.float32)
    direction /= np.linalg.norm(direction)
    x.q_nope[:] = 5.0 * direction[:512]
    x.q_pe[:] = 5.0 * direction[512:]
    spike = int(x.kv_indices[int(x.kv_indptr[seq]) + pos])
    x.kv_c[spike] = 200.0 * direction[:512]
    x.k_pe[spike] = 200.0 * direction[512:]
    if x.cfg.dtype == "bf16":
        for a in (x.q_nope, x.q_pe, x.kv_c, x.k_pe):
            round_to_bf16(a)
    return spike


def _excess_over_first_tile(x, seq, spike):
    """max over sequence `seq`'s rows of (spike score - max score of keys
    0..31), in log2 units (what the kernels compare with their slack)."""
    q = np.concatenate([x.q_nope, x.q_pe], axis=-1).astype(np.float64)  # [nodes, H, 576]
    kv = np.concatenate([x.kv_c, x.k_pe], axis=-1).astype(np.float64)
    first = x.kv_indices[int(x.kv_indptr[seq]):int(x.kv_indptr[seq]) + 32]
    rows = q[int(x.tree_indptr[seq]):int(x.tree_indptr[seq + 1])]
    s_first = np.einsum("thd,kd->thk", rows, kv[first]).max(-1)
    s_spike = np.einsum("thd,d->th", rows, kv[spike])
    return float(((s_spike - s_first) * x.scale * LOG2E).min())


def test_redo_bf16_single_split():
    cfg = get_config("b1_h64_p4096_t16_bf16", prefix=3000, seed=61)
    x = make_inputs(cfg)
    spike = _plant_late_spike(x, 0, 2500, 62)
    assert _excess_over_first_tile(x, 0, spike) > 64.0   # every row takes the redo
    o, lse, info = run_hip(x, 1)
    assert info["total_splits"] == 1 and info["uses_combine"] == 0, info
    o_ref, lse_ref = run_oracle(x)
    compare(o, lse, o_ref, lse_ref, "bf16", "plan=%s" % info)
    assert np.abs(o - x.kv_c[spike]).max() < 0.05         # every row locks onto the spike


@pytest.mark.parametrize("splits", [1, 3])
def test_redo_fp32(splits):
    cfg = get_config("tiny_f32_b1_h16_p256_t8", batch=2, prefix=300, seed=63)
    x = make_inputs(cfg)
    spike = _plant_late_spike(x, 1, 250, 64)
    assert _excess_over_first_tile(x, 1, spike) > 64.0
    o, lse, info = run_hip(x, splits)
    assert info["total_splits"] == 2 * splits, info
    o_ref, lse_ref = run_oracle(x)
    # Outputs: the fp32 bound (1e-4 of the output RMS). LSE: the 1e-5 absolute
    # bound is meant for scores of order one; the spike scores about 72 here,
    # and an fp32 dot product of 576 terms carries an error of order
    # 2^-24 * sqrt(576) * scale * sum|q*k|, which is added to it.
    d = np.abs(o.astype(np.float64) - o_ref)
    rms = np.sqrt(np.mean(o_ref ** 2))
    kv = np.concatenate([x.kv_c, x.k_pe], axis=-1).astype(np.float64)
    q = np.concatenate([x.q_nope, x.q_pe], axis=-1).astype(np.float64)
    mag = float((np.abs(q) * np.abs(kv[spike])).sum(-1).max())
    lse_tol = 1e-5 + 2.0 ** -24 * 32 * x.scale * mag
    dl = np.abs(lse.astype(np.float64) - lse_ref).max()
    log("  max|do|=%.3g (rms %.3g) max|dlse|=%.3g (bound %.3g) plan=%s" % (d.max(), rms, dl, lse_tol, info))
    assert np.isfinite(o).all() and d.max() <= 1e-4 * rms
    assert dl <= lse_tol
    assert np.abs(o[cfg.tree_nodes:] - x.kv_c[spike]).max() < 1e-3   # sequence 1 locks onto it


# --------------------------------------------------------------------------
# status words
# --------------------------------------------------------------------------

SENTINEL = 0x5A5A5A5A


def _status(mv, batch):
    return mv.workspace[:4 * batch].view(__import__("torch").int32).cpu().numpy().copy()


def test_status_words_eager_and_in_a_graph():
    """Five packed sequences: a valid tree, an empty one, a tree with a
    forward parent, a tree whose device KV length is shorter than the tree,
    and a trailing empty one. The empty ones have no workgroup; their words
    come from their neighbours' first workgroups."""
    import torch
    from mla_absorbed_tree_amd import binding as B
    from mla_absorbed_tree_amd.verify import MlaVerify, device_inputs

    cfg = get_config("b1_h64_p4096_t16_bf16", batch=5, heads=8, tree_nodes=5, prefix=70, seed=65)
    x = make_inputs(cfg, tree_lens=[3, 0, 4, 5, 0])
    x.parents[3 + 2] = 3                       # sequence 2, node 2 -> parent 3 (forward): invalid
    d = device_inputs(x)
    mv = MlaVerify(5, 8, 5, "bf16", x.kv_lens, 2, tree_lens=[3, 0, 4, 5, 0])
    short = x.kv_indptr.copy()
    short[4:] -= (x.kv_lens[3] - 3)            # sequence 3 keeps 3 keys on the device: N < T = 5
    kv_indptr = _dev(short)
    nodes = int(x.tree_indptr[-1])
    out = torch.empty((nodes, 8, 512), device="cuda")
    lse = torch.empty((nodes, 8), device="cuda")
    args = (d["q_nope"], d["q_pe"], d["kv_c"], d["k_pe"], kv_indptr, d["kv_indices"], d["tree_parents"],
            x.scale)
    want = [0, 0, B.MLA_VERIFY_STATUS_BAD_PARENT, B.MLA_VERIFY_STATUS_SHORT_KV, 0]

    mv.workspace[:4 * 5].view(torch.int32).fill_(SENTINEL)
    mv(*args, out=out, lse=lse)
    torch.cuda.synchronize()
    assert list(_status(mv, 5)) == want
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    assert np.isnan(o[7:12]).all() and np.isnan(l[7:12]).all()          # sequence 3: every row
    assert np.isnan(o[3 + 2]).all() and not np.isnan(o[3:5]).any()       # sequence 2: node 2 (and
    assert np.isnan(o[3 + 3]).all() == (x.parents[3 + 3] == 2)           # a child of it) only
    o_ref, lse_ref = run_oracle(x, nodes=[(0, t) for t in range(3)])
    compare(o[:3], l[:3], o_ref, lse_ref, "bf16")

    # Captured: the replay writes the words again; after fixing the parent
    # and the length in place, the next replay reports a clean batch.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mv(*args, out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mv(*args, out=out, lse=lse)
    torch.cuda.synchronize()
    mv.workspace[:4 * 5].view(torch.int32).fill_(SENTINEL)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert list(_status(mv, 5)) == want
    d["tree_parents"][3 + 2] = 0
    kv_indptr.copy_(_dev(x.kv_indptr))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert list(_status(mv, 5)) == [0, 0, 0, 0, 0]
    del g
    mv.close()


# --------------------------------------------------------------------------
# device tree offsets past the end of the node arrays
# --------------------------------------------------------------------------

def test_varlen_tree_ending_past_the_node_arrays_is_skipped():
    """tree_indptr = [0, 4, 7, 6]: sequence 1 has a size inside its bound (3)
    but ends at node 7 > tree_indptr[3] = 6; sequence 2 has a negative size.
    Both are skipped; out/lse carry sentinel-filled rows past the 6 nodes."""
    import torch
    from mla_absorbed_tree_amd import binding as B
    from mla_absorbed_tree_amd.verify import MlaVerify, device_inputs

    cfg = get_config("b1_h64_p4096_t16_bf16", batch=3, heads=8, tree_nodes=4, prefix=50, seed=66)
    x = make_inputs(cfg, tree_lens=[4, 2, 0])
    d = device_inputs(x)
    mv = MlaVerify(3, 8, 4, "bf16", np.asarray(x.prefix_lens) + 4, 2, tree_lens=[4, 4, 4])
    out = torch.full((10, 8, 512), 7.0, device="cuda")
    lse = torch.full((10, 8), 7.0, device="cuda")
    mv.workspace[:12].view(torch.int32).fill_(SENTINEL)
    B.mla_verify_run_varlen(mv.plan, d["q_nope"], d["q_pe"], d["kv_c"], d["k_pe"], d["kv_indptr"],
                            d["kv_indices"], _dev(np.array([0, 4, 7, 6], np.int32)), d["tree_parents"],
                            x.scale, out, lse, mv.workspace)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    assert (o[4:] == 7.0).all() and (l[4:] == 7.0).all()
    r = B.MLA_VERIFY_STATUS_TREE_RANGE
    assert list(_status(mv, 3)) == [0, r, r]
    o_ref, lse_ref = run_oracle(x, nodes=[(0, t) for t in range(4)])
    compare(o[:4], l[:4], o_ref, lse_ref, "bf16")
    mv.close()


def test_packed_acceptance_tree_ending_past_the_node_arrays_is_skipped():
    import torch
    from mla_absorbed_tree_amd import binding as B

    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    parents = np.array([-1, 0, 0, 1, -1, 0], np.int32)
    draft = np.array([5, 6, 7, 8, 5, 6], np.int32)
    target = np.array([6, 8, 9, 9, 6, 9], np.int32)
    root = np.array([5, 5, 5], np.int32)
    lens = torch.full((3,), -5, dtype=torch.int32, device="cuda")
    paths = torch.full((10,), -5, dtype=torch.int32, device="cuda")
    bonus = torch.full((3,), -5, dtype=torch.int32, device="cuda")
    B.mla_tree_accept_packed(dev(parents), dev(draft), dev(target), dev(root), dev([0, 4, 7, 6]), 3, 4,
                             lens, paths, bonus)
    torch.cuda.synchronize()
    L, Pth, Bo = lens.cpu().numpy(), paths.cpu().numpy(), bonus.cpu().numpy()
    assert L[1] == -1 and L[2] == -1 and Bo[1] == 5 and Bo[2] == 5
    assert (Pth[4:] == -5).all()                # no path slot of the skipped trees is written
    assert L[0] >= 1 and (Pth[:4] != -5).all()  # sequence 0 is served normally
