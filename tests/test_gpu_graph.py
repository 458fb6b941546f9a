"""mla_verify_run recorded into a HIP graph: every replay equals the eager run.

The run enqueues two kernels and nothing else (no allocation, no memset, no
host synchronisation), so it can be captured. Each replay is checked bitwise
against an eager run on the same inputs; between replays the program does its
own eager work (refilling the outputs, rewriting an input in place), so the
graph must read live data and rewrite every output element.
"""
import numpy as np
import pytest
import torch

from gen import get_config, make_inputs

pytestmark = pytest.mark.gpu


def _setup(name, tree_lens=None, **over):
    from mla_absorbed_tree_amd.verify import MlaVerify, device_inputs
    cfg = get_config(name, **over)
    x = make_inputs(cfg, tree_lens=tree_lens)
    d = device_inputs(x)
    mv = MlaVerify(cfg.batch, cfg.heads, cfg.tree_nodes, cfg.dtype, x.kv_lens, cfg.num_splits,
                   tree_lens=tree_lens)
    return cfg, x, d, mv


@pytest.mark.parametrize("name,over", [
    ("b1_h64_p4096_t16_bf16", dict(prefix=1000, batch=2)),            # split: attention + combine
    ("b1_h64_p4096_t16_bf16", dict(prefix=1000, batch=2, num_splits=1)),  # one split: attention only
    ("tiny_f32_b1_h16_p256_t8", {}),
    # packed trees of 200, 0 and 70 nodes: the workgroup mask builder, idle row blocks
    ("b1_h64_p4096_t16_bf16", dict(prefix=500, batch=3, heads=16, tree_nodes=200,
                                   tree_lens=[200, 0, 70])),
    ("tiny_f32_b1_h16_p256_t8", dict(batch=2, heads=4, tree_nodes=130, tree_lens=[130, 65])),
])
def test_graph_replays_match_eager(name, over):
    cfg, x, d, mv = _setup(name, **over)
    args = [d[k] for k in ("q_nope", "q_pe", "kv_c", "k_pe", "kv_indptr", "kv_indices", "tree_parents")]
    rows = int(x.tree_indptr[-1])
    out = torch.empty((rows, cfg.heads, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((rows, cfg.heads), dtype=torch.float32, device="cuda")

    def eager():
        o, l = mv(*args, x.scale)
        torch.cuda.synchronize()
        return o.clone(), l.clone()

    ref_o, ref_l = eager()
    assert torch.isfinite(ref_o).all() and torch.isfinite(ref_l).all()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the capture stream
        mv(*args, x.scale, out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mv(*args, x.scale, out=out, lse=lse)
    torch.cuda.synchronize()

    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), "replay %d output differs from eager" % rep
        assert torch.equal(lse, ref_l), "replay %d lse differs from eager" % rep

    # New query values written in place: the graph reads them, and matches a
    # fresh eager run on the same data.
    args[0].mul_(-1)
    args[1].mul_(-1)
    torch.cuda.synchronize()
    new_o, new_l = eager()
    assert not torch.equal(new_o, ref_o)
    out.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, new_o) and torch.equal(lse, new_l)
    del g
    mv.close()


def test_one_plan_and_graph_across_decode_steps():
    """One plan and one captured graph serve two decode steps whose lengths,
    slot tables, trees and queries change in place on the device. The second
    step's middle sequence is far shorter than planned, so 45 of its 48 splits
    get no keys (splits 0..2 keep theirs); each workgroup runs several splits
    (6 here), so empty splits also sit inside a group that has keys."""
    import dataclasses
    from gpu_util import compare, run_oracle
    from mla_absorbed_tree_amd.verify import MlaVerify, device_inputs
    cfg = get_config("b8_h64_paged600k_t16_bf16", batch=3, pool_slots=8000, seed=40)
    steps = [make_inputs(cfg, prefix_lens=np.array([1800, 1600, 2000])),
             make_inputs(dataclasses.replace(cfg, seed=41), prefix_lens=np.array([1900, 60, 2100]))]
    mv = MlaVerify(cfg.batch, cfg.heads, cfg.tree_nodes, cfg.dtype, steps[0].kv_lens, 48)
    assert 3 < mv.info["splits_per_workgroup"] < 48, mv.info
    d = device_inputs(steps[0])
    cap = max(len(x.kv_indices) for x in steps)
    idx = torch.zeros(cap, dtype=torch.int32, device="cuda")
    idx[:len(steps[0].kv_indices)] = d["kv_indices"]
    args = [d["q_nope"], d["q_pe"], d["kv_c"], d["k_pe"], d["kv_indptr"], idx, d["tree_parents"]]
    rows = cfg.batch * cfg.tree_nodes
    out = torch.empty((rows, cfg.heads, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((rows, cfg.heads), dtype=torch.float32, device="cuda")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mv(*args, steps[0].scale, out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mv(*args, steps[0].scale, out=out, lse=lse)
    torch.cuda.synchronize()

    for k, x in enumerate(steps):
        if k > 0:  # the next step's data, written in place
            nd = device_inputs(x)
            for name, t in zip(("q_nope", "q_pe", "kv_c", "k_pe", "kv_indptr"), args[:5]):
                t.copy_(nd[name])
            idx.zero_()
            idx[:len(x.kv_indices)] = nd["kv_indices"]
            args[6].copy_(nd["tree_parents"])
            torch.cuda.synchronize()
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        o_ref, lse_ref = run_oracle(x)
        compare(out.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, cfg.dtype, "step %d" % k)
        eo, el = mv(*args, x.scale)
        torch.cuda.synchronize()
        assert torch.equal(eo, out) and torch.equal(el, lse), "step %d: replay differs from eager" % k
    del g
    mv.close()
