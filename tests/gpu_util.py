"""Shared helpers of the GPU tests: run the HIP path, run the oracle, compare."""
import sys

import numpy as np

from oracle import verify_attention

# Tolerances. fp32: max |do| <= 1e-4 * rms(o_ref). bf16: max |do| <= 1.5e-2 and
# mean |do| <= 2e-3 (absolute), plus a stricter internal gate on the relative
# RMS error. LSE: fp32 1e-5, bf16 1e-3 absolute.
TOL = {
    "f32": dict(max_rel_rms=1e-4, lse=1e-5),
    "bf16": dict(max_abs=1.5e-2, mean_abs=2e-3, rel_rms=5e-3, lse=1e-3),
}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_hip(x, num_splits=0, kv_c=None, k_pe=None, strides=None, device_tensors=None):
    """Run libmlaverify on inputs `x` (gen.VerifyInputs); returns numpy (o, lse, info)."""
    import torch
    from mla_absorbed_tree_amd.verify import MlaVerify, device_inputs
    d = device_tensors or device_inputs(x)
    cfg = x.cfg
    kc_stride, kp_stride = strides or (512, 64)
    ragged = x.parents.ndim == 1
    mv = MlaVerify(cfg.batch, cfg.heads, cfg.tree_nodes, cfg.dtype, x.kv_lens, num_splits,
                   kc_stride, kp_stride, tree_lens=x.tree_lens if ragged else None)
    o, lse = mv(d["q_nope"], d["q_pe"], d["kv_c"] if kv_c is None else kv_c,
                d["k_pe"] if k_pe is None else k_pe, d["kv_indptr"], d["kv_indices"],
                d["tree_parents"], x.scale)
    torch.cuda.synchronize()
    info = mv.info
    mv.close()
    return o.cpu().numpy(), lse.cpu().numpy(), info


def run_oracle(x, nodes=None):
    return verify_attention(x.q_nope, x.q_pe, x.kv_c, x.k_pe, x.kv_indptr, x.kv_indices,
                            x.parents, x.scale, nodes=nodes, tree_indptr=x.tree_indptr)


def compare(o, lse, o_ref, lse_ref, dtype, what=""):
    """Assert the HIP result matches the oracle within the dtype's tolerance."""
    assert np.isfinite(o).all(), "non-finite output " + what
    assert np.isfinite(lse).all(), "non-finite lse " + what
    d = np.abs(o.astype(np.float64) - o_ref)
    dl = np.abs(lse.astype(np.float64) - lse_ref)
    rms = np.sqrt(np.mean(o_ref ** 2))
    t = TOL[dtype]
    stats = "max|do|=%.3g mean|do|=%.3g rel_rms=%.3g rms(o)=%.3g max|dlse|=%.3g %s" % (
        d.max(), d.mean(), np.sqrt(np.mean(d ** 2)) / rms, rms, dl.max(), what)
    log("  " + stats)
    if dtype == "f32":
        assert d.max() <= t["max_rel_rms"] * rms, stats
    else:
        assert d.max() <= t["max_abs"], stats
        assert d.mean() <= t["mean_abs"], stats
        assert np.sqrt(np.mean(d ** 2)) <= t["rel_rms"] * rms, stats
    assert dl.max() <= t["lse"], stats
    return stats


def node_rows(x, nodes):
    """Packed row indices (tree_indptr[b] + t) of the given (b, t) nodes."""
    return np.array([int(x.tree_indptr[b]) + t for b, t in nodes])
