"""GPU tests of the MlaVerify wrapper: its argument checks, the varlen call
and the status words it exposes."""
import numpy as np
import pytest

from gen import get_config, make_inputs
from gpu_util import compare, log, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_absorbed_tree_amd.binding  # noqa: F401  (fails loudly if the library is missing)


def _setup(tree_lens=(5, 0, 9)):
    from mla_absorbed_tree_amd.verify import MlaVerify, device_inputs
    cfg = get_config("b1_h64_p4096_t16_bf16", batch=len(tree_lens), heads=8, tree_nodes=max(tree_lens),
                     prefix=300, seed=91)
    x = make_inputs(cfg, tree_lens=np.array(tree_lens))
    d = device_inputs(x)
    mv = MlaVerify(cfg.batch, cfg.heads, cfg.tree_nodes, cfg.dtype, x.kv_lens, 3, tree_lens=x.tree_lens)
    args = (d["q_nope"], d["q_pe"], d["kv_c"], d["k_pe"], d["kv_indptr"], d["kv_indices"], d["tree_parents"])
    return cfg, x, d, mv, args


def test_wrapper_rejects_output_buffers_of_the_wrong_shape_or_type():
    """The C ABI sees bare pointers, so a short out or lse buffer would be
    written past its end; the wrapper checks them before the launch."""
    import torch
    cfg, x, d, mv, args = _setup()
    rows = int(x.tree_indptr[-1])
    bad_out = [torch.empty((rows - 1, cfg.heads, 512), dtype=torch.float32, device="cuda"),
               torch.empty((rows, cfg.heads, 512), dtype=torch.bfloat16, device="cuda"),
               torch.empty((rows, cfg.heads, 1024), dtype=torch.float32, device="cuda")[..., :512]]
    for out in bad_out:
        with pytest.raises(ValueError):
            mv(*args, x.scale, out=out)
    with pytest.raises(ValueError):
        mv(*args, x.scale, lse=torch.empty((rows, cfg.heads + 1), dtype=torch.float32, device="cuda"))
    with pytest.raises(TypeError):
        mv(args[0].float(), *args[1:], x.scale)
    mv.close()


def test_wrapper_varlen_equals_run_and_reports_status():
    """MlaVerify.varlen with the plan's own packing on the device gives the
    run's result bit for bit; status() reads 0 for valid trees and the
    bad-parent bit for a sequence whose parent entry is out of range."""
    import torch
    from mla_absorbed_tree_amd import binding as B
    cfg, x, d, mv, args = _setup()
    o1, l1 = mv(*args, x.scale)
    torch.cuda.synchronize()
    assert mv.status().cpu().tolist() == [0, 0, 0]
    tree_indptr = torch.from_numpy(x.tree_indptr.astype(np.int32)).cuda()
    o2, l2 = mv.varlen(*args[:6], tree_indptr, args[6], x.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, lse_ref = run_oracle(x)
    compare(o1.cpu().numpy(), l1.cpu().numpy(), o_ref, lse_ref, cfg.dtype, "plan=%s" % mv.info)
    # sequence 2 (nodes 5..13): node 3 of its tree points forward
    parents = x.parents.copy()
    parents[int(x.tree_indptr[2]) + 3] = 7
    mv(*args[:6], torch.from_numpy(parents.astype(np.int32)).cuda(), x.scale)
    torch.cuda.synchronize()
    st = mv.status().cpu().tolist()
    log("status after a bad parent: %s" % st)
    assert st[0] == 0 and st[1] == 0 and st[2] & B.MLA_VERIFY_STATUS_BAD_PARENT
    mv.close()
