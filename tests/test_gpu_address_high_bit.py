"""GPU regression test: kv_c rows whose 64-bit addresses have the top bit of
their low 32-bit word set (and others clear). A build of the gather once
rebuilt a row address from two 32-bit halves and sign-extended the low one,
which sent such rows to a wrong page; this runs the paged layout with the
cache pool placed inside a larger allocation so that its used rows fall on
both sides of that bit, and checks every output against the float64 oracle.
"""
import numpy as np
import pytest

from gen import get_config, make_inputs
from gpu_util import compare, log, run_hip, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_absorbed_tree_amd.binding  # noqa: F401


def test_rows_on_both_sides_of_address_bit_31():
    import torch
    from mla_absorbed_tree_amd.verify import device_inputs

    cfg = get_config("b8_h64_paged600k_t16_bf16", batch=3, heads=16, prefix_range=(3000, 6000), seed=67)
    x = make_inputs(cfg)
    slots = cfg.pool_slots
    c_bytes, p_bytes = slots * 512 * 2, slots * 64 * 2
    big = torch.empty((1 << 32) + c_bytes + p_bytes + 4096, dtype=torch.uint8, device="cuda")
    base = big.data_ptr()
    # kv_c starts where the low word of the address is 2^31 - c_bytes / 2, so
    # the pool's rows straddle bit 31 of the low word.
    target = ((1 << 31) - c_bytes // 2) & ~255
    off_c = (target - base) % (1 << 32)
    off_p = (off_c + c_bytes + 255) & ~255
    kv_c = big[off_c:off_c + c_bytes].view(torch.bfloat16).view(slots, 512)
    k_pe = big[off_p:off_p + p_bytes].view(torch.bfloat16).view(slots, 64)
    d = device_inputs(x)
    kv_c.copy_(d["kv_c"])
    k_pe.copy_(d["k_pe"])
    used = np.asarray(x.kv_indices, dtype=np.int64)
    low = (kv_c.data_ptr() + used * 1024) & 0xFFFFFFFF
    assert (low >= (1 << 31)).any() and (low < (1 << 31)).any()
    log("  kv_c at %#x: %d used rows with bit 31 of the low word set, %d clear"
        % (kv_c.data_ptr(), int((low >= (1 << 31)).sum()), int((low < (1 << 31)).sum())))
    del d["kv_c"], d["k_pe"]
    o, lse, info = run_hip(x, 0, kv_c=kv_c, k_pe=k_pe, device_tensors=d)
    o_ref, lse_ref = run_oracle(x)
    compare(o, lse, o_ref, lse_ref, "bf16", "plan=%s" % info)
    del big
    torch.cuda.empty_cache()
