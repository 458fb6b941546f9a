"""Plan + workspace owner around the libmlaverify C-ABI (torch for device memory)."""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import binding as B

_DTYPES = {"bf16": (B.MLA_DTYPE_BF16, torch.bfloat16), "f32": (B.MLA_DTYPE_F32, torch.float32)}


class MlaVerify:
    """One planned tree-verify problem: call it with device tensors.

    kv_lens are the host copies of N_b (prefix + tree nodes per sequence) that
    size the split schedule; the device kv_indptr passed at call time may
    describe other lengths (each still >= the sequence's tree size).
    tree_lens gives every sequence its own tree size (packed trees, each in
    0..tree_nodes); None means tree_nodes nodes everywhere.
    """

    def __init__(self, batch: int, heads: int, tree_nodes: int, dtype: str,
                 kv_lens: Sequence[int], num_splits: int = 0, kv_c_row_stride: int = 512,
                 k_pe_row_stride: int = 64, device="cuda",
                 tree_lens: Optional[Sequence[int]] = None):
        self.dtype_code, self.torch_dtype = _DTYPES[dtype]
        self.batch, self.heads, self.tree_nodes = batch, heads, tree_nodes
        self.nodes = batch * tree_nodes if tree_lens is None else int(np.sum(tree_lens))
        self.plan = None
        self.plan, self.workspace_bytes = B.mla_verify_plan(
            batch, heads, tree_nodes, self.dtype_code, kv_lens, num_splits,
            kv_c_row_stride, k_pe_row_stride, tree_len_host=tree_lens)
        self.info = B.mla_verify_plan_get_info(self.plan)
        self.workspace = torch.empty(max(self.workspace_bytes, 256), dtype=torch.uint8, device=device)
        # Batches above MLA_VERIFY_ARG_TABLE_BATCH read their per-sequence tables from device
        # memory: staged once here, on the current stream, kept alive with the plan.
        self.tables = None
        if self.info["table_bytes"] > 0:
            self.tables = torch.empty(self.info["table_bytes"] // 4, dtype=torch.int32, device=device)
            B.mla_verify_plan_stage_tables(self.plan, self.tables)

    def _check(self, q_nope, q_pe, kv_c, k_pe, int_tensors, out, lse):
        """Dtype, device and shape checks the C ABI cannot make (it sees bare
        pointers); returns (out, lse), allocated when not given."""
        rows = self.nodes
        for name, t in (("q_nope", q_nope), ("q_pe", q_pe), ("kv_c", kv_c), ("k_pe", k_pe)):
            if t.dtype != self.torch_dtype or not t.is_cuda:
                raise TypeError("%s must be a %s device tensor" % (name, self.torch_dtype))
        if tuple(q_nope.shape) != (rows, self.heads, 512) or not q_nope.is_contiguous():
            raise ValueError("q_nope must be contiguous [nodes, H, 512]")
        if tuple(q_pe.shape) != (rows, self.heads, 64) or not q_pe.is_contiguous():
            raise ValueError("q_pe must be contiguous [nodes, H, 64]")
        for name, t in int_tensors:
            if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
                raise TypeError("%s must be a contiguous int32 device tensor" % name)
        if out is None:
            out = torch.empty((rows, self.heads, 512), dtype=torch.float32, device=q_nope.device)
        elif (out.dtype != torch.float32 or not out.is_cuda or not out.is_contiguous()
              or tuple(out.shape) != (rows, self.heads, 512)):
            raise ValueError("out must be a contiguous float32 device tensor [nodes, H, 512]")
        if lse is None:
            lse = torch.empty((rows, self.heads), dtype=torch.float32, device=q_nope.device)
        elif (lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous()
              or tuple(lse.shape) != (rows, self.heads)):
            raise ValueError("lse must be a contiguous float32 device tensor [nodes, H]")
        return out, lse

    def __call__(self, q_nope, q_pe, kv_c, k_pe, kv_indptr, kv_indices, tree_parents, scale,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 stream=None):
        out, lse = self._check(q_nope, q_pe, kv_c, k_pe, (("kv_indptr", kv_indptr), ("kv_indices", kv_indices),
                                                          ("tree_parents", tree_parents)), out, lse)
        B.mla_verify_run(self.plan, q_nope, q_pe, kv_c, k_pe, kv_indptr, kv_indices, tree_parents,
                         scale, out, lse, self.workspace, self.workspace.numel(), stream)
        return out, lse

    def varlen(self, q_nope, q_pe, kv_c, k_pe, kv_indptr, kv_indices, tree_indptr, tree_parents, scale,
               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, stream=None):
        """mla_verify_run_varlen: the tree packing is read from the device
        tree_indptr [batch+1] at run time, each size within the plan's. The
        buffers hold the plan's node total, which bounds tree_indptr[batch]
        when tree_indptr[0] = 0; rows past tree_indptr[batch] are not written."""
        out, lse = self._check(q_nope, q_pe, kv_c, k_pe, (("kv_indptr", kv_indptr), ("kv_indices", kv_indices),
                                                          ("tree_indptr", tree_indptr),
                                                          ("tree_parents", tree_parents)), out, lse)
        B.mla_verify_run_varlen(self.plan, q_nope, q_pe, kv_c, k_pe, kv_indptr, kv_indices, tree_indptr,
                                tree_parents, scale, out, lse, self.workspace, self.workspace.numel(), stream)
        return out, lse

    def status(self) -> torch.Tensor:
        """The per-sequence status words of the last run (int32 [batch],
        MLA_VERIFY_STATUS_* bits, 0 = valid): a view of the workspace, so
        synchronise the run's stream before reading it on the host."""
        return self.workspace[: 4 * self.batch].view(torch.int32)

    def close(self):
        if self.plan is not None:
            B.mla_verify_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def device_inputs(x, device="cuda"):
    """Copy a seeded input set (numpy arrays, bf16-exact float32 for bf16
    workloads) to the device in its storage dtype. Returns a dict of tensors."""
    dt = torch.bfloat16 if x.cfg.dtype == "bf16" else torch.float32

    def fl(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device=device).to(dt)

    def it(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device=device)

    return dict(q_nope=fl(x.q_nope), q_pe=fl(x.q_pe), kv_c=fl(x.kv_c), k_pe=fl(x.k_pe),
                kv_indptr=it(x.kv_indptr), kv_indices=it(x.kv_indices), tree_parents=it(x.parents))
