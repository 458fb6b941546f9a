"""ctypes binding of libmlaverify (argument marshalling only).

Every function here has the name of the C entry point it forwards to. Device
buffers are torch tensors (or anything with ``data_ptr()``); torch supplies
device memory and streams, all compute runs in the library's HIP kernels.
Importing this module fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmlaverify.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_WORKSPACE = -3
MLA_ERR_HIP = -4
MLA_DTYPE_F32 = 0
MLA_DTYPE_BF16 = 1
# Per-sequence status words (int32 [batch] at workspace offset 0).
MLA_VERIFY_STATUS_BAD_PARENT = 1
MLA_VERIFY_STATUS_SHORT_KV = 2
MLA_VERIFY_STATUS_TREE_RANGE = 4
MLA_VERIFY_MAX_BATCH = 65536
MLA_VERIFY_ARG_TABLE_BATCH = 256
MLA_VERIFY_MAX_TREE = 256
MLA_TREE_ACCEPT_MAX_TREE = 256

# Symbols declared in include/*.h.
EXPORTED_SYMBOLS = ("mla_verify_plan", "mla_verify_plan_get_info", "mla_verify_plan_stage_tables",
                    "mla_verify_run",
                    "mla_verify_run_varlen", "mla_verify_run_noalloc",
                    "mla_verify_attend", "mla_verify_combine",
                    "mla_verify_tree_masks", "mla_verify_plan_destroy",
                    "mla_verify_status_string", "mla_verify_last_error", "mla_kv_compact",
                    "mla_tree_accept", "mla_tree_accept_packed")


class MlaVerifyError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_status_name(status), message))
        self.status = status


class mla_verify_problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("tree_nodes", ctypes.c_int32), ("d_latent", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("kv_len_host", ctypes.POINTER(ctypes.c_int32)), ("num_splits", ctypes.c_int32),
                ("kv_c_row_stride", ctypes.c_int64), ("k_pe_row_stride", ctypes.c_int64),
                ("tree_len_host", ctypes.POINTER(ctypes.c_int32))]


class mla_verify_plan_info(ctypes.Structure):
    _fields_ = [("total_splits", ctypes.c_int32), ("max_splits", ctypes.c_int32),
                ("rows_per_block", ctypes.c_int32), ("keys_per_tile", ctypes.c_int32),
                ("grid_blocks", ctypes.c_int32), ("uses_combine", ctypes.c_int32),
                ("splits_per_workgroup", ctypes.c_int32), ("total_groups", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t), ("table_bytes", ctypes.c_size_t),
                ("partial_rows", ctypes.c_int64)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libmlaverify.so is not built (expected at %s); run "
                          "`python -m mla_absorbed_tree_amd.build_lib` or __graft_entry__.build()"
                          % _LIB_PATH)
    # One HIP runtime per process: torch wheels ship their own libamdhip64
    # (soname libamdhip64.so.7, opened by the unversioned name). Loaded first,
    # torch's copy also serves this library's libamdhip64.so.7 dependency;
    # loaded after it, torch would open a second runtime next to the one this
    # library pulled in, and launches on torch's memory would fail.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.mla_verify_plan.argtypes = [ctypes.POINTER(mla_verify_problem), ctypes.POINTER(vp),
                                    ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_verify_plan_get_info.argtypes = [vp, ctypes.POINTER(mla_verify_plan_info)]
    lib.mla_verify_plan_stage_tables.argtypes = [vp, vp, ctypes.c_size_t, vp]
    lib.mla_verify_run.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp,
                                   ctypes.c_size_t, vp]
    lib.mla_verify_attend.argtypes = lib.mla_verify_run.argtypes
    lib.mla_verify_run_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp]
    lib.mla_verify_run_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp,
                                          ctypes.c_size_t, vp]
    lib.mla_verify_combine.argtypes = [vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.mla_verify_tree_masks.argtypes = [vp, i32, i32, vp, vp]
    lib.mla_verify_plan_destroy.argtypes = [vp]
    lib.mla_kv_compact.argtypes = [i32, i32, i64, vp, vp, i64, i64, vp, vp, vp, vp, i64, i64, i32, vp, vp]
    lib.mla_tree_accept.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp, vp]
    lib.mla_tree_accept_packed.argtypes = [vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp]
    lib.mla_verify_status_string.argtypes = [i32]
    lib.mla_verify_status_string.restype = ctypes.c_char_p
    lib.mla_verify_last_error.argtypes = []
    lib.mla_verify_last_error.restype = ctypes.c_char_p
    for name in ("mla_verify_plan", "mla_verify_plan_get_info", "mla_verify_run", "mla_verify_run_varlen",
                 "mla_verify_run_noalloc",
                 "mla_verify_attend", "mla_verify_combine", "mla_verify_tree_masks",
                 "mla_verify_plan_destroy", "mla_kv_compact", "mla_tree_accept",
                 "mla_tree_accept_packed"):
        getattr(lib, name).restype = i32
    return lib


_lib = _load()


def library_path() -> str:
    return _LIB_PATH


def _status_name(status: int) -> str:
    return _lib.mla_verify_status_string(int(status)).decode()


def _check(status: int):
    if status != MLA_OK:
        raise MlaVerifyError(status, _lib.mla_verify_last_error().decode())


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def mla_verify_status_string(status: int) -> str:
    return _status_name(status)


def mla_verify_last_error() -> str:
    return _lib.mla_verify_last_error().decode()


def mla_verify_plan(batch: int, num_heads: int, tree_nodes: int, dtype: int,
                    kv_len_host: Sequence[int], num_splits: int = 0,
                    kv_c_row_stride: int = 512, k_pe_row_stride: int = 64,
                    d_latent: int = 512, d_rope: int = 64,
                    tree_len_host: Optional[Sequence[int]] = None):
    """Returns (plan handle, workspace bytes). Raises MlaVerifyError on a bad problem.

    tree_len_host: per-sequence tree sizes (packed trees), or None for
    ``tree_nodes`` nodes in every sequence."""
    i32p = ctypes.POINTER(ctypes.c_int32)
    lens = np.ascontiguousarray(np.asarray(kv_len_host, dtype=np.int32))
    tlens = None if tree_len_host is None else \
        np.ascontiguousarray(np.asarray(tree_len_host, dtype=np.int32))
    prob = mla_verify_problem(batch, num_heads, tree_nodes, d_latent, d_rope, dtype,
                              lens.ctypes.data_as(i32p), num_splits,
                              kv_c_row_stride, k_pe_row_stride,
                              None if tlens is None else tlens.ctypes.data_as(i32p))
    plan = ctypes.c_void_p()
    ws = ctypes.c_size_t()
    _check(_lib.mla_verify_plan(ctypes.byref(prob), ctypes.byref(plan), ctypes.byref(ws)))
    return plan.value, ws.value


def mla_verify_plan_get_info(plan) -> dict:
    info = mla_verify_plan_info()
    _check(_lib.mla_verify_plan_get_info(plan, ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in info._fields_}


def mla_verify_plan_destroy(plan) -> None:
    _check(_lib.mla_verify_plan_destroy(plan))


def mla_verify_plan_stage_tables(plan, tables, tables_bytes: Optional[int] = None, stream=None) -> None:
    """Copy a large batch's per-sequence tables to `tables` (device) once, before the plan's
    first run (no-op for batches whose tables fit the launch arguments)."""
    if tables_bytes is None:
        tables_bytes = 0 if tables is None else tables.numel() * tables.element_size()
    _check(_lib.mla_verify_plan_stage_tables(plan, _ptr(tables), int(tables_bytes), _stream_handle(stream)))


def mla_verify_run(plan, q_nope, q_pe, kv_c, k_pe, kv_indptr, kv_indices, tree_parents,
                   scale: float, out, lse, workspace, workspace_bytes: Optional[int] = None,
                   stream=None) -> None:
    """Enqueue one tree-verify attention on `stream` (default: torch's current stream)."""
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.mla_verify_run(plan, _ptr(q_nope), _ptr(q_pe), _ptr(kv_c), _ptr(k_pe),
                               _ptr(kv_indptr), _ptr(kv_indices), _ptr(tree_parents),
                               float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
                               int(workspace_bytes), _stream_handle(stream)))


def mla_verify_run_varlen(plan, q_nope, q_pe, kv_c, k_pe, kv_indptr, kv_indices, tree_indptr,
                          tree_parents, scale: float, out, lse, workspace,
                          workspace_bytes: Optional[int] = None, stream=None) -> None:
    """mla_verify_run with the tree packing read from the device tree_indptr [batch+1]."""
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.mla_verify_run_varlen(plan, _ptr(q_nope), _ptr(q_pe), _ptr(kv_c), _ptr(k_pe),
                                      _ptr(kv_indptr), _ptr(kv_indices), _ptr(tree_indptr),
                                      _ptr(tree_parents), float(scale), _ptr(out), _ptr(lse),
                                      _ptr(workspace), int(workspace_bytes), _stream_handle(stream)))


def mla_verify_run_noalloc(plan, q_nope, q_pe, kv_c, k_pe, kv_indptr, kv_indices, tree_parents,
                           scale: float, out, lse, stream=None) -> None:
    """mla_verify_run with the library's built-in workspace (no workspace argument)."""
    _check(_lib.mla_verify_run_noalloc(plan, _ptr(q_nope), _ptr(q_pe), _ptr(kv_c), _ptr(k_pe),
                                       _ptr(kv_indptr), _ptr(kv_indices), _ptr(tree_parents),
                                       float(scale), _ptr(out), _ptr(lse), _stream_handle(stream)))


NOALLOC_WORKSPACE_BYTES = 64 << 20


def mla_verify_attend(plan, q_nope, q_pe, kv_c, k_pe, kv_indptr, kv_indices, tree_parents,
                      scale: float, out, lse, workspace, workspace_bytes: Optional[int] = None,
                      stream=None) -> None:
    """Enqueue only the attention kernel (sequences with several split groups leave one
    partial per group in the workspace)."""
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.mla_verify_attend(plan, _ptr(q_nope), _ptr(q_pe), _ptr(kv_c), _ptr(k_pe),
                                  _ptr(kv_indptr), _ptr(kv_indices), _ptr(tree_parents),
                                  float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                  int(workspace_bytes), _stream_handle(stream)))


def mla_verify_combine(plan, out, lse, workspace, workspace_bytes: Optional[int] = None,
                       stream=None) -> None:
    """Enqueue the log-sum-exp merge of the split-group partials (no-op when no sequence
    has more than one group)."""
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.mla_verify_combine(plan, _ptr(out), _ptr(lse), _ptr(workspace),
                                   int(workspace_bytes), _stream_handle(stream)))


def mla_verify_tree_masks(tree_parents, batch: int, tree_nodes: int, masks, stream=None) -> None:
    """masks: uint64-sized device buffer [batch, tree_nodes, ceil(tree_nodes / 64)]."""
    _check(_lib.mla_verify_tree_masks(_ptr(tree_parents), int(batch), int(tree_nodes), _ptr(masks),
                                      _stream_handle(stream)))


def mla_kv_compact(dtype: int, batch: int, total_tokens: int, kv_c, k_pe, kv_c_row_stride: int,
                   k_pe_row_stride: int, kv_indptr, kv_indices, dst_kv_c, dst_k_pe,
                   dst_kv_c_row_stride: int, dst_k_pe_row_stride: int, dst_base: int,
                   new_kv_indices, stream=None) -> None:
    _check(_lib.mla_kv_compact(int(dtype), int(batch), int(total_tokens), _ptr(kv_c), _ptr(k_pe),
                               int(kv_c_row_stride), int(k_pe_row_stride), _ptr(kv_indptr),
                               _ptr(kv_indices), _ptr(dst_kv_c), _ptr(dst_k_pe),
                               int(dst_kv_c_row_stride), int(dst_k_pe_row_stride), int(dst_base),
                               _ptr(new_kv_indices), _stream_handle(stream)))


def mla_tree_accept(tree_parents, draft_tokens, target_tokens, root_targets, batch: int,
                    tree_nodes: int, accept_len, accept_path, bonus_token, stream=None) -> None:
    _check(_lib.mla_tree_accept(_ptr(tree_parents), _ptr(draft_tokens), _ptr(target_tokens),
                                _ptr(root_targets), int(batch), int(tree_nodes), _ptr(accept_len),
                                _ptr(accept_path), _ptr(bonus_token), _stream_handle(stream)))


def mla_tree_accept_packed(tree_parents, draft_tokens, target_tokens, root_targets, tree_indptr,
                           batch: int, max_tree_nodes: int, accept_len, accept_path, bonus_token,
                           stream=None) -> None:
    _check(_lib.mla_tree_accept_packed(_ptr(tree_parents), _ptr(draft_tokens), _ptr(target_tokens),
                                       _ptr(root_targets), _ptr(tree_indptr), int(batch),
                                       int(max_tree_nodes), _ptr(accept_len), _ptr(accept_path),
                                       _ptr(bonus_token), _stream_handle(stream)))
