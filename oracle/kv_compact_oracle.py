"""CPU oracle for KV-cache compaction of page_size = 1 pools.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the tests and the benchmark use it. It shares no code
with the HIP library.

The pages name KV-cache defragmentation as the next phase after the verify
kernel, to undo the scatter of page_size = 1 caches ("Reading the Reference"
page, "The Context: A Pivot from Planning to Execution"; "The
Information-Gathering Pivot" page, "The Context: A Multi-Phase Kernel
Integration", phase 4), but give no mechanism. The reading taken here is the
plainest one: every sequence's slots, in logical order, move to one contiguous
run of a destination pool, and the page table is rewritten to point there.

    dst row (dst_base + i) = src row kv_indices[i]   for every logical position i
    new_kv_indices[i]      = dst_base + i

This is a definition, so the oracle is that definition written out with numpy
indexing (a library gather).
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def kv_compact(kv_c: np.ndarray, k_pe: np.ndarray, kv_indptr: np.ndarray, kv_indices: np.ndarray,
               dst_base: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Rows of the destination run and the rewritten page table.

    Returns (rows_kv_c [N, Dl], rows_k_pe [N, Dr], new_kv_indices [N] int32),
    N = kv_indptr[-1]; row i belongs at destination slot dst_base + i.
    """
    n = int(kv_indptr[-1])
    src = np.asarray(kv_indices[:n], dtype=np.int64)
    return kv_c[src].copy(), k_pe[src].copy(), (dst_base + np.arange(n)).astype(np.int32)
