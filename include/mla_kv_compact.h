/*
 * libmlaverify — KV-cache compaction for page_size = 1 pools (gfx950).
 *
 * The pages name KV-cache defragmentation as the follow-on to the verify
 * kernel, because page_size = 1 caches scatter each sequence's tokens over the
 * pool ["Reading the Reference" page, "The Context: A Pivot from Planning to
 * Execution"; "Ground Truth in Silicon" page, "Why This Message Was Written";
 * "The Information-Gathering Pivot" page, "The Context: A Multi-Phase Kernel
 * Integration", phase 4]. They give no mechanism (their two tiers are named,
 * not described). This entry point is the plainest such operation: copy every
 * sequence's slots, in logical order, into one contiguous run of a destination
 * pool and rewrite the page table to point there.
 *
 *   For every logical position i < N = kv_indptr[batch] (all sequences, in
 *   order):
 *     dst_kv_c row (dst_base + i) = kv_c row kv_indices[i]      (512 elements)
 *     dst_k_pe row (dst_base + i) = k_pe row kv_indices[i]      (64 elements)
 *     new_kv_indices[i]           = dst_base + i
 *   so sequence b occupies destination slots dst_base + kv_indptr[b] ...
 *   dst_base + kv_indptr[b+1] - 1, and (kv_indptr, new_kv_indices) describe
 *   the same cache as (kv_indptr, kv_indices). The copy is bit-exact.
 *
 * Conventions as in mla_verify.h (status codes, mla_verify_last_error(),
 * `stream` = hipStream_t as void*). Declared here, defined in libmlaverify.
 */
#ifndef MLA_KV_COMPACT_H_
#define MLA_KV_COMPACT_H_

#include <stdint.h>

#include "mla_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 *   dtype           mla_dtype of kv_c and k_pe (and of the destination)
 *   batch           number of sequences, 1..MLA_VERIFY_MAX_BATCH
 *   total_tokens    host copy of kv_indptr[batch] (sizes the launch; the
 *                   kernel copies min(total_tokens, kv_indptr[batch]) rows)
 *   kv_c, k_pe      device source pool, slot s at base + s * row_stride
 *                   elements (strides >= 512 / 64, multiples of 8; the two may
 *                   interleave in one buffer)
 *   kv_indptr       device int32 [batch + 1], kv_indptr[0] = 0, non-decreasing
 *   kv_indices      device int32 [N]: source slot of logical position i; every
 *                   entry must name a slot of the source pool (not checked)
 *   dst_kv_c, dst_k_pe  device destination pool with its own row strides;
 *                   rows dst_base .. dst_base + N - 1 are written and must not
 *                   overlap any source row that is read (no in-place moves)
 *   dst_base        first destination slot, >= 0, dst_base + total_tokens
 *                   must fit in int32
 *   new_kv_indices  device int32 [N], written (may not alias kv_indices)
 * All pointers 16-byte aligned. Asynchronous; allocates nothing, so it can be
 * captured in a HIP graph. Errors: MLA_ERR_INVALID_ARG for a bad argument
 * (nothing is launched), MLA_ERR_HIP if the launch fails.
 */
mla_status mla_kv_compact(int32_t dtype, int32_t batch, int64_t total_tokens, const void* kv_c,
                          const void* k_pe, int64_t kv_c_row_stride, int64_t k_pe_row_stride,
                          const int32_t* kv_indptr, const int32_t* kv_indices, void* dst_kv_c,
                          void* dst_k_pe, int64_t dst_kv_c_row_stride, int64_t dst_k_pe_row_stride,
                          int32_t dst_base, int32_t* new_kv_indices, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_KV_COMPACT_H_ */
