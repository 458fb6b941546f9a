// Argument block of the KV-compaction kernel (passed by value).
#pragma once

#include <cstdint>

namespace mlav {

struct KvCompactArgs {
  const void* kv_c;              // source slot s at kv_c + s * kv_c_stride_bytes
  const void* k_pe;              // source slot s at k_pe + s * k_pe_stride_bytes
  const int32_t* kv_indptr;      // [batch + 1]
  const int32_t* kv_indices;     // [N] source slot of logical position i
  void* dst_kv_c;                // destination slot d at dst_kv_c + d * dst_kv_c_stride_bytes
  void* dst_k_pe;
  int32_t* new_indices;          // [N] = dst_base + i
  int64_t kv_c_stride_bytes, k_pe_stride_bytes;
  int64_t dst_kv_c_stride_bytes, dst_k_pe_stride_bytes;
  int64_t total;                 // host copy of kv_indptr[batch]
  int32_t batch;
  int32_t dst_base;
};

// Defined in the HIP translation unit; es = element size (2 or 4). Returns the
// launch error.
int launch_kv_compact(const KvCompactArgs& a, int es, void* stream);

}  // namespace mlav
