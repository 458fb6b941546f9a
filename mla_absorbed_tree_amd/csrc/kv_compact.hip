// KV-cache compaction (page_size = 1 pools): gather each logical position's
// slot into a contiguous destination run and rewrite the page table.
//
// HBM-bound copy. One wave copies kRowsPerWave rows per step: every lane loads
// its 16-byte pieces of all those rows first and stores them afterwards, so
// several KB per wave are in flight. The page-table entries are read once per
// row with a scalar broadcast.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kv_compact_params.h"

namespace mlav {

namespace kvc {
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRowsPerWave = 4;
}  // namespace kvc

// Row bytes: kv_c 512 * es, k_pe 64 * es (es = 2 or 4), i.e. 64/128 and 8/16
// pieces of 16 bytes.
template <int kEs>
__global__ void __launch_bounds__(kvc::kThreads) mla_kv_compact_kernel(const KvCompactArgs a) {
  using namespace kvc;
  constexpr int kCPieces = 512 * kEs / 16, kPPieces = 64 * kEs / 16;
  constexpr int kCPerLane = kCPieces / 64;  // 1 or 2
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n = a.total < (int64_t)a.kv_indptr[a.batch] ? a.total : (int64_t)a.kv_indptr[a.batch];
  const int64_t step = (int64_t)gridDim.x * kWaves * kRowsPerWave;
  for (int64_t i0 = ((int64_t)blockIdx.x * kWaves + wave) * kRowsPerWave; i0 < n; i0 += step) {
    // Rows past n (the last step's tail) load row n-1 again and store nothing.
    u32x4_t c[kRowsPerWave][kCPerLane], p[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      const int64_t i = i0 + r < n ? i0 + r : n - 1;
      const int64_t src = __builtin_amdgcn_readfirstlane(a.kv_indices[i]);
      const char* sc = (const char*)a.kv_c + src * a.kv_c_stride_bytes;
#pragma unroll
      for (int k = 0; k < kCPerLane; ++k) c[r][k] = *(const u32x4_t*)(sc + 16 * (lane + 64 * k));
      p[r] = *(const u32x4_t*)((const char*)a.k_pe + src * a.k_pe_stride_bytes + 16 * (lane % kPPieces));
    }
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      if (i0 + r >= n) break;
      const int64_t d = (int64_t)a.dst_base + i0 + r;
      char* dc = (char*)a.dst_kv_c + d * a.dst_kv_c_stride_bytes;
#pragma unroll
      for (int k = 0; k < kCPerLane; ++k) *(u32x4_t*)(dc + 16 * (lane + 64 * k)) = c[r][k];
      if (lane < kPPieces) *(u32x4_t*)((char*)a.dst_k_pe + d * a.dst_k_pe_stride_bytes + 16 * lane) = p[r];
      if (lane == 0) a.new_indices[i0 + r] = (int32_t)d;
    }
  }
}

int launch_kv_compact(const KvCompactArgs& a, int es, void* stream) {
  using namespace kvc;
  // Enough workgroups to keep every CU streaming (each wave copies 4 rows per
  // step), never more than the rows need.
  const int64_t rows_per_block = (int64_t)kWaves * kRowsPerWave;
  int64_t blocks = (a.total + rows_per_block - 1) / rows_per_block;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  if (es == 2)
    hipLaunchKernelGGL(mla_kv_compact_kernel<2>, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(mla_kv_compact_kernel<4>, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace mlav
