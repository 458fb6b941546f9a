// Wave-level helpers shared by the kernels: lane index, lane shuffles and the
// ancestor-or-self bitmask of every node of a tree of at most 64 nodes (one
// node per lane of a 64-lane wave).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace mlav {

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ int shfl_i32(int v, int src_lane) {
  return __builtin_amdgcn_ds_bpermute(src_lane << 2, v);
}

// Ancestor-or-self mask of tree node `lane` (lanes >= T return 0), by pointer
// doubling over the parent array: after r rounds a node has OR-ed the masks of
// the 2^r nearest nodes on its root path; 6 rounds cover a 64-deep chain.
// A node whose root path holds an invalid parent (>= its node, or < -1) gets 0.
// Every lane of the wave must execute this.
__device__ __forceinline__ uint64_t wave_tree_mask(const int32_t* __restrict__ parents_b, int T) {
  const int lane = lane_id();
  const bool live = lane < T;
  const int par = live ? parents_b[lane] : -1;
  int bad = (live && (par < -1 || par >= lane)) ? 1 : 0;
  int ptr = bad ? -1 : par;
  uint32_t lo = (live && lane < 32) ? (1u << lane) : 0u;
  uint32_t hi = (live && lane >= 32) ? (1u << (lane - 32)) : 0u;
#pragma unroll
  for (int r = 0; r < 6; ++r) {
    const int src = ptr >= 0 ? ptr : lane;
    const uint32_t slo = (uint32_t)shfl_i32((int)lo, src);
    const uint32_t shi = (uint32_t)shfl_i32((int)hi, src);
    const int sptr = shfl_i32(ptr, src);
    const int sbad = shfl_i32(bad, src);
    if (ptr >= 0) {
      lo |= slo;
      hi |= shi;
      bad |= sbad;
      ptr = sptr;
    }
  }
  return bad ? 0ull : ((uint64_t)hi << 32) | lo;
}

// Mask of `node` fetched from the lane that built it.
__device__ __forceinline__ uint64_t node_mask(uint64_t tmask, int node) {
  const uint32_t lo = (uint32_t)shfl_i32((int)(uint32_t)tmask, node);
  const uint32_t hi = (uint32_t)shfl_i32((int)(uint32_t)(tmask >> 32), node);
  return ((uint64_t)hi << 32) | lo;
}

}  // namespace mlav
