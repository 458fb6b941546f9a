// Tree helpers shared by the kernels: lane index, lane shuffles, the
// ancestor-or-self bitmask of every node of a tree of at most 64 nodes (one
// node per lane of a 64-lane wave), and the multi-word masks of trees of up to
// 256 nodes built by a whole workgroup.
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

// Trees of up to kMaxTreeNodes nodes: node t's ancestor-or-self set is
// kMaskWords 64-bit words, bit u % 64 of word u / 64 standing for node u.
constexpr int kMaxTreeNodes = 256;
constexpr int kMaskWords = kMaxTreeNodes / 64;
// LDS scratch of block_tree_masks: the masks, then parent pointers and
// invalid-chain flags.
constexpr int kTreeScratchBytes = kMaxTreeNodes * (kMaskWords * 8 + 2 * 4);

// Ancestor-or-self masks of every node of a tree of T <= kMaxTreeNodes nodes,
// built by the kThreadsN threads of the workgroup by pointer doubling in LDS
// (`scratch`, kTreeScratchBytes, 8-byte aligned): each node keeps the OR of
// the masks of the nodes between it and its current pointer, and each round
// merges the pointed-to node's range and doubles the pointer's reach, so
// ceil(log2 T) rounds cover the deepest chain. A node whose root path holds an
// invalid parent (>= its node, or < -1) ends with an all-zero mask. On return
// (after a barrier) node t's words are at tree_scratch_masks(scratch) +
// t * kMaskWords. Every thread of the workgroup must call it, with the same T.
__device__ __forceinline__ uint64_t* tree_scratch_masks(char* scratch) { return (uint64_t*)scratch; }

template <int kThreadsN>
__device__ __forceinline__ void block_tree_masks(const int32_t* __restrict__ parents_b, int T, char* scratch) {
  constexpr int kPer = (kMaxTreeNodes + kThreadsN - 1) / kThreadsN;
  uint64_t* const msk = tree_scratch_masks(scratch);
  int* const ptr = (int*)(msk + kMaxTreeNodes * kMaskWords);
  int* const bad = ptr + kMaxTreeNodes;
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int t = tid + k * kThreadsN;
    if (t < T) {
      const int p = parents_b[t];
      const int bd = (p < -1 || p >= t) ? 1 : 0;
      ptr[t] = bd ? -1 : p;
      bad[t] = bd;
#pragma unroll
      for (int w = 0; w < kMaskWords; ++w) msk[t * kMaskWords + w] = w == (t >> 6) ? 1ull << (t & 63) : 0ull;
    }
  }
  __syncthreads();
  for (int reach = 1; reach < T; reach <<= 1) {
    uint64_t m[kPer][kMaskWords];
    int np[kPer], nb[kPer];
    bool act[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int t = tid + k * kThreadsN;
      const int p = t < T ? ptr[t] : -1;
      act[k] = p >= 0;
      np[k] = -1;
      nb[k] = 0;
#pragma unroll
      for (int w = 0; w < kMaskWords; ++w) m[k][w] = 0ull;
      if (act[k]) {
#pragma unroll
        for (int w = 0; w < kMaskWords; ++w) m[k][w] = msk[p * kMaskWords + w];
        np[k] = ptr[p];
        nb[k] = bad[p];
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int t = tid + k * kThreadsN;
      if (act[k]) {
#pragma unroll
        for (int w = 0; w < kMaskWords; ++w) msk[t * kMaskWords + w] |= m[k][w];
        ptr[t] = np[k];
        bad[t] |= nb[k];
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int t = tid + k * kThreadsN;
    if (t < T && bad[t]) {
#pragma unroll
      for (int w = 0; w < kMaskWords; ++w) msk[t * kMaskWords + w] = 0ull;
    }
  }
  __syncthreads();
}

// Bits u0 .. u0+31 of a multi-word node mask (bit i of the result = node
// u0 + i), given the word holding bit max(u0, 0) (`lo`) and the next word
// (`hi`, 0 past the last). Bits for u < 0 are 0.
__device__ __forceinline__ uint32_t mask_window(int u0, uint64_t lo, uint64_t hi) {
  if (u0 <= -32) return 0u;
  if (u0 < 0) return (uint32_t)(lo << (-u0));
  const int sh = u0 & 63;
  return (uint32_t)(sh == 0 ? lo : (lo >> sh) | (hi << (64 - sh)));
}

}  // namespace mlav
