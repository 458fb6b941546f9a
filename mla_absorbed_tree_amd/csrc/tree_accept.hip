// Greedy token acceptance over verified draft trees (one tree per sequence,
// of a uniform size or packed with a size each): one 64-lane wave per tree
// with one node per lane for trees of up to 64 nodes, one 256-lane workgroup
// above that. Acceptance of a node is the AND of a local
// test (its draft token equals the target's token after its parent) over its
// ancestor-or-self set, which the shared pointer-doubling mask gives directly:
// accepted(t) = (anc(t) & ~ok) == 0.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "wave_tree.h"

namespace mlav {

// Outputs of one sequence: its accept_len / bonus slots and its path row.
struct AcceptOut {
  int32_t* len;
  int32_t* bonus;
  int32_t* path;  // T entries
};

// Trees of up to 64 nodes: one wave, one node per lane (lanes >= T idle).
__device__ __forceinline__ void wave_accept(const int32_t* __restrict__ par_b, const int32_t* __restrict__ draft_b,
                                            const int32_t* __restrict__ target_b, int root_tok, int T,
                                            const AcceptOut& o) {
  const int lane = lane_id();
  const bool live = lane < T;
  const uint64_t anc = wave_tree_mask(par_b, T);
  bool ok = false;
  if (live && anc != 0) {
    const int par = par_b[lane];
    const int want = par < 0 ? root_tok : target_b[par];
    ok = draft_b[lane] == want;
  }
  const uint64_t ok_mask = __ballot(ok);
  const bool accepted = live && anc != 0 && (anc & ~ok_mask) == 0;
  const int depth = __popcll(anc);
  // Deepest accepted node, smallest index among equals: maximise
  // depth * 64 + (63 - lane) over the wave.
  int key = accepted ? depth * 64 + (63 - lane) : -1;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) key = max(key, shfl_i32(key, lane ^ off));
  if (live) o.path[lane] = -1;
  if (key < 0) {
    if (lane == 0) {
      *o.len = 0;
      *o.bonus = root_tok;
    }
    return;
  }
  const int best = 63 - (key & 63), len = key >> 6;
  const uint64_t path = node_mask(anc, best);
  // Every node on the path writes itself at its own depth (the path holds one
  // node per depth). The -1 fill above comes first in program order on the
  // same lane, or on another lane whose slot this lane does not write.
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  if (live && ((path >> lane) & 1ull)) o.path[depth - 1] = lane;
  if (lane == 0) {
    *o.len = len;
    *o.bonus = target_b[best];
  }
}

// Trees of 65..256 nodes: thread t owns node t. The masks come from the
// workgroup builder (kMaskWords words per node, zero on an invalid chain);
// each wave's ballot of the local test is one word of the OK mask. The
// deepest accepted node wins (smallest index among equals), and every slot of
// the path row is written exactly once, from the path gathered in LDS. Every
// thread of the kMaxTreeNodes-lane workgroup must call it.
constexpr int kAcceptThreads = kMaxTreeNodes;
__device__ __forceinline__ void block_accept(const int32_t* __restrict__ par_b, const int32_t* __restrict__ draft_b,
                                             const int32_t* __restrict__ target_b, int root_tok, int T,
                                             const AcceptOut& o) {
  __shared__ __attribute__((aligned(16))) char scratch[kTreeScratchBytes];
  __shared__ uint64_t ok_words[kMaskWords];
  __shared__ int wave_key[kAcceptThreads / 64];
  __shared__ int path_lds[kMaxTreeNodes];
  const int t = threadIdx.x, wave = t >> 6;
  const bool live = t < T;
  block_tree_masks<kAcceptThreads>(par_b, T, scratch);
  const uint64_t* anc = tree_scratch_masks(scratch) + t * kMaskWords;
  uint64_t any = 0;
  int depth = 0;
  if (live) {
#pragma unroll
    for (int w = 0; w < kMaskWords; ++w) {
      any |= anc[w];
      depth += __popcll(anc[w]);
    }
  }
  bool ok = false;
  if (live && any != 0) {
    const int par = par_b[t];
    const int want = par < 0 ? root_tok : target_b[par];
    ok = draft_b[t] == want;
  }
  const uint64_t ballot = __ballot(ok);
  if ((t & 63) == 0) ok_words[wave] = ballot;
  __syncthreads();
  bool accepted = live && any != 0;
  if (accepted) {
#pragma unroll
    for (int w = 0; w < kMaskWords; ++w) accepted &= (anc[w] & ~ok_words[w]) == 0;
  }
  // Deepest accepted node, smallest index among equals: maximise
  // depth * kMaxTreeNodes + (kMaxTreeNodes - 1 - t) over the workgroup.
  int key = accepted ? depth * kMaxTreeNodes + (kMaxTreeNodes - 1 - t) : -1;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) key = max(key, shfl_i32(key, lane_id() ^ off));
  if ((t & 63) == 0) wave_key[wave] = key;
  __syncthreads();
  key = wave_key[0];
#pragma unroll
  for (int w = 1; w < kAcceptThreads / 64; ++w) key = max(key, wave_key[w]);
  const int len = key < 0 ? 0 : key / kMaxTreeNodes;
  const int best = key < 0 ? -1 : kMaxTreeNodes - 1 - key % kMaxTreeNodes;
  // The nodes of the winner's path: node u is on it iff bit u of its mask is set.
  if (best >= 0 && live) {
    const uint64_t* pm = tree_scratch_masks(scratch) + best * kMaskWords;
    if ((pm[t >> 6] >> (t & 63)) & 1ull) path_lds[depth - 1] = t;
  }
  __syncthreads();
  if (live) o.path[t] = t < len ? path_lds[t] : -1;
  if (t == 0) {
    *o.len = len;
    *o.bonus = best < 0 ? root_tok : target_b[best];
  }
}

// One workgroup per sequence. Sequence b's tree is nodes base .. base+T-1 of
// the flat arrays: base = b * T_uniform without `indptr`, else
// indptr[b] .. indptr[b+1]-1. A packed size outside 0..max_T, a negative
// offset, or a tree that ends past indptr[batch] gives accept_len = -1 and
// bonus = root_target, and writes no path.
// Launched with 64 lanes when max_T <= 64, else kAcceptThreads.
template <int kThreadsN>
__global__ void __launch_bounds__(kThreadsN) mla_tree_accept_kernel(
    const int32_t* __restrict__ parents, const int32_t* __restrict__ draft, const int32_t* __restrict__ target,
    const int32_t* __restrict__ root_target, const int32_t* __restrict__ indptr, int T_uniform, int max_T,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ accept_path, int32_t* __restrict__ bonus) {
  const int b = blockIdx.x;
  int64_t base = (int64_t)b * T_uniform;
  int T = T_uniform;
  if (indptr) {
    base = indptr[b];
    T = indptr[b + 1] - indptr[b];
  }
  const int root_tok = root_target[b];
  // The packed tree must also end inside the node arrays, which hold
  // indptr[batch] nodes.
  const bool past_end = indptr && base + T > (int64_t)indptr[gridDim.x];
  if (base < 0 || T < 0 || T > max_T || past_end) {
    if (threadIdx.x == 0) {
      accept_len[b] = -1;
      bonus[b] = root_tok;
    }
    return;
  }
  const AcceptOut o{accept_len + b, bonus + b, accept_path + base};
  if (T <= 64) {
    if (threadIdx.x < 64) wave_accept(parents + base, draft + base, target + base, root_tok, T, o);
    return;
  }
  if constexpr (kThreadsN >= kAcceptThreads) block_accept(parents + base, draft + base, target + base, root_tok, T, o);
}

int launch_tree_accept(const int32_t* parents, const int32_t* draft, const int32_t* target,
                       const int32_t* root_target, const int32_t* indptr, int32_t batch, int32_t T,
                       int32_t* accept_len, int32_t* accept_path, int32_t* bonus, void* stream) {
  const int T_uniform = indptr ? 0 : T;
  if (T <= 64)
    hipLaunchKernelGGL(mla_tree_accept_kernel<64>, dim3((unsigned)batch), dim3(64), 0, (hipStream_t)stream,
                       parents, draft, target, root_target, indptr, T_uniform, (int)T, accept_len, accept_path,
                       bonus);
  else
    hipLaunchKernelGGL(mla_tree_accept_kernel<kAcceptThreads>, dim3((unsigned)batch), dim3(kAcceptThreads), 0,
                       (hipStream_t)stream, parents, draft, target, root_target, indptr, T_uniform, (int)T,
                       accept_len, accept_path, bonus);
  return (int)hipGetLastError();
}

}  // namespace mlav
