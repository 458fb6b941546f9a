// Tree-verify attention for absorbed-form MLA on gfx950 (MI355X).
//
// Per query row (b, t, h): score(j) = scale * (q_nope . kv_c[j] + q_pe . k_pe[j])
// over the prefix and the node's ancestor-or-self tree tail, softmax, then the
// weighted sum of kv_c (latent-space output) and the log-sum-exp.
//
// Work decomposition: one workgroup per (sequence b, block of query rows,
// group of consecutive KV splits). Every key tile (kv_c | k_pe) is staged in
// LDS once and serves all query rows of the block, so the head-shared latent
// is read from L2 once per block instead of once per head. A workgroup with
// several splits streams their tiles through one pipeline against one
// reference max, so merging their (m, l, O) is a plain sum, done in the
// accumulators; it writes one partial for the group.
//
// bf16 kernel: 4 waves (one per SIMD), 128 query rows, 32-key tiles.
//   * A 3-deep LDS ring of key tiles is filled by global_load_lds_dwordx4
//     (global -> LDS without registers); the loads of tile t+2 go out while
//     tiles t and t+1 are computed on. Page-table entries travel the same
//     way, eight tiles per load.
//   * QK: wave w owns query rows 32w..32w+31 and keeps the latent 512
//     features of their Q in VGPRs (the rope 64 in LDS). S^T[32 keys x 32
//     rows] = K . Q^T with 36 mfma_f32_32x32x16_bf16 whose accumulator stays
//     in VGPRs.
//   * Softmax weights in fp32 (exp2 domain) against a per-row reference max,
//     computed by the row's own wave and spread between the MFMAs of the
//     next tile's PV; rounded to bf16 as the P^T operand.
//   * PV: waves 2i and 2i+1 form a pair; wave w accumulates feature half w%2
//     (256 features) of O^T for its own 32 rows and for its partner's, so
//     each V^T fragment (two ds_read_b64_tr_b16) feeds two MFMAs. The
//     partner's P^T arrives through LDS (2 KB per wave and tile).
//   * O^T lives in the 256 accumulation registers of each lane.
// One wave streams about one LDS read per 24 cycles whatever its width
// (measured), so the number of operand reads per MFMA matters more than LDS
// bandwidth: 36 K + 4 rope-Q + 32 V^T + 2 P^T reads per wave and tile
// against 68 MFMAs of 32 cycles.
// The key order inside each 16-deep MFMA step is permuted consistently in P^T
// and V^T so that P^T comes straight from the S^T accumulator layout.
//
// fp32 kernel (parity workloads stored in fp32): 1 wave, 32 rows, one LDS tile,
// mfma_f32_32x32x2_f32, Q staged in LDS; same softmax and epilogue rules.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>
#include <utility>

#include "kernel_params.h"
#include "wave_tree.h"
#include "plan.h"

namespace mlav {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Two floats rounded to fp16 (nearest even), the first in the low half.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)lo, (_Float16)hi});
}

typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void global_void_t;

constexpr float kLn2 = 0.693147180559945309f;
// Largest excess (log2 units) of a score over the row's reference max that a
// pass accepts: weights stay below 2^64, far from fp32/bf16 overflow even when
// summed over millions of keys.
constexpr float kOverflowSlack = 64.f;

__device__ __forceinline__ float shfl_f32(float v, int src_lane) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(v)));
}
// Value of lane i ^ 32: one v_permlane32_swap (lanes i and i + 32 trade
// registers; measured layout: lane i < 32 finds lane i + 32's first operand
// in the second result, lane i + 32 finds lane i's second operand in the
// first), no LDS round trip.
__device__ __forceinline__ float swap_halves(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, lane_id() < 32 ? r[1] : r[0]);
}

// s_waitcnt with only the vector-memory counter bounded (<= N outstanding).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// s_waitcnt lgkmcnt(0): this wave's LDS reads/writes are complete.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }
// Workgroup barrier without the memory fence of __syncthreads (which would
// also drain every outstanding global->LDS load). Callers wait for exactly the
// counters they need first.
__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// f(std::integral_constant<int, I>) for I = 0..N-1, as straight-line code:
// every index is a compile-time constant, whatever the size of the body.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Ancestor masks of sequence blockIdx.x's tree, masks[(b*T + t) * W + w] with
// W = ceil(T / 64): the one-wave builder for T <= 64 (the first wave), the
// workgroup builder above, as in the attention kernels.
constexpr int kTreeMaskThreads = 256;
__global__ void __launch_bounds__(kTreeMaskThreads) mla_tree_masks_kernel(const int32_t* __restrict__ parents,
                                                                          int T, uint64_t* __restrict__ masks) {
  __shared__ __attribute__((aligned(16))) char scratch[kTreeScratchBytes];
  const int b = blockIdx.x;
  const int32_t* par = parents + (int64_t)b * T;
  if (T <= 64) {
    if (threadIdx.x >= 64) return;
    const uint64_t m = wave_tree_mask(par, T);
    if (lane_id() < T) masks[(int64_t)b * T + lane_id()] = m;
    return;
  }
  const int W = (T + 63) >> 6;
  block_tree_masks<kTreeMaskThreads>(par, T, scratch);
  const uint64_t* msk = tree_scratch_masks(scratch);
  for (int i = threadIdx.x; i < T * W; i += kTreeMaskThreads)
    masks[(int64_t)b * T * W + i] = msk[(i / W) * kMaskWords + i % W];
}

// ---------------------------------------------------------------------------
// Workgroup -> (sequence, group of consecutive KV splits, row block),
// XCD-aware. Consecutive workgroup ids are dealt to different XCDs; every row
// block of one split group gets the same XCD so its keys stream through a
// single L2. A workgroup runs the splits of its group one after the other as
// one stream of key tiles (the splits of a sequence are adjacent), writing a
// partial result at the end of each.
// ---------------------------------------------------------------------------
struct BlockWork {
  int b, S, rb;
  int T, rows, node0;         // tree nodes of the sequence, T * H, its first packed node
  int s;                      // the group's first split (index within the sequence)
  int s_last;                 // one past the group's last split (within the sequence)
  int G, part;                // split groups of the sequence; global index of this group's partial
  int kv0, N, P, ntiles;
  int tile_begin, tile_end;   // key tiles of the whole group
  bool seq_ok;
  int tree_status;            // MLA_VERIFY_STATUS_TREE_RANGE or 0 (seq_tree)
};

// First key tile of split s of a sequence with ntiles tiles and S splits.
__device__ __forceinline__ int split_tile(int s, int ntiles, int S) { return (int)(((int64_t)s * ntiles) / S); }

// First packed node and size of sequence b's tree: the plan's packing, or the
// device offsets of a run that reads them. Device entries out of range (a size
// outside 0..the planned size, a negative offset, or a tree ending past
// tree_indptr[batch]) give an empty tree, so the sequence is skipped, and
// return MLA_VERIFY_STATUS_TREE_RANGE; otherwise 0.
// Per-sequence tables: from the argument block, or from device memory for
// batches above MLA_VERIFY_ARG_TABLE_BATCH.
// Every index is wave-uniform and the device tables are never written during
// a launch, so they are read through the constant address space: scalar
// loads, whose results stay in scalar registers like the argument block's.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
__device__ __forceinline__ int table_entry(const VerifyArgs& a, int t, int i) {
  return ((const_i32_ptr)(uintptr_t)a.dev_tables)[t * (a.batch + 1) + i];
}
__device__ __forceinline__ int split_off(const VerifyArgs& a, int i) {
  if (a.dev_tables) return table_entry(a, 0, i);
  return a.split_offset[i];
}
__device__ __forceinline__ int group_off(const VerifyArgs& a, int i) {
  if (a.dev_tables) return table_entry(a, 1, i);
  return a.group_offset[i];
}
__device__ __forceinline__ int node_off(const VerifyArgs& a, int i) {
  if (a.dev_tables) return table_entry(a, 2, i);
  return a.node_offset[i];
}

__device__ __forceinline__ int seq_tree(const VerifyArgs& a, int b, int& node0, int& T) {
  node0 = node_off(a, b);
  T = node_off(a, b + 1) - node0;
  if (a.tree_indptr) {
    const int cap = T;
    node0 = a.tree_indptr[b];
    T = a.tree_indptr[b + 1] - node0;
    const int64_t total = a.tree_indptr[a.batch];
    if (node0 < 0 || T < 0 || T > cap || (int64_t)node0 + T > total) {
      T = 0;
      return MLA_VERIFY_STATUS_TREE_RANGE;
    }
  }
  return 0;
}

// Fills w for this workgroup. Returns false past the last split group (no
// work at all). A row block past its sequence's T_b * H rows (row blocks are
// counted for the largest tree) is still mapped; the caller checks w.rows.
__device__ __forceinline__ bool map_block(const VerifyArgs& a, BlockWork& w) {
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds;
  const int local = bid / kXcds;
  w.rb = local % a.row_blocks;
  const int cg = (local / a.row_blocks) * kXcds + xcd;
  if (cg >= group_off(a, a.batch)) return false;
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (group_off(a, mid) <= cg) lo = mid;
    else hi = mid - 1;
  }
  w.b = lo;
  w.tree_status = seq_tree(a, w.b, w.node0, w.T);
  w.rows = w.T * a.heads;
  w.S = split_off(a, w.b + 1) - split_off(a, w.b);
  w.s = (cg - group_off(a, w.b)) * a.group;
  w.s_last = min(w.s + a.group, w.S);
  w.G = group_off(a, w.b + 1) - group_off(a, w.b);
  w.part = cg;
  w.kv0 = a.kv_indptr[w.b];
  w.N = a.kv_indptr[w.b + 1] - w.kv0;
  w.P = w.N - w.T;
  w.seq_ok = w.P >= 0;
  w.ntiles = w.seq_ok ? (w.N + kKeysPerTile - 1) / kKeysPerTile : 0;
  w.tile_begin = split_tile(w.s, w.ntiles, w.S);
  w.tile_end = split_tile(w.s_last, w.ntiles, w.S);
  return true;
}

// The per-sequence status words of the run (one int32 per sequence, written
// by every run): the workgroup of a sequence's first split group and first row
// block writes its word, and also the words of the neighbouring sequences that
// have no workgroup at all (planned with an empty tree), up to the previous
// sequence with one and, for the last such sequence, to the end of the batch.
// Bits: MLA_VERIFY_STATUS_BAD_PARENT when some node's parent is not in
// -1..node-1 (the rows of every node whose ancestor chain meets it are NaN);
// MLA_VERIFY_STATUS_SHORT_KV when N_b < T_b (every row is NaN);
// MLA_VERIFY_STATUS_TREE_RANGE when the device tree entries are out of range
// (no row of the sequence is written). Every thread of the workgroup calls it.
template <int kThreadsN>
__device__ void write_status(const VerifyArgs& a, const BlockWork& w) {
  if (!(w.rb == 0 && w.s == 0)) return;  // uniform over the workgroup
  int bad = 0;
  for (int t = threadIdx.x; t < w.T; t += kThreadsN) {
    const int p = a.parents[w.node0 + t];
    bad |= (p < -1 || p >= t) ? 1 : 0;
  }
  bad = __syncthreads_or(bad);
  if (threadIdx.x != 0) return;
  a.status[w.b] = w.tree_status | (bad ? MLA_VERIFY_STATUS_BAD_PARENT : 0) |
                  (w.P < 0 ? MLA_VERIFY_STATUS_SHORT_KV : 0);
  // Sequences without a split group hold no tree node in the plan; with
  // device tree offsets, one that claims nodes is out of range.
  auto empty_status = [&](int b2) {
    int n0, t2;
    return seq_tree(a, b2, n0, t2);
  };
  for (int b2 = w.b - 1; b2 >= 0 && split_off(a, b2 + 1) == split_off(a, b2); --b2) a.status[b2] = empty_status(b2);
  if (split_off(a, w.b + 1) == split_off(a, a.batch))
    for (int b2 = w.b + 1; b2 < a.batch; ++b2) a.status[b2] = empty_status(b2);
}

// Masks and scales the 16 scores this lane holds in an S^T block and returns
// the row max over the 32 keys. Register i holds key k0 + (i/4)*8 + 4*half +
// i%4. Prefix keys are visible; tail key P+u iff node u is in the row's
// ancestor mask, whose bits for the tile's keys k0..k0+31 are `win`
// (mask_window at u0 = k0 - P); keys >= N are padding.
__device__ __forceinline__ float mask_scale_max(float (&sv)[16], const f32x16_t& sacc, float scale_log2,
                                                int k0, int half, int P, int N, uint32_t win) {
  const bool no_mask = k0 + kKeysPerTile <= P;
  const uint32_t hwin = win >> (4 * half);
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int j = k0 + (i >> 2) * 8 + half * 4 + (i & 3);
    const bool tail_bit = ((hwin >> ((i >> 2) * 8 + (i & 3))) & 1u) != 0;
    const bool vis = no_mask | (j < P) | ((j < N) & tail_bit);
    sv[i] = vis ? sacc[i] * scale_log2 : -INFINITY;
    mx = fmaxf(mx, sv[i]);
  }
  return fmaxf(mx, swap_halves(mx));
}

// ===========================================================================
// bf16 kernel
// ===========================================================================
namespace bf16k {
constexpr int kThreads = 256;
constexpr int kRows = 128;
constexpr int kNbuf = 3;                        // LDS ring of key tiles
// The kv_c part of a tile: wave w's 8 keys (8w..8w+7) fill region w, eight
// 1 KB blocks and a 128 B pad. Block j holds 16-byte chunks 8j..8j+7
// (features 64j..64j+63) of the 8 keys, ordered [chunk c % 8][key slot], and
// key r sits in slot r ^ 4 when (c % 8) / 2 is odd. Every load of a tile
// then takes its address per lane (lane i: chunk i/8 of key slot i%8, no
// row address to broadcast), and both read patterns are conflict-free: a QK
// operand read (16 keys, one chunk) covers 2 x 128 contiguous bytes in two
// regions 128 bytes apart (mod 256), and a PV transpose read (4 keys x 16
// features per 16 lanes) puts the two 16-lane groups of a half-wave on
// disjoint banks through the key-slot swizzle.
constexpr int kRegion = 8 * 1024 + 128;
constexpr int kCBytes = 4 * kRegion;           // kv_c part of a tile
constexpr int kPeRow = kDr * 2;                 // 128 B, 16-byte chunks XOR-swizzled by key
constexpr int kBufBytes = kCBytes + kKeysPerTile * kPeRow;  // 37376
__host__ __device__ constexpr int kvc_swizzle(int chunk_in_block) { return ((chunk_in_block >> 1) & 1) << 2; }
// Page-table entries travel global -> LDS too, in batches of kIdxBatch tiles
// (tiles 8B..8B+7, one 64-lane load per wave: its 8 keys of each tile) into
// a per-wave ring of two batches; batch B goes out in the iteration of tile
// 8B - kIdxLead, at least one iteration before the addresses of its first
// tile's loads are prepared (tile t+3 in iteration t).
constexpr int kIdxBatch = 8;
constexpr int kIdxLead = 4;
constexpr int kIdxWaveBytes = 2 * kIdxBatch * 8 * 4;          // 512 per wave
constexpr int kIdxBytes = 4 * kIdxWaveBytes;                  // 2048
constexpr int kAncBytes = kRows * kMaskWords * 8;             // ancestor mask words of each row
// The rope part of Q (64 features of each row) as each lane's four MFMA
// operand fragments, [wave][fragment][lane] x 16 bytes.
constexpr int kQpeBytes = kRows * kDr * 2;                     // 16384

// The P^T fragments of a tile pass between the two waves of a pair (waves
// 2i and 2i+1) through LDS: [tile parity][wave][key step][lane] x 16 bytes.
constexpr int kPxWaveBytes = 2 * 64 * 16;
constexpr int kPxBytes = 2 * 4 * kPxWaveBytes;                // 16384
// Row sums exchanged for the final normalisation, one float per row.
constexpr int kLxBytes = kRows * 4;
constexpr int kSmem = kNbuf * kBufBytes + kIdxBytes + kAncBytes + kQpeBytes + kPxBytes + kLxBytes;
static_assert(kSmem <= 160 * 1024, "LDS budget");
// Trees above 64 nodes build their masks in the ring buffer of the third
// tile, which is first loaded after the pipeline's first barrier.
static_assert(kTreeScratchBytes <= kBufBytes, "tree mask scratch");

// One pipeline iteration (tile t in LDS for PV, tile t+1 for QK) issues 68
// MFMAs. PV is split between the two waves of a pair by output features:
// wave w keeps O^T of feature half w%2 (256 features) for its own 32 rows
// and for its partner's, so each V^T fragment (two transpose reads) feeds two
// MFMAs: one with this wave's weights P^T, one with the partner's, read from
// LDS after the barrier. PV operand p (0..15) is key step p/8 (16 keys) of
// feature block p%8 of the half. Order: own-row PV of operands 0..2 (their
// V^T read before the barrier), partner-row PV of the same operands (the
// partner's P^T has arrived by then), the 36 QK MFMAs of tile t+1 (4 rope,
// 32 latent chunks), then own and partner PV of operands 3..15, beside which
// the softmax of tile t+1 runs.
constexpr int kPvHead = 3;               // operands whose MFMAs open the iteration
constexpr int kQkOps = 36;
constexpr int kPvOps = 32;
constexpr int kOps = kQkOps + kPvOps;
constexpr int kQk0 = 2 * kPvHead;        // slot of the first QK MFMA
struct Op {
  bool pv;
  bool partner;  // PV: the partner's rows
  int p;         // PV: operand (key step p/8, feature block p%8 of the half)
  int c;         // QK: 0..3 rope chunks, 4..35 latent chunks 0..31
  int r;         // operand read (fragment) this MFMA consumes
};
__host__ __device__ constexpr Op iter_op(int j) {
  if (j < kPvHead) return Op{true, false, j, 0, j};
  if (j < kQk0) return Op{true, true, j - kPvHead, 0, j - kPvHead};
  if (j < kQk0 + kQkOps) return Op{false, false, 0, j - kQk0, kPvHead + j - kQk0};
  const int i = j - kQk0 - kQkOps;  // 0..25: operands kPvHead.., own then partner
  return Op{true, (i & 1) != 0, kPvHead + (i >> 1), 0, kPvHead + kQkOps + (i >> 1)};
}
// Operand reads: kReads fragments per iteration, read r going to ring entry
// r % kRing. Read r is issued kAhead reads ahead of its first use, but not
// before the last use of the ring entry's previous fragment; reads 0..kPvHead-1
// (V^T of tile t) before the barrier, the QK reads (tile t+1) after it.
constexpr int kReads = kPvHead + kQkOps + (kPvOps / 2 - kPvHead);  // 52
constexpr int kAhead = 4;
constexpr int kRing = 6;
constexpr int kPreBarrier = -2, kPostBarrier = -1;
__host__ __device__ constexpr int first_use(int r) {
  for (int j = 0; j < kOps; ++j)
    if (iter_op(j).r == r) return j;
  return kOps;
}
__host__ __device__ constexpr int last_use(int r) {
  int u = -3;
  for (int j = 0; j < kOps; ++j)
    if (iter_op(j).r == r) u = j;
  return u;
}
__host__ __device__ constexpr int issue_slot(int r) {
  if (r < kPvHead) return kPreBarrier;
  int s = kPostBarrier;
  if (r >= kAhead && first_use(r - kAhead) > s) s = first_use(r - kAhead);
  if (r >= kRing && last_use(r - kRing) + 1 > s) s = last_use(r - kRing) + 1;
  return s;
}
__host__ __device__ constexpr bool schedule_ok() {
  for (int r = 0; r < kReads; ++r) {
    if (issue_slot(r) >= first_use(r)) return false;                           // read before use
    if (r >= kRing && issue_slot(r) <= last_use(r - kRing)) return false;      // ring entry free
    if (r >= kPvHead && r < kPvHead + kQkOps && issue_slot(r) < kPostBarrier) return false;
  }
  for (int j = 0; j < kOps; ++j)
    if (iter_op(j).r < 0 || iter_op(j).r >= kReads) return false;
  return true;
}
static_assert(schedule_ok(), "operand read schedule");
static_assert(kRing > kPvHead, "the pre-barrier reads fit the ring");
// Slots (MFMA indices) of the other work of an iteration: the loads of tile
// t+2 (one part every third MFMA from the second, the page-table block with
// the first),
// the softmax of tile t+1 (after its last QK MFMA has left the pipe), the
// hand-over of its weights to the partner, and the address preparation of
// tile t+3's loads.
constexpr int kDmaSlot0 = 1, kDmaStride = 3;
constexpr int kSoftmaxSlot0 = kQk0 + kQkOps;
constexpr int kSoftmaxSteps = 26;
constexpr int kPrepSlots[3] = {kQk0 + kQkOps + 1, kQk0 + kQkOps + 12, kQk0 + kQkOps + 22};
static_assert(kDmaSlot0 + kDmaStride * 8 < kQk0 + kQkOps, "loads go out before the softmax");
static_assert(kSoftmaxSlot0 + kSoftmaxSteps <= kOps, "softmax fits the PV MFMAs");
}  // namespace bf16k

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// The global -> LDS copies below are issued as inline asm so that the
// compiler's own wait insertion does not treat every later LDS read as
// dependent on them (which would drain the whole prefetch ring); the kernel
// waits for them explicitly with wait_vmem<>. Vector-memory loads retire in
// order, so the compiler's waits for its own loads stay correct. Each asm
// block sets M0 (the LDS destination) and lists it as clobbered; the compiler
// reserves M0 and warns that it will not restore a value of its own around
// the block. It keeps none: the generated code of this file uses M0 only
// inside these blocks (a CPU test checks the assembly, implicit uses
// included).

// The page-table entries of this wave's 8 keys of tiles 8B..8B+7 (batch B >=
// 0), lane i fetching key i%8 of tile 8B + i/8 into ring half B % 2 (one
// 64-lane global_load_lds_dword, no divergence). Positions past `jmax` (the
// group's last key) are clamped to it: those keys are loaded but either
// masked out of the softmax (past the sequence) or never computed (past the
// group), and their data is a real, finite token.
__device__ __forceinline__ void issue_index_batch(const VerifyArgs& a, char* idx_ring, int kv0, int jmax, int batch) {
  using namespace bf16k;
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6;
  const int j = min((batch * kIdxBatch + (lane >> 3)) * kKeysPerTile + wave * 8 + (lane & 7), jmax);
  const uint32_t m0 = lds_addr(idx_ring) + wave * kIdxWaveBytes + (batch & 1) * (kIdxWaveBytes / 2);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(m0),
               "v"((uint64_t)(a.kv_indices + kv0 + j))
               : "memory", "m0");
}

// Key slot (0..7 within this wave's 8 keys) whose kv_c this lane loads:
// chunk lane/8 of the key in slot lane%8, un-swizzled.
__device__ __forceinline__ int lane_kvc_key() {
  const int lane = lane_id();
  return (lane & 7) ^ bf16k::kvc_swizzle(lane >> 3);
}
// Page-table entry of key `key` (0..7) of this wave's share of `tile`, read
// back from the index ring once this wave's load of it has completed.
__device__ __forceinline__ int tile_slot(const char* idx_ring, int tile, int key) {
  using namespace bf16k;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6;
  return *(const int*)(idx_ring + wave * kIdxWaveBytes + ((tile & (2 * kIdxBatch - 1)) * 8 + key) * 4);
}

// Loads of this wave's share of one tile (keys 8w..8w+7) into an LDS buffer,
// every address prepared once per tile and held per lane. Parts 0..7 are the
// kv_c blocks: part j copies chunks 8j..8j+7 of the 8 keys (lane i: chunk
// 8j + i/8 of the key in slot i%8) with one 64-lane 16-byte load whose
// immediate offset, 128j, moves the global and the LDS address alike. Part 8
// is the eight 128-byte k_pe rows together, lane i fetching chunk
// (i%8) ^ (i/8) so that the chunks of one key land XOR-swizzled by the key.
constexpr int kTileParts = 9;
struct TileLoads {
  uint64_t kvc;       // per lane: global address of its kv_c chunk in block 0
  uint64_t kpe;       // per lane: k_pe chunk address
  uint32_t lds_base;  // wave-uniform: LDS address of this wave's region
};

// prepare_tile in two steps (so a loop can spread them between MFMAs).
// buf_lds: LDS address of the destination buffer; kslot: page-table entry
// of lane_kvc_key(); pslot: that of key lane/8.
__device__ __forceinline__ void prepare_rows(TileLoads& t, const VerifyArgs& a, uint32_t buf_lds, int kslot, int wave) {
  using namespace bf16k;
  t.kvc = (uint64_t)(uintptr_t)a.kv_c + (uint64_t)(int64_t)kslot * (uint64_t)a.kv_c_stride * 2u +
          (uint32_t)(lane_id() >> 3) * 16u;
  t.lds_base = buf_lds + wave * kRegion;
}
__device__ __forceinline__ void prepare_kpe(TileLoads& t, const VerifyArgs& a, int pslot) {
  const int lane = lane_id();
  const int chunk = (lane & 7) ^ (lane >> 3);
  t.kpe = (uint64_t)(uintptr_t)a.k_pe + ((uint64_t)(int64_t)pslot * (uint64_t)a.k_pe_stride + chunk * 8) * 2u;
}
__device__ __forceinline__ TileLoads prepare_tile(const VerifyArgs& a, const char* buf, const char* idx_ring, int tile,
                                                  int wave) {
  TileLoads t;
  prepare_rows(t, a, lds_addr(buf), tile_slot(idx_ring, tile, lane_kvc_key()), wave);
  prepare_kpe(t, a, tile_slot(idx_ring, tile, lane_id() >> 3));
  return t;
}

template <int kPart>
__device__ __forceinline__ void issue_tile_part(const TileLoads& t, int wave) {
  using namespace bf16k;
  if constexpr (kPart < 8) {
    // LDS destination M0 + 128*kPart + 16*lane = block kPart of the region.
    const uint32_t m0 = t.lds_base + (1024 - 128) * kPart;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:%2" ::"s"(m0), "v"(t.kvc),
                 "i"(128 * kPart)
                 : "memory", "m0");
  } else {
    const uint32_t m0 = t.lds_base - wave * kRegion + kCBytes + wave * 8 * kPeRow;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(t.kpe)
                 : "memory", "m0");
  }
}

__device__ __forceinline__ void issue_tile(const TileLoads& t, int wave) {
  static_for<kTileParts>([&](auto part) { issue_tile_part<decltype(part)::value>(t, wave); });
}

// Values 4*gi .. 4*gi+3 of an accumulator block, read out of the
// accumulation registers one at a time by inline asm: left to itself the
// compiler moves whole 16-register blocks to VGPRs (which do not fit next to
// Q) and places the move where it likes. The compiler does not insert the
// wait states an MFMA result needs before such a read: a caller that may run
// within 20 cycles of the MFMA that wrote `acc` calls mfma_result_wait()
// first.
__device__ __forceinline__ f32x4_t read_acc4(const f32x16_t& acc, int gi) {
  float t0, t1, t2, t3;
  asm volatile(
      "v_accvgpr_read_b32 %0, %4\n\tv_accvgpr_read_b32 %1, %5\n\t"
      "v_accvgpr_read_b32 %2, %6\n\tv_accvgpr_read_b32 %3, %7"
      : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
      : "a"(acc[4 * gi]), "a"(acc[4 * gi + 1]), "a"(acc[4 * gi + 2]), "a"(acc[4 * gi + 3]));
  return f32x4_t{t0, t1, t2, t3};
}
// 20 wait states: more than any 32x32 MFMA result needs before it is read.
__device__ __forceinline__ void mfma_result_wait() { asm volatile("s_nop 15\n\ts_nop 3" ::: "memory"); }

// QK MFMAs with the S^T accumulator in VGPRs. Left to itself the compiler
// gives every MFMA accumulator an AGPR block; all 256 hold O, so it would park
// an output block in VGPRs around every QK and copy the scores out after it.
// The compiler does not see these as MFMAs: the reader of the result waits
// with qk_result_wait() (after which the scores are ordinary VGPR values), and
// the accumulation chain keeps the same registers (srcC = vdst), which needs
// no wait states between its MFMAs.
__device__ __forceinline__ void mfma_qk_first(f32x16_t& acc, const bf16x8_t& k, const bf16x8_t& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(k), "v"(q));
}
__device__ __forceinline__ void mfma_qk(f32x16_t& acc, const bf16x8_t& k, const bf16x8_t& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(k), "v"(q));
}
__device__ __forceinline__ void qk_result_wait(f32x16_t& acc) { asm volatile("s_nop 15\n\ts_nop 3" : "+v"(acc)); }

__global__ void __launch_bounds__(bf16k::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_verify_attn_bf16_kernel(const VerifyArgs a) {
  using namespace bf16k;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  char* const idx_ring = smem + kNbuf * kBufBytes;
  uint64_t* const anc_lds = (uint64_t*)(idx_ring + kIdxBytes);
  char* const qpe_lds = idx_ring + kIdxBytes + kAncBytes;
  char* const px_lds = qpe_lds + kQpeBytes;
  float* const lx_lds = (float*)(px_lds + kPxBytes);

  BlockWork w;
  if (!map_block(a, w)) return;
  write_status<kThreads>(a, w);
  if (w.rb * kRows >= w.rows) return;
  const int H = a.heads;

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6;  // uniform: keep it scalar
  const int half = lane >> 5;   // k slice of MFMA operands / key quartet of S^T rows
  const int qcol = lane & 31;   // column of the 32x32 blocks: this lane's query row
  const int partner = wave ^ 1;  // the wave whose rows share this wave's V^T reads
  const int fhalf = wave & 1;    // output features 256*fhalf.. of both waves' rows

  // The page-table entries of the first two batches of tiles go out first,
  // so that their round trip overlaps the loads of Q and of the tree.
  const int jmax0 = min(w.N, w.tile_end * kKeysPerTile) - 1;
  if (w.tile_begin < w.tile_end) {
    issue_index_batch(a, idx_ring, w.kv0, jmax0, w.tile_begin / kIdxBatch);
    issue_index_batch(a, idx_ring, w.kv0, jmax0, w.tile_begin / kIdxBatch + 1);
  }

  // ---- this lane's query row: wave w owns rows 32w..32w+31 of the block ----
  const int r_local = w.rb * kRows + wave * 32 + qcol;
  const int r_eff = min(r_local, w.rows - 1);
  const int64_t grow = (int64_t)w.node0 * H + r_eff;
  bf16x8_t qreg[32];
  const char* const qpe_lane = qpe_lds + (wave * 4 * 64 + lane) * 16;
  {
    const __bf16* qn = (const __bf16*)a.q_nope + grow * kDl + half * 8;
    const __bf16* qp = (const __bf16*)a.q_pe + grow * kDr + half * 8;
#pragma unroll
    for (int kc = 0; kc < 32; ++kc) qreg[kc] = *(const bf16x8_t*)(qn + kc * 16);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)  // only this lane reads these back
      *(bf16x8_t*)(qpe_lane + kc * 64 * 16) = *(const bf16x8_t*)(qp + kc * 16);
  }
  // This lane's ancestor mask waits in LDS (read by the few tiles that reach
  // the tree tail and by the epilogue) instead of holding registers through
  // the tile loop. Only half 0 writes it; the first barrier of the pipeline
  // orders the write before every read. Trees of up to 64 nodes take the
  // one-wave builder; larger ones are built by the workgroup in the ring
  // buffer of the third tile, first loaded after that barrier.
  {
    uint64_t* const dst = anc_lds + (wave * 32 + qcol) * kMaskWords;
    if (w.T <= 64) {
      const uint64_t tmask = wave_tree_mask(a.parents + w.node0, w.T);
      const uint64_t anc = node_mask(tmask, r_eff / H);
      if (half == 0) {
        dst[0] = w.seq_ok ? anc : 0ull;
#pragma unroll
        for (int k = 1; k < kMaskWords; ++k) dst[k] = 0ull;
      }
    } else {
      char* const scratch = smem + ((w.tile_begin + 2) % kNbuf) * kBufBytes;
      block_tree_masks<kThreads>(a.parents + w.node0, w.T, scratch);
      const uint64_t* src = tree_scratch_masks(scratch) + (r_eff / H) * kMaskWords;
      if (half == 0) {
#pragma unroll
        for (int k = 0; k < kMaskWords; ++k) dst[k] = w.seq_ok ? src[k] : 0ull;
      }
    }
  }
  // Mask bits of this lane's row for tail nodes u0..u0+31 (mask_window),
  // loaded afresh so that nothing is carried through the loop in registers.
  auto row_window = [&](int u0) {
    int i = wave * 32 + qcol;
    asm volatile("" : "+v"(i));
    const int w0 = min(max(u0, 0) >> 6, kMaskWords - 1);
    const uint64_t* m = anc_lds + i * kMaskWords;
    return mask_window(u0, m[w0], w0 + 1 < kMaskWords ? m[w0 + 1] : 0ull);
  };
  // Whether row 32*wv + (lane%32) of the block belongs to a valid node (its
  // mask is not empty).
  auto row_valid = [&](int wv) {
    int i = wv * 32 + qcol;
    asm volatile("" : "+v"(i));
    uint64_t any = 0;
#pragma unroll
    for (int k = 0; k < kMaskWords; ++k) any |= anc_lds[i * kMaskWords + k];
    return any != 0;
  };

  // Per-lane LDS address pieces.
  // K (A operand of QK): key = qcol, chunk 2*kc + half (8 features at
  // 16*kc + 8*half): region qcol/8, block kc/4, chunk slot 2*(kc%4) + half,
  // key slot qcol%8 swizzled when kc is odd (k_off[kc % 2]).
  const int k_reg = (qcol >> 3) * kRegion + half * 128;
  const int k_off0 = k_reg + 16 * (qcol & 7), k_off1 = k_reg + 16 * ((qcol & 7) ^ 4);
  const int kpe_off = kCBytes + qcol * kPeRow;
  const int kpe_sw = qcol & 7;
  // V^T (A operand of PV) via transpose reads: 16-lane group g reads 4 keys x
  // 16 features; lane i of the group points at key 4*half + i/4, features
  // 16*(g%2) + 4*(i%4) of the feature block. Lane l then holds feature l%32
  // of the block for keys 4*half + 0..3 (+8 for the second read). Feature
  // block fb of those keys: chunk 4*fb + 2*(g%2) + (i%4)/2, at byte 8*(i%2) of
  // it, in the region of the keys' wave (plus 512*fb); this wave's feature
  // half starts at block 8*fhalf.
  const int g16 = lane >> 4, i16 = lane & 15;
  const int v_off = 256 * (g16 & 1) + 128 * ((i16 & 3) >> 1) +
                    16 * ((4 * half + (i16 >> 2)) ^ kvc_swizzle(2 * (g16 & 1))) + 8 * (i16 & 1) +
                    fhalf * 8 * 512;
  // P^T fragments: this lane's slot in this wave's and in the partner's area.
  char* const px_own = px_lds + wave * kPxWaveBytes + lane * 16;
  const char* const px_partner = px_lds + partner * kPxWaveBytes + lane * 16;
  // Weights of a tile (parity tp) for the partner: fragment u at u*1024.
  auto write_p = [&](const bf16x8_t& frag, int u, int tp) {
    *(bf16x8_t*)(px_own + tp * 4 * kPxWaveBytes + u * 1024) = frag;
  };

  // Softmax state of this lane's row (same rules as the fp32 kernel):
  // m_ref = reference max (log2 units, scaled) fixed at the first tile where
  // the row sees a key; weights are 2^(s - m_ref); if some score exceeds it by
  // more than kOverflowSlack the block repeats the split with the exact max.
  // O^T of feature half fhalf: oacc[0][fb] for this wave's 32 rows,
  // oacc[1][fb] for the partner's, features 256*fhalf + 32fb..+31.
  f32x16_t oacc[2][8];
  float m_ref = -INFINITY, m_max = -INFINITY, l_run = 0.f;

  // Invisible keys of one S^T block get -inf (register i holds key
  // k0 + (i/4)*8 + 4*half + i%4): keys from jend on, and tail keys (from P
  // on) outside the row's ancestor mask.
  auto mask_tile = [&](f32x16_t& sacc, int k0, int jend) {
    const uint32_t hwin = row_window(k0 - w.P) >> (4 * half);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = k0 + (i >> 2) * 8 + half * 4 + (i & 3);
      const bool tail_bit = ((hwin >> ((i >> 2) * 8 + (i & 3))) & 1u) != 0;
      const bool vis = (j < jend) & ((j < w.P) | tail_bit);
      sacc[i] = vis ? sacc[i] : -INFINITY;
    }
  };
  // Weights of one (masked) tile for this lane's row, 2^(scale*s*log2e -
  // m_ref), as the two bf16 P^T fragments of the PV MFMAs (key steps 0 and
  // 1). Register i of the S^T block is key (i/4)*8 + 4*half + i%4, so
  // fragment u (values 8u..8u+7) covers keys 16u..16u+15, in the order the
  // V^T reads follow. Split into steps 0..kSoftmaxSteps-1 that the loop runs
  // one per MFMA. With one wave per SIMD a VALU instruction that waits for
  // the one before it stalls the whole instruction stream, MFMAs included,
  // so every step only consumes results of earlier steps: the max is a tree
  // spread over steps 0..5, and the weights are a three-stage pipeline
  // (scale, exp2, sum) with value i in stage 1 at step 8+i. The max is taken
  // on raw scores (scale > 0 keeps the order).
  struct SoftmaxState {
    float t[7], mswap, mx, nmu, psum;
  } sm;
  auto softmax_step = [&](auto kc, f32x16_t& sc, bf16x8_t (&pw)[2], bool& overflow) {
    constexpr int k = decltype(kc)::value;
    if constexpr (k == 0) {
      sm.t[0] = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
      sm.t[1] = fmaxf(fmaxf(sc[3], sc[4]), sc[5]);
      sm.t[2] = fmaxf(fmaxf(sc[6], sc[7]), sc[8]);
    } else if constexpr (k == 1) {
      sm.t[3] = fmaxf(fmaxf(sc[9], sc[10]), sc[11]);
      sm.t[4] = fmaxf(fmaxf(sc[12], sc[13]), sc[14]);
      sm.t[5] = fmaxf(fmaxf(sm.t[0], sm.t[1]), sc[15]);
    } else if constexpr (k == 2) {
      sm.t[6] = fmaxf(fmaxf(sm.t[2], sm.t[3]), sm.t[4]);
    } else if constexpr (k == 3) {
      sm.t[0] = fmaxf(sm.t[5], sm.t[6]);
    } else if constexpr (k == 4) {
      sm.mswap = swap_halves(sm.t[0]);
    } else if constexpr (k == 5) {
      sm.mx = fmaxf(sm.t[0], sm.mswap) * a.scale_log2;
    } else if constexpr (k == 6) {
      m_max = fmaxf(m_max, sm.mx);
      if (m_ref == -INFINITY) m_ref = sm.mx;
    } else if constexpr (k == 7) {
      overflow |= sm.mx > m_ref + kOverflowSlack;
      sm.nmu = m_ref == -INFINITY ? 0.f : -m_ref;
      sm.psum = 0.f;
    } else if constexpr (k >= 8 && k < 8 + 18) {
      constexpr int i = k - 8;
      if constexpr (i < 16) sc[i] = __builtin_fmaf(sc[i], a.scale_log2, sm.nmu);
      if constexpr (i >= 1 && i <= 16) sc[i - 1] = __builtin_amdgcn_exp2f(sc[i - 1]);
      if constexpr (i >= 2) sm.psum += sc[i - 2];
      if constexpr (i == 10 || i == 17) {
        constexpr int u = i == 10 ? 0 : 1;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) pw[u][jj] = (__bf16)sc[8 * u + jj];
      }
      if constexpr (i == 17) l_run += sm.psum;
    }
  };
  constexpr int kStepsUsed = 26;
  static_assert(kSoftmaxSteps >= kStepsUsed, "softmax steps");
  // A tile needs masking when it reaches the tree tail (or the sequence end).
  auto needs_mask = [&](int k0) { return k0 + kKeysPerTile > w.P; };

  // Partial c of the sequence's split groups (sequences with several
  // groups): (m, l) of this wave's rows (both lanes of a row hold the same
  // values), written by this wave, and the raw O of feature half fhalf of its
  // own and its partner's rows. Nothing is exchanged, so no barrier.
  // Accumulator register i of block fb holds feature 256*fhalf + 32fb +
  // (i/4)*8 + 4*half + i%4.
  //
  // O goes out in fp16 times a power of two per (row, feature half), 2^(15 -
  // e) where 2^e bounds the half's largest |O|, and that power's inverse goes
  // to the row's (m, l) record. The result moves by at most 2^-12 of the
  // feature half's largest |o|, where bf16's 8 significant bits would move
  // each element by up to 2^-9 of itself: about 8e-3 on rows whose weight
  // sits on a few keys with latent values near 4. The bytes are those of
  // bf16, half those of fp32: at a long prefix every workgroup ends at once,
  // and nothing hides this store burst.
  //
  // The partial arrays have a.part_rows (a multiple of kRows) rows per
  // group, so the rows past T_b * H of the last row block have room and every
  // store below is unconditional.
  auto emit_partial = [&](int c, float l_part) {
    // Lane indices taken afresh (an opaque copy), so that no address below is
    // computed ahead of the tile loop and kept live through it.
    int lq = lane;
    asm volatile("" : "+v"(lq));
    const int qcol = lq & 31, half = lq >> 5;
    const float l_tot = l_part + swap_halves(l_part);
    const bool node_ok = row_valid(wave);
    mfma_result_wait();  // the last PV MFMAs may have just been issued
    const int64_t prow0 = (int64_t)c * a.part_rows + w.rb * kRows + qcol;
    *(float2*)(a.part_ml + 4 * (prow0 + wave * 32)) = make_float2(node_ok ? m_ref : NAN, node_ok ? l_tot : NAN);
#pragma unroll
    for (int rbk = 0; rbk < 2; ++rbk) {
      const int64_t prow = prow0 + (rbk ? partner : wave) * 32;
      // Largest |O| of the row's feature half (128 values in each wave half).
      float mx = 0.f;
#pragma unroll
      for (int fb = 0; fb < 8; ++fb)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const f32x4_t t = read_acc4(oacc[rbk][fb], gi);
          mx = fmaxf(mx, fmaxf(fmaxf(fabsf(t[0]), fabsf(t[1])), fmaxf(fabsf(t[2]), fabsf(t[3]))));
        }
      mx = fmaxf(mx, swap_halves(mx));
      // mx = f * 2^e with f in [0.5, 1), so |O| * 2^(15 - e) < 2^15, inside
      // fp16's range however large O is; e is held at -100 or above so that
      // both powers stay normal floats.
      const int e = max(__builtin_amdgcn_frexp_expf(mx), -100);
      const float down = __builtin_amdgcn_ldexpf(1.f, 15 - e);
      if (half == 0) a.part_ml[4 * prow + 2 + fhalf] = __builtin_amdgcn_ldexpf(1.f, e - 15);
      _Float16* dst = (_Float16*)a.part_o + prow * kDl + fhalf * 256 + 8 * half;
#pragma unroll
      for (int fb = 0; fb < 8; ++fb)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          // Values 2m and 2m+1 (features 16m + 4*half + 0..3 and 16m + 8 +
          // 4*half + 0..3 of the block) become 8 consecutive features per
          // lane by one exchange between the wave halves: the lower half
          // keeps 16m..16m+7, the upper half gets 16m+8..16m+15.
          const f32x4_t t0 = read_acc4(oacc[rbk][fb], 2 * m) * down;
          const f32x4_t t1 = read_acc4(oacc[rbk][fb], 2 * m + 1) * down;
          uint32_t x[2], y[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            x[k] = pack_f16x2(t0[2 * k], t0[2 * k + 1]);
            y[k] = pack_f16x2(t1[2 * k], t1[2 * k + 1]);
            const auto sw = __builtin_amdgcn_permlane32_swap(x[k], y[k], false, false);
            x[k] = sw[0];
            y[k] = sw[1];
          }
          *(u32x4_t*)(dst + 32 * fb + 16 * m) = u32x4_t{x[0], x[1], y[0], y[1]};
          // One pair at a time: otherwise the scheduler reads every
          // accumulator out at once and runs out of registers.
          __builtin_amdgcn_sched_barrier(0);
        }
    }
  };
  // Output of a sequence with one split group: O / l and lse. The partner's
  // row sums come through LDS (every wave of the workgroup calls this).
  auto emit_final = [&]() {
    const float l_tot = l_run + swap_halves(l_run);
    if (half == 0) lx_lds[wave * 32 + qcol] = l_tot;
    __syncthreads();
    const float l_par = lx_lds[partner * 32 + qcol];
    const bool ok_own = row_valid(wave), ok_par = row_valid(partner);
    mfma_result_wait();
    const int r_own = w.rb * kRows + wave * 32 + qcol, r_par = w.rb * kRows + partner * 32 + qcol;
    if (r_own < w.rows && half == 0 && a.lse) {
      const int64_t g = (int64_t)w.node0 * H + r_own;
      a.lse[g] = ok_own ? (m_ref + __log2f(l_tot)) * kLn2 : NAN;
    }
#pragma unroll
    for (int rbk = 0; rbk < 2; ++rbk) {
      const int r = rbk ? r_par : r_own;
      if (r < w.rows) {
        const int64_t g = (int64_t)w.node0 * H + r;
        float* dst = a.out + g * kDl + fhalf * 256 + 4 * half;
        const float mul = (rbk ? ok_par : ok_own) ? 1.f / (rbk ? l_par : l_tot) : NAN;
#pragma unroll
        for (int fb = 0; fb < 8; ++fb)
#pragma unroll
          for (int gi = 0; gi < 4; ++gi) {
            const f32x4_t v = read_acc4(oacc[rbk][fb], gi);
            *(f32x4_t*)(dst + 32 * fb + 8 * gi) = v * mul;
          }
      }
    }
  };

  for (int pass = 0; pass < 2; ++pass) {
    l_run = 0.f;
    bool overflow = false;
#pragma unroll
    for (int rbk = 0; rbk < 2; ++rbk)
#pragma unroll
      for (int x = 0; x < 8; ++x)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[rbk][x][i] = 0.f;

    if (w.tile_begin < w.tile_end) {
      const int tb = w.tile_begin, te = w.tile_end;
      const int jmax = min(w.N, te * kKeysPerTile) - 1;
      // Pipeline. Iteration t: tiles t and t+1 are in LDS, tile t+2 is
      // fetched (and, when t+kIdxLead starts a batch, the page-table entries
      // of tiles t+kIdxLead..t+kIdxLead+7); the QK and softmax
      // of tile t+1 run between the PV MFMAs of tile t, whose weights this
      // wave computed in the previous iteration and holds in registers (the
      // partner's arrive through LDS). The tiles past the group repeat its
      // last key (loaded, never visible), which keeps the number of loads per
      // iteration constant; the QK of the group's last iteration runs on
      // such a tile and is masked out.
      if (pass > 0) {  // pass 0 issued these at the start
        issue_index_batch(a, idx_ring, w.kv0, jmax, tb / kIdxBatch);
        issue_index_batch(a, idx_ring, w.kv0, jmax, tb / kIdxBatch + 1);
      }
      wait_vmem<0>();
      issue_tile(prepare_tile(a, smem + (tb % kNbuf) * kBufBytes, idx_ring, tb, wave), wave);
      issue_tile(prepare_tile(a, smem + ((tb + 1) % kNbuf) * kBufBytes, idx_ring, tb + 1, wave), wave);
      // Loads of tile tb+2, issued during the first iteration.
      TileLoads pending = prepare_tile(a, smem + ((tb + 2) % kNbuf) * kBufBytes, idx_ring, tb + 2, wave);
      wait_vmem<kTileParts>();  // this wave's part of tile tb
      block_sync();
      // Scores and weights of the first tile.
      bf16x8_t pk[2];
      {
        const char* const kb = smem + (tb % kNbuf) * kBufBytes;
        // K fragment of QK MFMA c (0..3 rope, 4..35 latent chunks)
        auto read_k = [&](auto cc) -> bf16x8_t {
          constexpr int c = decltype(cc)::value;
          if constexpr (c < 4) return *(const bf16x8_t*)(kb + kpe_off + (((2 * c + half) ^ kpe_sw) << 4));
          else {
            constexpr int kc = c - 4;
            return *(const bf16x8_t*)(kb + ((kc & 1) ? k_off1 : k_off0) + 1024 * (kc >> 2) + 256 * (kc & 3));
          }
        };
        bf16x8_t qf[4], ring[kRing];
#pragma unroll
        for (int j = 0; j < 4; ++j) qf[j] = *(const bf16x8_t*)(qpe_lane + j * 64 * 16);
        static_for<kAhead>([&](auto j) { ring[j % kRing] = read_k(j); });
        f32x16_t s0;
        static_for<kQkOps>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          if constexpr (c + kAhead < kQkOps) ring[(c + kAhead) % kRing] = read_k(std::integral_constant<int, c + kAhead>{});
          if constexpr (c == 0) mfma_qk_first(s0, ring[0], qf[0]);
          else if constexpr (c < 4) mfma_qk(s0, ring[c % kRing], qf[c]);
          else mfma_qk(s0, ring[c % kRing], qreg[c - 4]);
          __builtin_amdgcn_sched_barrier(0);
        });
        qk_result_wait(s0);
        if (needs_mask(tb * kKeysPerTile)) mask_tile(s0, tb * kKeysPerTile, w.N);
        static_for<kSoftmaxSteps>([&](auto k) { softmax_step(k, s0, pk, overflow); });
        write_p(pk[0], 0, tb & 1);
        write_p(pk[1], 1, tb & 1);
      }

      // Byte offsets of the buffers of tiles t, t+1 and t+2, rotated each
      // iteration (tile t+3 reuses the buffer of tile t).
      int bo0 = (tb % kNbuf) * kBufBytes, bo1 = ((tb + 1) % kNbuf) * kBufBytes, bo2 = ((tb + 2) % kNbuf) * kBufBytes;
      // The group's splits are consecutive ranges of key tiles: one stream
      // through the pipeline.
      for (int tile = tb; tile < te; ++tile) {
        // Everything this wave issued in the previous iteration (the keys of
        // tile+1, a page-table batch, its weights for the partner) has landed.
        wait_vmem<0>();
        wait_lds();
        const char* const vbase = smem + bo0 + v_off;  // tile t (PV)
        const char* const kbuf = smem + bo1;           // tile t+1 (QK)
        const bool has_next = tile + 1 < te;
        const int k1 = (tile + 1) * kKeysPerTile;
        // Fragment r of the iteration: a V^T fragment of tile t (two
        // transpose reads) or a K fragment of tile t+1.
        auto read_op = [&](auto rc) -> bf16x8_t {
          constexpr int r = decltype(rc)::value;
          constexpr Op o = iter_op(first_use(r));
          if constexpr (o.pv) {
            // keys 16u + 4*half + 0..3 in region 2u, the next 8 keys in region 2u+1
            constexpr int u = o.p >> 3, fb = o.p & 7;
            const char* vp = vbase + 2 * u * kRegion + fb * 512;
            const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)vp);
            const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vp + kRegion));
            return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
          else if constexpr (o.c < 4) return *(const bf16x8_t*)(kbuf + kpe_off + (((2 * o.c + half) ^ kpe_sw) << 4));
          else {
            constexpr int kc = o.c - 4;
            return *(const bf16x8_t*)(kbuf + ((kc & 1) ? k_off1 : k_off0) + 1024 * (kc >> 2) + 256 * (kc & 3));
          }
        };
        bf16x8_t ring[kRing];
        auto issue_reads = [&](auto sc) {
          constexpr int sl = decltype(sc)::value;
          static_for<kReads>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            if constexpr (issue_slot(r) == sl) ring[r % kRing] = read_op(rc);
          });
        };
        // Before the barrier: the V^T operands of the first PV MFMAs (tile t
        // has been visible since the previous barrier).
        issue_reads(std::integral_constant<int, kPreBarrier>{});
        block_sync();  // tile+1 and the partner's weights of tile t are visible; every wave has finished with tile-1
        bf16x8_t pp[2];
        {
          const char* src = px_partner + (tile & 1) * 4 * kPxWaveBytes;
          pp[0] = *(const bf16x8_t*)src;
          pp[1] = *(const bf16x8_t*)(src + 1024);
        }
        issue_reads(std::integral_constant<int, kPostBarrier>{});
        // The rope part of Q (this lane's own LDS data, written once before
        // the loop), for QK MFMAs 0..3.
        bf16x8_t qf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) qf[j] = *(const bf16x8_t*)(qpe_lane + j * 64 * 16);
        f32x16_t sacc;
        bf16x8_t pn[2];
        int pslots = 0, pkslot = 0;
        static_for<kOps>([&](auto sc) {
          constexpr int s = decltype(sc)::value;
          issue_reads(sc);
          constexpr Op o = iter_op(s);
          if constexpr (o.pv) {
            constexpr int u = o.p >> 3, fb = o.p & 7;
            if constexpr (o.partner)
              oacc[1][fb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[o.r % kRing], pp[u], oacc[1][fb], 0, 0, 0);
            else
              oacc[0][fb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[o.r % kRing], pk[u], oacc[0][fb], 0, 0, 0);
          } else if constexpr (o.c == 0) {
            mfma_qk_first(sacc, ring[o.r % kRing], qf[0]);
          } else if constexpr (o.c < 4) {
            mfma_qk(sacc, ring[o.r % kRing], qf[o.c]);
          } else {
            mfma_qk(sacc, ring[o.r % kRing], qreg[o.c - 4]);
          }
          // Tile t+2 goes into the buffer tile t-1 used, free since every
          // wave passed the barrier; its addresses were prepared during the
          // previous iteration. One load every third MFMA from the start of
          // the iteration: a burst of all of them from every wave queues in
          // the vector-memory path and stalls the issuing waves, and the
          // earlier they go out, the more of their latency the iteration
          // hides (page_size=1 pools, whose tiles miss L2 more often, gained
          // 2.5-4% over loads that started at the third QK MFMA).
          if constexpr (s >= kDmaSlot0 && (s - kDmaSlot0) % kDmaStride == 0 &&
                        (s - kDmaSlot0) / kDmaStride < kTileParts) {
            constexpr int part = (s - kDmaSlot0) / kDmaStride;
            issue_tile_part<part>(pending, wave);
            // The next page-table batch, once its ring half is free.
            if constexpr (part == 0) {
              const int nb = tile + kIdxLead;
              if ((nb & (kIdxBatch - 1)) == 0 && nb / kIdxBatch >= tb / kIdxBatch + 2)
                issue_index_batch(a, idx_ring, w.kv0, jmax, nb / kIdxBatch);
            }
          }
          // Scores of tile t+1: tail tiles are masked; past the group's last
          // tile nothing is visible.
          if constexpr (s == kSoftmaxSlot0 - 1) {
            qk_result_wait(sacc);
            if (!has_next || needs_mask(k1)) mask_tile(sacc, k1, has_next ? w.N : 0);
          }
          if constexpr (s >= kSoftmaxSlot0 && s - kSoftmaxSlot0 < kSoftmaxSteps)
            softmax_step(std::integral_constant<int, s - kSoftmaxSlot0>{}, sacc, pn, overflow);
          // Weights of tile t+1 for the partner, as soon as each fragment is
          // complete (softmax steps 18 and 25).
          if constexpr (s == kSoftmaxSlot0 + 19) write_p(pn[0], 0, (tile + 1) & 1);
          if constexpr (s == kSoftmaxSlot0 + 25) write_p(pn[1], 1, (tile + 1) & 1);
          // Addresses of tile t+3's loads (entries landed before this
          // iteration's wait).
          if constexpr (s == kPrepSlots[0]) {
            pslots = tile_slot(idx_ring, tile + 3, lane_kvc_key());
            pkslot = tile_slot(idx_ring, tile + 3, lane >> 3);
          }
          if constexpr (s == kPrepSlots[1]) prepare_rows(pending, a, lds_addr(smem) + (uint32_t)bo0, pslots, wave);
          if constexpr (s == kPrepSlots[2]) prepare_kpe(pending, a, pkslot);
          __builtin_amdgcn_sched_barrier(0);
        });
        pk[0] = pn[0];
        pk[1] = pn[1];
        const int bt = bo0;
        bo0 = bo1;
        bo1 = bo2;
        bo2 = bt;
      }
      // The group's partial goes out (a redo pass rewrites it).
      if (w.G > 1) emit_partial(w.part, l_run);
      wait_vmem<0>();
    } else {
      // No key tiles: empty partials (m = -inf, l = 0, O = 0).
      if (w.G > 1) emit_partial(w.part, 0.f);
    }
    if (pass == 1 || !__syncthreads_or(overflow)) break;
    m_ref = m_max;
  }

  // ---- epilogue: a sequence with one split group writes its output -------
  if (w.G == 1) emit_final();
}

// ===========================================================================
// fp32 kernel
// ===========================================================================
namespace f32k {
constexpr int kThreads = 64;
constexpr int kRows = 32;
constexpr int kRowBytes = kDk * 4 + 16;                 // kv_c | k_pe, padded
constexpr int kTileBytes = kKeysPerTile * kRowBytes;
constexpr int kSmem = kTileBytes + kRows * kRowBytes;   // tile + Q rows
// Trees above 64 nodes build their masks in the tile buffer before the first tile.
static_assert(kTreeScratchBytes <= kTileBytes, "tree mask scratch");
}  // namespace f32k

__global__ void __launch_bounds__(f32k::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_verify_attn_f32_kernel(const VerifyArgs a) {
  using namespace f32k;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  char* const qs = smem + kTileBytes;

  BlockWork w;
  if (!map_block(a, w)) return;
  write_status<kThreads>(a, w);
  if (w.rb * kRows >= w.rows) return;
  const int H = a.heads;
  const int lane = lane_id();
  const int half = lane >> 5;
  const int qcol = lane & 31;
  const int r_local = w.rb * kRows + qcol;
  const bool row_ok = r_local < w.rows;
  const int r_eff = row_ok ? r_local : w.rows - 1;
  const int64_t grow = (int64_t)w.node0 * H + r_eff;
  // Ancestor mask words of this lane's row: the one-wave builder for trees of
  // up to 64 nodes, else the workgroup builder in the (not yet used) tile buffer.
  uint64_t anc[kMaskWords];
  if (w.T <= 64) {
    anc[0] = node_mask(wave_tree_mask(a.parents + w.node0, w.T), r_eff / H);
#pragma unroll
    for (int k = 1; k < kMaskWords; ++k) anc[k] = 0ull;
  } else {
    block_tree_masks<kThreads>(a.parents + w.node0, w.T, smem);
    const uint64_t* src = tree_scratch_masks(smem) + (r_eff / H) * kMaskWords;
#pragma unroll
    for (int k = 0; k < kMaskWords; ++k) anc[k] = src[k];
  }
  uint64_t any = 0;
#pragma unroll
  for (int k = 0; k < kMaskWords; ++k) any |= anc[k];
  const bool node_ok = w.seq_ok && any != 0;

  // Q rows of the block into LDS: row qr = [q_nope | q_pe].
  for (int idx = lane; idx < kRows * 144; idx += 64) {
    const int qr = idx / 144, ch = idx % 144;
    const int rr = min(w.rb * kRows + qr, w.rows - 1);
    const int64_t gr = (int64_t)w.node0 * H + rr;
    const float* src = ch < 128 ? (const float*)a.q_nope + gr * kDl + ch * 4
                                : (const float*)a.q_pe + gr * kDr + (ch - 128) * 4;
    *(u32x4_t*)(qs + qr * kRowBytes + ch * 16) = *(const u32x4_t*)src;
  }

  // Softmax state of this lane's row. m_ref is the reference max (log2 units,
  // scale applied): the max of the first tile in which the row sees a key. It
  // never moves during a pass, so O is never rescaled; weights are
  // 2^(s - m_ref). If a later score exceeds m_ref by more than kOverflowSlack,
  // the whole workgroup repeats the split once with m_ref = the exact max of
  // the split (m_max), which cannot overflow.
  f32x16_t oacc[16];
  float m_ref = -INFINITY, m_max = -INFINITY, l_run = 0.f;
  const float* k_rd = (const float*)(smem + qcol * kRowBytes) + half;
  const float* q_rd = (const float*)(qs + qcol * kRowBytes) + half;

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int fb = 0; fb < 16; ++fb)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[fb][i] = 0.f;
    l_run = 0.f;
    bool overflow = false;
    for (int tile = w.tile_begin; tile < w.tile_end; ++tile) {
      const int k0 = tile * kKeysPerTile;
      __syncthreads();
      {
        // Stage keys k0..k0+31: kv_c rows are 2 KB (two loads each), four
        // 256-byte k_pe rows per load. Past-the-end keys repeat the last token.
        const int my_slot = a.kv_indices[w.kv0 + min(k0 + (lane & 31), w.N - 1)];
        const float* kvc = (const float*)a.kv_c;
        const float* kpe = (const float*)a.k_pe;
#pragma unroll 4
        for (int key = 0; key < kKeysPerTile; ++key) {
          const int slot = __builtin_amdgcn_readlane(my_slot, key);
#pragma unroll
          for (int part = 0; part < 2; ++part)
            *(u32x4_t*)(smem + key * kRowBytes + part * 1024 + lane * 16) =
                *(const u32x4_t*)(kvc + (int64_t)slot * a.kv_c_stride + part * 256 + lane * 4);
        }
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          const int key = g * 4 + (lane >> 4), ch = lane & 15;
          const int slot = shfl_i32(my_slot, key);
          *(u32x4_t*)(smem + key * kRowBytes + kDl * 4 + ch * 16) =
              *(const u32x4_t*)(kpe + (int64_t)slot * a.k_pe_stride + ch * 4);
        }
      }
      __syncthreads();

      f32x16_t sacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll 8
      for (int kc = 0; kc < kDk / 2; ++kc)
        sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(k_rd[2 * kc], q_rd[2 * kc], sacc, 0, 0, 0);

      float sv[16];
      const int u0 = k0 - w.P, w0 = min(max(u0, 0) >> 6, kMaskWords - 1);
      uint64_t lo = anc[0], hi = anc[1];
#pragma unroll
      for (int k = 1; k < kMaskWords; ++k) {
        lo = w0 == k ? anc[k] : lo;
        hi = w0 + 1 == k ? anc[k] : hi;
      }
      if (w0 + 1 >= kMaskWords) hi = 0ull;
      const float mx = mask_scale_max(sv, sacc, a.scale_log2, k0, half, w.P, w.N, mask_window(u0, lo, hi));
      m_max = fmaxf(m_max, mx);
      if (m_ref == -INFINITY) m_ref = mx;
      overflow |= mx > m_ref + kOverflowSlack;
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sv[i] = __builtin_amdgcn_exp2f(sv[i] - m_use);
        psum += sv[i];
      }
      l_run += psum;

      // O^T[512 x 32 rows] += V^T . P^T: step i pairs key (i/4)*8 + i%4
      // (lanes 0-31) with key (i/4)*8 + 4 + i%4 (lanes 32-63).
#pragma unroll
      for (int fb = 0; fb < 16; ++fb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = (i >> 2) * 8 + 4 * half + (i & 3);
          const float v = ((const float*)(smem + key * kRowBytes))[32 * fb + qcol];
          oacc[fb] = __builtin_amdgcn_mfma_f32_32x32x2f32(v, sv[i], oacc[fb], 0, 0, 0);
        }
      }
    }
    if (!__syncthreads_or(overflow)) break;
    m_ref = m_max;
  }

  // Accumulator register i of block fb holds feature 32*fb + (i/4)*8 + 4*half + i%4.
  const float l_tot = l_run + swap_halves(l_run);
  if (!row_ok) return;
  float* dst;
  float mul;
  if (w.G == 1) {
    dst = a.out + grow * kDl;
    mul = node_ok ? 1.f / l_tot : NAN;
    if (half == 0 && a.lse) a.lse[grow] = node_ok ? (m_ref + __log2f(l_tot)) * kLn2 : NAN;
  } else {
    const int64_t prow = (int64_t)w.part * a.part_rows + r_eff;
    dst = (float*)a.part_o + prow * kDl;
    mul = 1.f;
    if (half == 0) {
      a.part_ml[4 * prow] = node_ok ? m_ref : NAN;
      a.part_ml[4 * prow + 1] = node_ok ? l_tot : NAN;
    }
  }
#pragma unroll
  for (int fb = 0; fb < 16; ++fb)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      f32x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = oacc[fb][4 * gi + e] * mul;
      *(f32x4_t*)(dst + 32 * fb + 8 * gi + 4 * half) = v;
    }
}

// ===========================================================================
// Split combine
// ===========================================================================
// Merge the partials (one per split group) of kCombineRows consecutive query
// rows of one sequence: M = max m_c, w_c = 2^(m_c - M), L = sum w_c l_c,
// out = sum w_c O_c / L, lse = (M + log2 L) ln 2. Each partial row is a
// record (m, l, s_0, s_1) and its O_c: fp32 for fp32 problems (s unused),
// fp16 for bf16 problems, where feature half f of O_c is the stored value
// times s_f. Each row has 4 lane groups of 32 lanes (16 features per lane);
// lane group g sums the partials c = g (mod 4), and their sums meet in LDS.
// The rows of a workgroup are adjacent in every partial block. Empty
// partials (m = -inf, or l = 0 and O = 0) get weight 0; a NaN partial
// (invalid tree) makes the row NaN.
constexpr int kCombineRows = 2;
constexpr int kCombineGroups = 4;
constexpr int kCombineThreads = 32 * kCombineGroups * kCombineRows;
constexpr int kCombineStage = 256;

template <typename PartT>
__global__ void __launch_bounds__(kCombineThreads) mla_verify_combine_kernel(const VerifyArgs a) {
  constexpr bool kF16 = sizeof(PartT) == 2;
  __shared__ float wsh[kCombineRows][kCombineStage][2];
  __shared__ f32x4_t accsh[kCombineRows][kCombineGroups - 1][32][4];
  const int row_groups = (a.max_rows_per_seq + kCombineRows - 1) / kCombineRows;
  const int b = (int)(blockIdx.x / row_groups);
  int node0, T;
  seq_tree(a, b, node0, T);
  const int rows = T * a.heads;
  const int tid = threadIdx.x;
  const int j = tid / (32 * kCombineGroups), grp = (tid >> 5) % kCombineGroups, t32 = tid & 31;
  const int r = (int)(blockIdx.x % row_groups) * kCombineRows + j;
  const int s0 = group_off(a, b);
  const int S = group_off(a, b + 1) - s0;
  // Whole workgroup: no split partials, or every row past this sequence's rows.
  if (S <= 1 || (int)(blockIdx.x % row_groups) * kCombineRows >= rows) return;
  const bool live = r < rows;
  const int rr = live ? r : rows - 1;
  const float* ml = a.part_ml + 4 * ((int64_t)s0 * a.part_rows + rr);
  const int64_t ml_stride = 4 * (int64_t)a.part_rows;

  // Row max and NaN flag over the splits (every group computes it).
  float M = -INFINITY;
  int nan = 0;
  for (int cc = t32; cc < S; cc += 32) {
    const float m = ml[cc * ml_stride];
    nan |= m != m;
    M = fmaxf(M, m);
  }
  for (int off = 16; off > 0; off >>= 1) {
    M = fmaxf(M, shfl_f32(M, lane_id() ^ off));
    nan |= shfl_i32(nan, lane_id() ^ off);
  }

  f32x4_t acc[4] = {};
  float lloc = 0.f;
  // Lane t32 of a group holds 16 of the row's 512 features: for fp16 the
  // 8-feature runs starting at 8*t32 (feature half 0) and 256 + 8*t32
  // (feature half 1), for fp32 the 4-feature runs at 4*t32 + 128*q, so that
  // each load instruction of a group reads contiguous bytes.
  const PartT* po = (const PartT*)a.part_o + ((int64_t)s0 * a.part_rows + rr) * kDl + (kF16 ? 8 : 4) * t32;
  const int64_t po_stride = (int64_t)a.part_rows * kDl;
  for (int base = 0; base < S; base += kCombineStage) {
    const int cnt = min(kCombineStage, S - base);
    __syncthreads();
    if (grp == 0) {
      for (int cc = t32; cc < cnt; cc += 32) {
        const f32x4_t rec = *(const f32x4_t*)(ml + (base + cc) * ml_stride);
        const float wgt = rec[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(rec[0] - M);
        wsh[j][cc][0] = kF16 ? wgt * rec[2] : wgt;
        wsh[j][cc][1] = kF16 ? wgt * rec[3] : wgt;
        lloc += wgt * rec[1];
      }
    }
    __syncthreads();
    // Unconditional loads (an empty split's partial is zeros with weight 0),
    // so that several are in flight at once.
#pragma unroll 4
    for (int cc = grp; cc < cnt; cc += kCombineGroups) {
      const PartT* src = po + (base + cc) * po_stride;
      if constexpr (kF16) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float wgt = wsh[j][cc][q];
          const f16x8_t v = *(const f16x8_t*)(src + 256 * q);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * q][e] += wgt * (float)v[e];
            acc[2 * q + 1][e] += wgt * (float)v[4 + e];
          }
        }
      } else {
        const float wgt = wsh[j][cc][0];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += wgt * *(const f32x4_t*)(src + 128 * q);
      }
    }
  }
  if (grp > 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) accsh[j][grp - 1][t32][q] = acc[q];
  } else {
    for (int off = 16; off > 0; off >>= 1) lloc += shfl_f32(lloc, lane_id() ^ off);
  }
  __syncthreads();
  if (grp > 0 || !live) return;
#pragma unroll
  for (int g = 0; g < kCombineGroups - 1; ++g)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] += accsh[j][g][t32][q];
  const int64_t grow = (int64_t)node0 * a.heads + r;
  const float inv = nan ? NAN : 1.f / lloc;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    // acc[q]: features 8*t32 + 256*(q/2) + 4*(q%2) (fp16) or 4*t32 + 128*q (fp32).
    const int f = kF16 ? 8 * t32 + 256 * (q >> 1) + 4 * (q & 1) : 4 * t32 + 128 * q;
    *(f32x4_t*)(a.out + grow * kDl + f) = acc[q] * inv;
  }
  if (t32 == 0 && a.lse) a.lse[grow] = nan ? NAN : (M + __log2f(lloc)) * kLn2;
}

// The same merge when no sequence has more than kCombineSmallMax split
// groups, one wave per row and no LDS: lane l holds features 8l..8l+7 (of
// feature half l/32), so each partial is one 16-byte (fp16) or 32-byte
// (fp32) load per lane and the wave reads it as one contiguous block; every
// lane reads the row's (m, l, s_0, s_1) records itself (the same addresses
// across the wave). Measured against the kernel above: 20 -> 9 us at 2
// groups per row (32k prefix, 16k rows); at 16 groups per row and 2k rows
// (200k prefix) one wave per row has too little parallelism and ran about
// 5 us slower, hence the bound of 8.
constexpr int kCombineSmallMax = 8;
constexpr int kCombineSmallRows = 4;  // waves (rows) per workgroup

template <typename PartT>
__global__ void __launch_bounds__(64 * kCombineSmallRows) mla_verify_combine_small_kernel(const VerifyArgs a) {
  constexpr bool kF16 = sizeof(PartT) == 2;
  const int row_groups = (a.max_rows_per_seq + kCombineSmallRows - 1) / kCombineSmallRows;
  const int b = (int)(blockIdx.x / row_groups);
  int node0, T;
  seq_tree(a, b, node0, T);
  const int rows = T * a.heads;
  const int s0 = group_off(a, b);
  const int S = group_off(a, b + 1) - s0;
  const int r = (int)(blockIdx.x % row_groups) * kCombineSmallRows + (int)(threadIdx.x >> 6);
  if (S <= 1 || r >= rows) return;  // uniform over the wave
  const int lane = lane_id();
  const float* ml = a.part_ml + 4 * ((int64_t)s0 * a.part_rows + r);
  const int64_t ml_stride = 4 * (int64_t)a.part_rows;
  float m[kCombineSmallMax], l[kCombineSmallMax], sc[kCombineSmallMax];
  float M = -INFINITY;
  bool nan = false;
#pragma unroll
  for (int c = 0; c < kCombineSmallMax; ++c) {
    if (c < S) {
      const f32x4_t v = *(const f32x4_t*)(ml + c * ml_stride);
      m[c] = v[0];
      l[c] = v[1];
      sc[c] = lane < 32 ? v[2] : v[3];
      nan |= v[0] != v[0];
      M = fmaxf(M, v[0]);
    }
  }
  float L = 0.f;
  f32x4_t acc[2] = {};
  const PartT* po = (const PartT*)a.part_o + ((int64_t)s0 * a.part_rows + r) * kDl + 8 * lane;
  const int64_t po_stride = (int64_t)a.part_rows * kDl;
#pragma unroll
  for (int c = 0; c < kCombineSmallMax; ++c) {
    if (c < S) {
      // An empty group (m = -inf) has weight 0 and a zero partial.
      const float wgt = m[c] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[c] - M);
      L += wgt * l[c];
      const PartT* src = po + c * po_stride;
      if constexpr (kF16) {
        const float ws = wgt * sc[c];
        const f16x8_t v = *(const f16x8_t*)src;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[0][e] += ws * (float)v[e];
          acc[1][e] += ws * (float)v[4 + e];
        }
      } else {
        acc[0] += wgt * *(const f32x4_t*)src;
        acc[1] += wgt * *(const f32x4_t*)(src + 4);
      }
    }
  }
  const int64_t grow = (int64_t)node0 * a.heads + r;
  const float inv = nan ? NAN : 1.f / L;
  float* dst = a.out + grow * kDl + 8 * lane;
  *(f32x4_t*)dst = acc[0] * inv;
  *(f32x4_t*)(dst + 4) = acc[1] * inv;
  if (lane == 0 && a.lse) a.lse[grow] = nan ? NAN : (M + __log2f(L)) * kLn2;
}

// ===========================================================================
// Launchers
// ===========================================================================
int launch_verify_attention(const VerifyArgs& a, int dtype, int64_t grid_blocks, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (grid_blocks == 0) return 0;  // no tree nodes in the batch
  if (dtype == MLA_DTYPE_BF16)
    hipLaunchKernelGGL(mla_verify_attn_bf16_kernel, dim3((unsigned)grid_blocks), dim3(bf16k::kThreads), 0,
                       st, a);
  else
    hipLaunchKernelGGL(mla_verify_attn_f32_kernel, dim3((unsigned)grid_blocks), dim3(f32k::kThreads), 0, st,
                       a);
  return (int)hipGetLastError();
}

int launch_verify_combine(const VerifyArgs& a, int dtype, void* stream) {
  // Partials are fp16 (with scales) for bf16 problems, fp32 for fp32 problems.
  if (a.max_groups <= kCombineSmallMax) {
    const int64_t wgs = (int64_t)a.batch * ((a.max_rows_per_seq + kCombineSmallRows - 1) / kCombineSmallRows);
    if (wgs == 0) return 0;
    if (dtype == MLA_DTYPE_BF16)
      hipLaunchKernelGGL(mla_verify_combine_small_kernel<_Float16>, dim3((unsigned)wgs),
                         dim3(64 * kCombineSmallRows), 0, (hipStream_t)stream, a);
    else
      hipLaunchKernelGGL(mla_verify_combine_small_kernel<float>, dim3((unsigned)wgs), dim3(64 * kCombineSmallRows),
                         0, (hipStream_t)stream, a);
    return (int)hipGetLastError();
  }
  const int64_t groups = (int64_t)a.batch * ((a.max_rows_per_seq + kCombineRows - 1) / kCombineRows);
  if (groups == 0) return 0;
  if (dtype == MLA_DTYPE_BF16)
    hipLaunchKernelGGL(mla_verify_combine_kernel<_Float16>, dim3((unsigned)groups), dim3(kCombineThreads), 0,
                       (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(mla_verify_combine_kernel<float>, dim3((unsigned)groups), dim3(kCombineThreads), 0,
                       (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int copy_tables_to_device(void* dst, const void* src, size_t bytes, void* stream) {
  return (int)hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, (hipStream_t)stream);
}

// ===========================================================================
// Built-in workspace of mla_verify_run_noalloc
// ===========================================================================
// For callers that cannot allocate device memory: a file-scope device array
// that every such call on a GPU shares; each GPU holds its own copy from the
// first call on it until the process ends. In host code the array's name is
// only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever handed to a kernel.
constexpr size_t kNoAllocScratchBytes = size_t(MLA_VERIFY_NOALLOC_WORKSPACE_BYTES);
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

int noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return 0;
}

int launch_tree_masks(const int32_t* parents, int32_t batch, int32_t tree_nodes, uint64_t* masks,
                      void* stream) {
  hipLaunchKernelGGL(mla_tree_masks_kernel, dim3(batch), dim3(kTreeMaskThreads), 0, (hipStream_t)stream,
                     parents, tree_nodes, masks);
  return (int)hipGetLastError();
}

}  // namespace mlav
