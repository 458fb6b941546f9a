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
// several splits streams their tiles through one pipeline and writes one
// partial per split.
//
// bf16 kernel: 4 waves, 128 query rows, 32-key tiles.
//   * A 3-deep LDS ring of key tiles is filled by global_load_lds_dwordx4
//     (global -> LDS without registers); the loads of tile t+2 go out while
//     tiles t and t+1 are computed on.
//   * QK: wave w owns query rows 32w..32w+31 and keeps the latent 512
//     features of their Q in VGPRs (the rope 64 in LDS). S^T[32 keys x 32
//     rows] = K . Q^T with 36 mfma_f32_32x32x16_bf16.
//   * Softmax weights in fp32 (exp2 domain) against a per-row reference max,
//     rounded to bf16 and shared through LDS (P, 8 KB per tile).
//   * PV: wave w owns output features 128w..128w+127 of all 128 rows:
//     O^T[128 x 128] += V^T . P^T with 32 MFMAs; V^T comes from the same LDS
//     tile through ds_read_b64_tr_b16, P^T with plain 16-byte LDS reads.
//     Splitting PV by features (not rows) cuts the transpose reads, whose LDS
//     rate is a third of plain reads, by 4x.
//   * O^T lives in 256 accumulation registers per lane.
// The key order inside each 16-deep MFMA step is permuted consistently in P^T
// and V^T so that P^T comes straight from the S^T accumulator layout.
//
// fp32 kernel (parity workloads stored in fp32): 1 wave, 32 rows, one LDS tile,
// mfma_f32_32x32x2_f32, Q staged in LDS; same softmax and epilogue rules.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernel_params.h"
#include "wave_tree.h"
#include "plan.h"

namespace mlav {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats rounded to bf16 (nearest even), the first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)lo, (__bf16)hi});
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
  int s, c;                   // current split: index within the sequence, global index
  int s_last;                 // one past the group's last split (within the sequence)
  int kv0, N, P, ntiles;
  int tile_begin, tile_end;   // key tiles of the whole group
  bool seq_ok;
};

// First key tile of split s of a sequence with ntiles tiles and S splits.
__device__ __forceinline__ int split_tile(int s, int ntiles, int S) { return (int)(((int64_t)s * ntiles) / S); }

// First packed node and size of sequence b's tree: the plan's packing, or the
// device offsets of a run that reads them (a size outside 0..the planned size,
// or a negative offset, gives an empty tree: the sequence is skipped).
__device__ __forceinline__ void seq_tree(const VerifyArgs& a, int b, int& node0, int& T) {
  node0 = a.node_offset[b];
  T = a.node_offset[b + 1] - node0;
  if (a.tree_indptr) {
    const int cap = T;
    node0 = a.tree_indptr[b];
    T = a.tree_indptr[b + 1] - node0;
    if (node0 < 0 || T < 0 || T > cap) T = 0;
  }
}

// Returns false for a workgroup with nothing to do: past the last split group,
// or a row block past its sequence's T_b * H rows (row blocks are counted for
// the largest tree; smaller trees leave the rest idle).
__device__ __forceinline__ bool map_block(const VerifyArgs& a, BlockWork& w, int rows_per_block) {
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds;
  const int local = bid / kXcds;
  w.rb = local % a.row_blocks;
  const int cg = (local / a.row_blocks) * kXcds + xcd;
  if (cg >= a.group_offset[a.batch]) return false;
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.group_offset[mid] <= cg) lo = mid;
    else hi = mid - 1;
  }
  w.b = lo;
  seq_tree(a, w.b, w.node0, w.T);
  w.rows = w.T * a.heads;
  if (w.rb * rows_per_block >= w.rows) return false;
  w.S = a.split_offset[w.b + 1] - a.split_offset[w.b];
  w.s = (cg - a.group_offset[w.b]) * a.group;
  w.s_last = min(w.s + a.group, w.S);
  w.c = a.split_offset[w.b] + w.s;
  w.kv0 = a.kv_indptr[w.b];
  w.N = a.kv_indptr[w.b + 1] - w.kv0;
  w.P = w.N - w.T;
  w.seq_ok = w.P >= 0;
  w.ntiles = w.seq_ok ? (w.N + kKeysPerTile - 1) / kKeysPerTile : 0;
  w.tile_begin = split_tile(w.s, w.ntiles, w.S);
  w.tile_end = split_tile(w.s_last, w.ntiles, w.S);
  return true;
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
// Padded kv_c row: 1168 B = 292 dwords = 36 (mod 64 banks). The 16 keys one
// QK operand read serves per LDS cycle then start in 16 distinct 4-bank
// groups (conflict-free); the transpose reads of PV see 2-way conflicts,
// which no plain padding avoids together with the former.
constexpr int kCRow = kDl * 2 + 144;
constexpr int kCBytes = kKeysPerTile * kCRow;   // kv_c part of a tile
constexpr int kPeRow = kDr * 2;                 // 128 B, 16-byte chunks XOR-swizzled by key
constexpr int kBufBytes = kCBytes + kKeysPerTile * kPeRow;  // 41472
constexpr int kPBytes = kRows * kKeysPerTile * 2;           // 8192 per tile, double-buffered
// Page-table entries travel global -> LDS too, into a ring of kIdxRing tiles,
// kIdxLead tiles before the keys they name are fetched; the addresses of a
// tile's loads are prepared one iteration before the loads are issued.
constexpr int kIdxRing = 4;
constexpr int kIdxLead = 3;
constexpr int kIdxBytes = kIdxRing * kKeysPerTile * 4;      // 512
constexpr int kAncBytes = kRows * kMaskWords * 8;             // ancestor mask words of each row
// The rope part of Q (64 features of each row) as each lane's four MFMA
// operand fragments, [wave][fragment][lane] x 16 bytes.
constexpr int kQpeBytes = kRows * kDr * 2;                     // 16384
constexpr int kSmem = kNbuf * kBufBytes + 2 * kPBytes + kIdxBytes + kAncBytes + kQpeBytes;
// Vector-memory stores one wave issues for a split partial: (m, l) plus
// 4 row blocks x 4 feature blocks x 2 16-byte pieces. The wait after a split
// boundary lets this many operations stay outstanding; it is safe as long as
// the compiler emits at least this many store instructions, which holds
// because no two of these stores are adjacent in memory (none can merge) and
// none is wider than the widest store instruction.
constexpr int kPartialStores = 1 + 4 * 4 * 2;
// Vector-memory instructions each wave issues per tile: 8 kv_c rows, one
// block of 8 k_pe rows, one block of 8 page-table entries.
constexpr int kVmemPerTile = 10;
static_assert(kSmem <= 160 * 1024, "LDS budget");
// Trees above 64 nodes build their masks in the P buffers before first use.
static_assert(kTreeScratchBytes <= 2 * kPBytes, "tree mask scratch");
}  // namespace bf16k

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// The global -> LDS copies below are issued as inline asm so that the
// compiler's own wait insertion does not treat every later LDS read as
// dependent on them (which would drain the whole prefetch ring); the kernel
// waits for them explicitly with wait_vmem<>. Vector-memory loads retire in
// order, so the compiler's waits for its own loads stay correct.

// Lanes 0..7 fetch the page-table entries of this wave's 8 keys of `tile`
// into ring slot tile % kIdxRing (one global_load_lds_dword; tile >= 0 and
// kIdxRing is a power of two). Positions past
// `jmax` (the split's last key) are clamped to it: those keys are loaded but
// either masked out of the softmax (past the sequence) or never computed
// (past the split), and their data is a real, finite token.
__device__ __forceinline__ void issue_tile_index(const VerifyArgs& a, char* idx_ring, int kv0, int jmax,
                                                 int tile) {
  using namespace bf16k;
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6;
  if (lane < 8) {
    const int j = min(tile * kKeysPerTile + wave * 8 + lane, jmax);
    const uint32_t m0 =
        __builtin_amdgcn_readfirstlane(lds_addr(idx_ring + ((tile & (kIdxRing - 1)) * kKeysPerTile + wave * 8) * 4));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(m0),
                 "v"((uint64_t)(a.kv_indices + kv0 + j))
                 : "memory", "m0");
  }
}

// Slots of this wave's 8 keys of `tile` (lane & 7 -> key), read back from the
// index ring once this wave's load of them has completed.
__device__ __forceinline__ int tile_slots(const char* idx_ring, int tile) {
  using namespace bf16k;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6;
  return *(const int*)(idx_ring + ((tile & (kIdxRing - 1)) * kKeysPerTile + wave * 8 + (lane_id() & 7)) * 4);
}

// Loads of this wave's share of one tile (keys 8w..8w+7) into an LDS buffer,
// with every address prepared once so that each load is a couple of
// instructions: the 64-bit kv_c row addresses sit in lanes 0..7, the k_pe
// address is per lane. Parts 0..7 are the kv_c rows (1 KB, one 64-lane
// 16-byte load from a scalar row address each); part 8 is the eight 128-byte
// k_pe rows together, lane i fetching chunk (i%8) ^ (i/8) so that the chunks of
// one key land XOR-swizzled by the key index.
constexpr int kTileParts = 9;
struct TileLoads {
  uint32_t row_lo, row_hi;  // lanes 0..7: kv_c row address of key 8w + lane
  uint64_t kpe;             // per lane: k_pe chunk address
  uint32_t lds_base;        // wave-uniform: LDS address of this wave's first row
};

// prepare_tile in three steps (so a loop can spread them between MFMAs):
// kv_c row addresses, then the lane shuffle for k_pe, then the k_pe address.
// buf_lds: LDS address of the destination buffer.
__device__ __forceinline__ void prepare_rows(TileLoads& t, const VerifyArgs& a, uint32_t buf_lds, int slots, int wave) {
  using namespace bf16k;
  const uint64_t row = (uint64_t)(uintptr_t)a.kv_c + (uint64_t)(int64_t)slots * (uint64_t)a.kv_c_stride * 2u;
  t.row_lo = (uint32_t)row;
  t.row_hi = (uint32_t)(row >> 32);
  t.lds_base = buf_lds + wave * 8 * kCRow;
}
__device__ __forceinline__ int prepare_kpe_slot(int slots) { return shfl_i32(slots, lane_id() >> 3); }
__device__ __forceinline__ void prepare_kpe(TileLoads& t, const VerifyArgs& a, int kslot) {
  const int lane = lane_id();
  const int chunk = (lane & 7) ^ (lane >> 3);
  t.kpe = (uint64_t)(uintptr_t)a.k_pe + ((uint64_t)(int64_t)kslot * (uint64_t)a.k_pe_stride + chunk * 8) * 2u;
}
__device__ __forceinline__ TileLoads prepare_tile(const VerifyArgs& a, const char* buf, int slots, int wave) {
  TileLoads t;
  prepare_rows(t, a, lds_addr(buf), slots, wave);
  prepare_kpe(t, a, prepare_kpe_slot(slots));
  return t;
}

__device__ __forceinline__ void issue_tile_part(const TileLoads& t, int wave, int part) {
  using namespace bf16k;
  if (part < 8) {
    // readlane returns int: widen through uint32_t so the low word is not sign-extended.
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)t.row_lo, part);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)t.row_hi, part);
    const uint64_t row = ((uint64_t)hi << 32) | (uint64_t)lo;
    const uint32_t m0 = t.lds_base + part * kCRow;
    // s_nop 4: the scalar base was just written by v_readlane, and a VMEM read
    // of a VALU-written SGPR needs 5 wait states; it also covers the one wait
    // state between writing M0 and an LDS-DMA load.
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0),
                 "v"((uint32_t)lane_id() * 16), "s"(row)
                 : "memory", "m0");
  } else {
    const uint32_t m0 = t.lds_base - wave * 8 * kCRow + kCBytes + wave * 8 * kPeRow;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(t.kpe)
                 : "memory", "m0");
  }
}

__device__ __forceinline__ void issue_tile(const TileLoads& t, int wave) {
#pragma unroll
  for (int part = 0; part < kTileParts; ++part) issue_tile_part(t, wave, part);
}

// S^T[32 keys x 32 rows] = K . Q^T for this wave's rows from LDS tile `buf`:
// 9 batches of 4 MFMAs over the 576 features. Batch kQkRopeBatch is the rope
// part, with both operands from LDS (Q's rope fragments live there, at `qpe`
// for this lane, to spare 16 registers); the others take the latent part of Q
// from registers. First is best (measured: the middle costs 1.5%, the end
// 18%, where its extra operand registers meet the PV prefetch). Each batch's
// LDS reads are issued during the previous batch; the scheduling barriers
// stop the compiler from hoisting every read at once. between(kb) runs after
// the MFMAs of batch kb.
constexpr int kQkRopeBatch = 0;
// With kQpePreloaded the caller has already read the rope part of Q into
// qf_pre (the tile loop reads it across its barrier); otherwise qf_pre is
// unused and it is read here.
template <bool kQpePreloaded, typename Between>
__device__ __forceinline__ f32x16_t qk_tile(const char* buf, const bf16x8_t (&qreg)[32], const char* qpe, int k_off,
                                            int kpe_off, int kpe_sw, int half, const bf16x8_t (&qf_pre)[4],
                                            Between&& between) {
  f32x16_t sacc;
#pragma unroll
  for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
  bf16x8_t kf[2][4], qf[4];
  if constexpr (kQpePreloaded) {
#pragma unroll
    for (int j = 0; j < 4; ++j) qf[j] = qf_pre[j];
  }
  auto load_batch = [&](int b, bf16x8_t (&dst)[4]) {
    if (b == kQkRopeBatch) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dst[j] = *(const bf16x8_t*)(buf + kpe_off + (((2 * j + half) ^ kpe_sw) << 4));
        if constexpr (!kQpePreloaded) qf[j] = *(const bf16x8_t*)(qpe + j * 64 * 16);
      }
    } else {
      const int c0 = 4 * (b < kQkRopeBatch ? b : b - 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[j] = *(const bf16x8_t*)(buf + k_off + (c0 + j) * 32);
    }
  };
  load_batch(0, kf[0]);
#pragma unroll
  for (int kb = 0; kb < 9; ++kb) {
    if (kb + 1 < 9) load_batch(kb + 1, kf[(kb + 1) & 1]);
    // Keep the reads of batch kb+1 ahead of the MFMAs of batch kb (left to
    // itself the scheduler sinks them below and reuses the registers).
    __builtin_amdgcn_sched_barrier(0);
    const int c0 = 4 * (kb < kQkRopeBatch ? kb : kb - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb & 1][j], kb == kQkRopeBatch ? qf[j] : qreg[c0 + j], sacc, 0,
                                                     0, 0);
    between(kb);
    __builtin_amdgcn_sched_barrier(0);
  }
  return sacc;
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

__global__ void __launch_bounds__(bf16k::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_verify_attn_bf16_kernel(const VerifyArgs a) {
  using namespace bf16k;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  char* const pbuf0 = smem + kNbuf * kBufBytes;
  char* const idx_ring = pbuf0 + 2 * kPBytes;
  uint64_t* const anc_lds = (uint64_t*)(idx_ring + kIdxBytes);
  char* const qpe_lds = idx_ring + kIdxBytes + kAncBytes;

  BlockWork w;
  if (!map_block(a, w, kRows)) return;
  const int H = a.heads;

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6;  // uniform: keep it scalar
  const int half = lane >> 5;   // k slice of MFMA operands / key quartet of S^T rows
  const int qcol = lane & 31;   // column of the 32x32 blocks

  // The page-table entries of the first three tiles go out first, so that
  // their round trip overlaps the loads of Q and of the tree.
  const int jmax0 = min(w.N, w.tile_end * kKeysPerTile) - 1;
  if (w.tile_begin < w.tile_end) {
#pragma unroll
    for (int t = 0; t < 3; ++t) issue_tile_index(a, idx_ring, w.kv0, jmax0, w.tile_begin + t);
  }

  // ---- QK role: this lane's query row (wave owns rows 32w..32w+31) ---------
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
  // the tile loop. Only the QK owner (half 0) writes it; the first barrier of
  // the pipeline orders the write before every read. Trees of up to 64 nodes
  // take the one-wave builder; larger ones are built by the workgroup in the
  // P buffers, which are first written after that barrier.
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
      block_tree_masks<kThreads>(a.parents + w.node0, w.T, pbuf0);
      const uint64_t* src = tree_scratch_masks(pbuf0) + (r_eff / H) * kMaskWords;
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
  // Whether this lane's row belongs to a valid node (its mask is not empty).
  auto row_valid = [&]() {
    int i = wave * 32 + qcol;
    asm volatile("" : "+v"(i));
    uint64_t any = 0;
#pragma unroll
    for (int k = 0; k < kMaskWords; ++k) any |= anc_lds[i * kMaskWords + k];
    return any != 0;
  };

  // Per-lane LDS address pieces.
  // K (A operand of QK): key = qcol, 8 features at 16*kc + 8*half.
  const int k_off = qcol * kCRow + half * 16;
  const int kpe_off = kCBytes + qcol * kPeRow;
  const int kpe_sw = qcol & 7;
  // V^T (A operand of PV) via transpose reads: 16-lane group g reads 4 keys x
  // 16 features; lane i of the group points at key 4*half + i/4, features
  // 16*(g%2) + 4*(i%4) of this wave's feature range.
  const int g16 = lane >> 4, i16 = lane & 15;
  const int v_off = (4 * half + (i16 >> 2)) * kCRow + (16 * (g16 & 1) + 4 * (i16 & 3)) * 2 + wave * 4 * 64;

  // Softmax state of this lane's row (same rules as the fp32 kernel):
  // m_ref = reference max (log2 units, scaled) fixed at the first tile where
  // the row sees a key; weights are 2^(s - m_ref); if some score exceeds it by
  // more than kOverflowSlack the block repeats the split with the exact max.
  f32x16_t oacc[16];  // [f4 * 4 + rb]: feature block 4*wave + f4, row block rb
  float m_ref = -INFINITY, m_max = -INFINITY, l_run = 0.f;
  // Split boundaries inside the group: the weight sum of a tile that starts
  // the next split stays out of l_run (it is still in sm.psum when the split
  // ends, and starts the next split's sum).
  bool next_starts_split = false;
  const int s_first = w.s, c_first = w.c;

  // Invisible keys of one S^T block get -inf (only tiles that reach the tree
  // tail or the end of the sequence need this; register i holds key
  // k0 + (i/4)*8 + 4*half + i%4).
  auto mask_tile = [&](f32x16_t& sacc, int k0) {
    const uint32_t hwin = row_window(k0 - w.P) >> (4 * half);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = k0 + (i >> 2) * 8 + half * 4 + (i & 3);
      const bool tail_bit = ((hwin >> ((i >> 2) * 8 + (i & 3))) & 1u) != 0;
      const bool vis = (j < w.P) | ((j < w.N) & tail_bit);
      sacc[i] = vis ? sacc[i] : -INFINITY;
    }
  };
  // Weights of one (masked) tile for this lane's row, 2^(scale*s*log2e -
  // m_ref), written as bf16 P^T fragments to P buffer `pb` for every wave.
  // Split into steps 0..27 so the PV loop can interleave them with its MFMAs;
  // step k only uses results of earlier steps. The max is taken on raw scores
  // (scale > 0 keeps the order).
  struct SoftmaxState {
    float m[6], mloc, mswap, nmu, psum, p[16];
    bf16x8_t pk[2];
  } sm;
  auto softmax_step = [&](int k, const f32x16_t& sc, char* pb, bool& overflow) {
    if (k == 0) {
      sm.m[0] = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
      sm.m[1] = fmaxf(fmaxf(sc[3], sc[4]), sc[5]);
    } else if (k == 1) {
      sm.m[2] = fmaxf(fmaxf(sc[6], sc[7]), sc[8]);
      sm.m[3] = fmaxf(fmaxf(sc[9], sc[10]), sc[11]);
    } else if (k == 2) {
      sm.m[4] = fmaxf(fmaxf(sc[12], sc[13]), sc[14]);
      sm.mloc = fmaxf(fmaxf(fmaxf(sm.m[0], sm.m[1]), sm.m[2]), fmaxf(fmaxf(sm.m[3], sm.m[4]), sc[15]));
    } else if (k == 3) {
      sm.mswap = swap_halves(sm.mloc);
    } else if (k == 4) {
      const float mx = fmaxf(sm.mloc, sm.mswap) * a.scale_log2;  // row max of the tile, log2 units
      m_max = fmaxf(m_max, mx);
      if (m_ref == -INFINITY) m_ref = mx;
      overflow |= mx > m_ref + kOverflowSlack;
      sm.nmu = m_ref == -INFINITY ? 0.f : -m_ref;
      sm.psum = 0.f;
    } else if (k >= 5 && k < 21) {
      const int i = k - 5;
      sm.p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], a.scale_log2, sm.nmu));
      sm.psum += sm.p[i];
    } else if (k == 21 || k == 22) {
      const int u = k - 21;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) sm.pk[u][jj] = (__bf16)sm.p[8 * u + jj];
    } else if (k == 23 || k == 24) {
      const int u = k - 23;
      *(bf16x8_t*)(pb + ((wave * 2 + u) * 64 + lane) * 16) = sm.pk[u];
    } else if (k == 25) {
      if (!next_starts_split) l_run += sm.psum;
    }
  };
  constexpr int kSoftmaxSteps = 26;
  constexpr int kSoftmaxLag = 3;  // PV MFMAs issued before the first softmax step
  auto softmax_to_lds = [&](const f32x16_t& sc, char* pb, bool& overflow) {
#pragma unroll
    for (int k = 0; k < kSoftmaxSteps; ++k) softmax_step(k, sc, pb, overflow);
  };
  // A tile needs masking when it reaches the tree tail (or the sequence end).
  auto needs_mask = [&](int k0) { return k0 + kKeysPerTile > w.P; };

  // Partial of global split c (sequences with several splits): (m, l) from the QK
  // owner lanes of each row, and this wave's raw O^T blocks in bf16 (half the
  // bytes of fp32; the rounding is relative to each partial and averages out
  // in the merge). No exchange between waves, so no barrier.
  // Accumulator register i of block (f4, rb) holds feature
  // 32*(4*wave + f4) + (i/4)*8 + 4*half + i%4 of row 32*rb + qcol.
  //
  // The partial arrays have a.part_rows (a multiple of kRows) rows per split,
  // so the rows past T_b * H of the last row block have room and every
  // store below is unconditional: exactly kPartialStores vector-memory
  // instructions, which the wait after a split boundary relies on.
  auto emit_partial = [&](int c, float l_part) {
    // Lane indices taken afresh (an opaque copy), so that no address below is
    // computed ahead of the tile loop and kept live through it.
    int lq = lane;
    asm volatile("" : "+v"(lq));
    const int qcol = lq & 31, half = lq >> 5;
    const float l_tot = l_part + swap_halves(l_part);
    const bool node_ok = row_valid();
    mfma_result_wait();  // the last PV MFMAs may have just been issued
    // (m, l) of the row; both lanes of a row hold the same values.
    const int64_t prow = (int64_t)c * a.part_rows + w.rb * kRows + wave * 32 + qcol;
    *(float2*)(a.part_ml + 2 * prow) = make_float2(node_ok ? m_ref : NAN, node_ok ? l_tot : NAN);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int r = w.rb * kRows + rb * 32 + qcol;
      __bf16* dst = (__bf16*)a.part_o + ((int64_t)c * a.part_rows + r) * kDl + 8 * half;
#pragma unroll
      for (int f4 = 0; f4 < 4; ++f4)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          // Values 2m and 2m+1 (features 16m + 4*half + 0..3 and 16m + 8 +
          // 4*half + 0..3) become 8 consecutive features per lane by one
          // exchange between the wave halves: the lower half keeps 16m..16m+7,
          // the upper half gets 16m+8..16m+15.
          const f32x4_t t0 = read_acc4(oacc[f4 * 4 + rb], 2 * m);
          const f32x4_t t1 = read_acc4(oacc[f4 * 4 + rb], 2 * m + 1);
          uint32_t x[2], y[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            x[e] = pack_bf16x2(t0[2 * e], t0[2 * e + 1]);
            y[e] = pack_bf16x2(t1[2 * e], t1[2 * e + 1]);
            const auto sw = __builtin_amdgcn_permlane32_swap(x[e], y[e], false, false);
            x[e] = sw[0];
            y[e] = sw[1];
          }
          *(u32x4_t*)(dst + 32 * (4 * wave + f4) + 16 * m) = u32x4_t{x[0], x[1], y[0], y[1]};
          // One pair at a time: otherwise the scheduler reads every
          // accumulator out at once and runs out of registers.
          __builtin_amdgcn_sched_barrier(0);
        }
    }
  };
  // Output of a sequence with one split: O / l and lse; each row's
  // statistics travel from its QK owner to every wave through LDS.
  auto emit_final = [&]() {
    const float l_tot = l_run + swap_halves(l_run);
    float2* stats = (float2*)pbuf0;  // the P buffers are free after the loop
    const bool node_ok = row_valid();
    mfma_result_wait();
    __syncthreads();
    if (half == 0) stats[wave * 32 + qcol] = make_float2(node_ok ? m_ref : NAN, l_tot);
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int r = w.rb * kRows + rb * 32 + qcol;
      if (r >= w.rows) continue;
      const float2 st = stats[rb * 32 + qcol];
      const bool ok = !(st.x != st.x);
      const int64_t g = (int64_t)w.node0 * H + r;
      float* dst = a.out + g * kDl;
      const float mul = ok ? 1.f / st.y : NAN;
      if (wave == 0 && half == 0 && a.lse) a.lse[g] = ok ? (st.x + __log2f(st.y)) * kLn2 : NAN;
#pragma unroll
      for (int f4 = 0; f4 < 4; ++f4)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const f32x4_t v = read_acc4(oacc[f4 * 4 + rb], gi);
          *(f32x4_t*)(dst + 32 * (4 * wave + f4) + 8 * gi + 4 * half) = v * mul;
        }
    }
  };

  for (int pass = 0; pass < 2; ++pass) {
    l_run = 0.f;
    next_starts_split = false;
    bool overflow = false;

    if (w.tile_begin < w.tile_end) {
      const int tb = w.tile_begin, te = w.tile_end;
      const int jmax = min(w.N, te * kKeysPerTile) - 1;
      // Pipeline. Iteration t: tiles t and t+1 are in LDS, tile t+2 and the
      // page-table entries of t+2+kIdxLead are fetched; QK and softmax of
      // tile t+1 run while the PV of tile t (whose weights every wave wrote in
      // the previous iteration) keeps the matrix cores busy. Tiles past the
      // split repeat its last key (loaded, never computed), which keeps the
      // number of loads per iteration constant.
      if (pass > 0) {  // pass 0 issued these at the start
        issue_tile_index(a, idx_ring, w.kv0, jmax, tb);
        issue_tile_index(a, idx_ring, w.kv0, jmax, tb + 1);
        issue_tile_index(a, idx_ring, w.kv0, jmax, tb + 2);
      }
      wait_vmem<0>();
      issue_tile(prepare_tile(a, smem + (tb % kNbuf) * kBufBytes, tile_slots(idx_ring, tb), wave), wave);
      issue_tile_index(a, idx_ring, w.kv0, jmax, tb + kIdxLead);
      issue_tile(prepare_tile(a, smem + ((tb + 1) % kNbuf) * kBufBytes, tile_slots(idx_ring, tb + 1), wave), wave);
      issue_tile_index(a, idx_ring, w.kv0, jmax, tb + 1 + kIdxLead);
      // Loads of tile tb+2, issued at the top of the first iteration.
      TileLoads pending =
          prepare_tile(a, smem + ((tb + 2) % kNbuf) * kBufBytes, tile_slots(idx_ring, tb + 2), wave);
      wait_vmem<kVmemPerTile + 1>();  // this wave's part of tile tb
      block_sync();
      {
        bf16x8_t qf_none[4];
        f32x16_t s0 = qk_tile<false>(smem + (tb % kNbuf) * kBufBytes, qreg, qpe_lane, k_off, kpe_off, kpe_sw, half,
                                     qf_none, [](int) {});
        if (needs_mask(tb * kKeysPerTile)) mask_tile(s0, tb * kKeysPerTile);
        softmax_to_lds(s0, pbuf0 + (tb & 1) * kPBytes, overflow);
      }

      // Byte offsets of the buffers of tiles t, t+1 and t+2, rotated each
      // iteration (tile t+3 reuses the buffer of tile t).
      int bo0 = (tb % kNbuf) * kBufBytes, bo1 = ((tb + 1) % kNbuf) * kBufBytes, bo2 = ((tb + 2) % kNbuf) * kBufBytes;
      int tile = tb;
      // The splits of the group (at least one), one after the other; the
      // tile pipeline runs on across their boundaries.
      int sp = s_first;
      do {
#pragma unroll
      for (int x = 0; x < 16; ++x)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[x][i] = 0.f;
      const int split_begin = tile, split_end = split_tile(sp + 1, w.ntiles, w.S);
      for (; tile < split_end; ++tile) {
        // Everything this wave issued in the previous iteration (the keys of
        // tile+1 and the index block of tile+1+kIdxLead) has landed. After a
        // split boundary the partial's stores, issued after those loads, may
        // still be on their way.
        if (tile == split_begin && sp != s_first) wait_vmem<kPartialStores>();
        else wait_vmem<0>();
        wait_lds();
        // The rope part of Q is this lane's own LDS data, written once before
        // the loop, so its reads may cross the barrier: the batch that follows
        // it then waits for the key reads alone (measured 0.5-1.3% faster).
        bf16x8_t qf_pre[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) qf_pre[j] = *(const bf16x8_t*)(qpe_lane + j * 64 * 16);
        block_sync();  // P(tile) and tile+1 are visible; every wave has finished PV(tile-1)
        // Tile+2 goes into the buffer tile-1 used; its addresses were prepared
        // during the previous iteration. One load goes after each QK batch (a
        // burst of all nine from every wave queues in the vector-memory path
        // and stalls the issuing waves), the page-table block with the first.
        const char* buf = smem + bo0;
        const char* pb = pbuf0 + (tile & 1) * kPBytes;
        // Does tile+1 start the next split of the group?
        next_starts_split = tile + 1 == split_end && tile + 1 < te;
        // PV operands: P^T fragments [u][rb] and V^T fragments of two groups.
        // The first ones are read during the last QK batch so that the first
        // PV MFMA does not wait for them.
        bf16x8_t pbr[2][4];
        i16x4_t vf[2][2];
        auto load_v = [&](int g, i16x4_t (&dst)[2]) {
          const char* vp = buf + v_off + (16 * (g >> 2)) * kCRow + (g & 3) * 64;
          dst[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)vp);
          dst[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vp + 8 * kCRow));
        };
        auto load_p = [&](int u) {
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) pbr[u][rb] = *(const bf16x8_t*)(pb + ((rb * 2 + u) * 64 + lane) * 16);
        };
        auto late_part = [&](int kb) {
          issue_tile_part(pending, wave, kb);
          if (kb == 0) issue_tile_index(a, idx_ring, w.kv0, jmax, tile + 2 + kIdxLead);
          if (kb == 7) {
            load_p(0);
            load_v(0, vf[0]);
          }
        };
        // Scores of tile+1. On the last tile there is none: all -inf (set in
        // the PV loop) makes the softmax steps a no-op for the row state.
        f32x16_t snext;
        const int k1 = (tile + 1) * kKeysPerTile;
        const bool has_next = tile + 1 < te;
        if (has_next) {
          snext = qk_tile<true>(smem + bo1, qreg, qpe_lane, k_off, kpe_off, kpe_sw, half, qf_pre, late_part);
        } else {
          issue_tile(pending, wave);
          issue_tile_index(a, idx_ring, w.kv0, jmax, tile + 2 + kIdxLead);
          load_p(0);
          load_v(0, vf[0]);
          // snext stays unset here: it is set to -inf below (a value
          // assigned here would make the compiler move the QK result out of
          // the accumulation registers right after the QK, to merge the two).
        }
        __builtin_amdgcn_sched_barrier(0);

        // ---- O^T[this wave's 128 features x 128 rows] += V^T . P^T (tile),
        //      with the weights of tile+1 (VALU) threaded between the MFMAs.
        // Group g = (u, f4) = (g/4, g%4) issues 4 MFMAs (row blocks); V^T for
        // group g+1 and P^T for u=1 are read one group ahead.
        // Addresses of tile+3's loads (entries landed before this iteration's
        // wait), prepared in steps between the PV MFMAs.
        int pslots = 0, pkslot = 0;
        auto prepare_step = [&](int k) {
          if (k == 0) pslots = tile_slots(idx_ring, tile + 3);
          else if (k == 10) {
            prepare_rows(pending, a, lds_addr(smem) + (uint32_t)bo0, pslots, wave);
            pkslot = prepare_kpe_slot(pslots);
          } else if (k == 20) prepare_kpe(pending, a, pkslot);
        };
        {
#pragma unroll
          for (int g = 0; g < 8; ++g) {
            if (g + 1 < 8) load_v(g + 1, vf[(g + 1) & 1]);
            if (g == 2) load_p(1);
            const bf16x8_t va = __builtin_bit_cast(
                bf16x8_t, __builtin_shufflevector(vf[g & 1][0], vf[g & 1][1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int rb = (rr + 1) & 3;  // row block 0 last (see below)
              const int f4 = g & 3;
              oacc[f4 * 4 + rb] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pbr[g >> 2][rb], oacc[f4 * 4 + rb], 0, 0, 0);
              const int k = 4 * g + rr;
              if (k == kSoftmaxLag - 1) {
                // The scores of tile+1 leave the accumulation registers only
                // here, behind the first PV MFMAs: read right after the last
                // QK MFMA they would stall the wave until the matrix pipe
                // drains. (The compiler parks the QK accumulator where an
                // output block lives; that block's first MFMA comes after.)
                asm volatile("" : "+v"(snext));
                if (!has_next) {
#pragma unroll
                  for (int i = 0; i < 16; ++i) snext[i] = -INFINITY;
                } else if (needs_mask(k1)) {
                  mask_tile(snext, k1);
                }
              }
              if (k >= kSoftmaxLag && k - kSoftmaxLag < kSoftmaxSteps)
                softmax_step(k - kSoftmaxLag, snext, pbuf0 + ((tile + 1) & 1) * kPBytes, overflow);
              prepare_step(k);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
        const int bt = bo0;
        bo0 = bo1;
        bo1 = bo2;
        bo2 = bt;
      }
      // Split sp is complete: its partial goes out (a redo pass rewrites
      // it), and the weight sum of the next split's first tile, taken in the
      // last iteration, starts the next sum. A split can be empty when the
      // sequence is shorter than the plan assumed: its partial has l = 0 and
      // O = 0, and the carried sum waits for the next split with tiles.
      if (w.S > 1) {
        if (split_end > split_begin) {
          emit_partial(c_first + (sp - s_first), l_run);
          l_run = sm.psum;
        } else {
          emit_partial(c_first + (sp - s_first), 0.f);
        }
      }
      } while (++sp < w.s_last);
      wait_vmem<0>();
    } else {
      // No key tiles: empty partials (m = -inf, l = 0, O = 0).
#pragma unroll
      for (int x = 0; x < 16; ++x)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[x][i] = 0.f;
      if (w.S > 1)
        for (int sp = s_first; sp < w.s_last; ++sp) emit_partial(c_first + (sp - s_first), 0.f);
    }
    if (pass == 1 || !__syncthreads_or(overflow)) break;
    m_ref = m_max;
  }

  // ---- epilogue: a sequence with one split writes its output -------------
  if (w.S == 1) emit_final();
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
  if (!map_block(a, w, kRows)) return;
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
  if (w.S == 1) {
    dst = a.out + grow * kDl;
    mul = node_ok ? 1.f / l_tot : NAN;
    if (half == 0 && a.lse) a.lse[grow] = node_ok ? (m_ref + __log2f(l_tot)) * kLn2 : NAN;
  } else {
    const int64_t prow = (int64_t)w.c * a.part_rows + r_eff;
    dst = (float*)a.part_o + prow * kDl;
    mul = 1.f;
    if (half == 0) {
      a.part_ml[2 * prow] = node_ok ? m_ref : NAN;
      a.part_ml[2 * prow + 1] = node_ok ? l_tot : NAN;
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
// Merge the split partials of kCombineRows consecutive query rows of one
// sequence: M = max m_c, w_c = 2^(m_c - M), L = sum w_c l_c,
// out = sum w_c O_c / L, lse = (M + log2 L) ln 2. Partials O_c are fp32 (fp32
// problems) or bf16 (bf16 problems). Each row
// has 4 groups of 32 lanes (16 features per lane); group g sums the splits
// c = g (mod 4), and the groups' sums meet in LDS. The rows of a workgroup
// are adjacent in every split's partial block. Empty splits (m = -inf) get
// weight 0 (their partial is zeros); a NaN partial (invalid tree) makes the
// row NaN.
constexpr int kCombineRows = 2;
constexpr int kCombineGroups = 4;
constexpr int kCombineThreads = 32 * kCombineGroups * kCombineRows;
constexpr int kCombineStage = 256;

template <typename PartT>
__global__ void __launch_bounds__(kCombineThreads) mla_verify_combine_kernel(const VerifyArgs a) {
  constexpr bool kBf16 = sizeof(PartT) == 2;
  __shared__ float wsh[kCombineRows][kCombineStage];
  __shared__ float lsh[kCombineRows][kCombineGroups];
  __shared__ f32x4_t accsh[kCombineRows][kCombineGroups - 1][32][4];
  const int row_groups = (a.max_rows_per_seq + kCombineRows - 1) / kCombineRows;
  const int b = (int)(blockIdx.x / row_groups);
  int node0, T;
  seq_tree(a, b, node0, T);
  const int rows = T * a.heads;
  const int tid = threadIdx.x;
  const int j = tid / (32 * kCombineGroups), grp = (tid >> 5) % kCombineGroups, t32 = tid & 31;
  const int r = (int)(blockIdx.x % row_groups) * kCombineRows + j;
  const int s0 = a.split_offset[b];
  const int S = a.split_offset[b + 1] - s0;
  // Whole workgroup: no split partials, or every row past this sequence's rows.
  if (S <= 1 || (int)(blockIdx.x % row_groups) * kCombineRows >= rows) return;
  const bool live = r < rows;
  const int rr = live ? r : rows - 1;
  const float* ml = a.part_ml + 2 * ((int64_t)s0 * a.part_rows + rr);
  const int64_t ml_stride = 2 * (int64_t)a.part_rows;

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
  // Lane t32 of a group holds 16 of the row's 512 features: for bf16 the
  // 8-feature runs starting at 8*t32 and 256 + 8*t32, for fp32 the 4-feature
  // runs at 4*t32 + 128*q, so that each load instruction of a group reads
  // 512 contiguous bytes.
  const PartT* po = (const PartT*)a.part_o + ((int64_t)s0 * a.part_rows + rr) * kDl + (kBf16 ? 8 : 4) * t32;
  const int64_t po_stride = (int64_t)a.part_rows * kDl;
  for (int base = 0; base < S; base += kCombineStage) {
    const int cnt = min(kCombineStage, S - base);
    __syncthreads();
    if (grp == 0) {
      for (int cc = t32; cc < cnt; cc += 32) {
        const float m = ml[(base + cc) * ml_stride];
        const float l = ml[(base + cc) * ml_stride + 1];
        const float wgt = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
        wsh[j][cc] = wgt;
        lloc += wgt * l;
      }
    }
    __syncthreads();
    // Unconditional loads (an empty split's partial is zeros with weight 0),
    // so that several are in flight at once.
#pragma unroll 4
    for (int cc = grp; cc < cnt; cc += kCombineGroups) {
      const float wgt = wsh[j][cc];
      const PartT* src = po + (base + cc) * po_stride;
      if constexpr (kBf16) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const bf16x8_t v = *(const bf16x8_t*)(src + 256 * q);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * q][e] += wgt * (float)v[e];
            acc[2 * q + 1][e] += wgt * (float)v[4 + e];
          }
        }
      } else {
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
    // acc[q]: features 8*t32 + 256*(q/2) + 4*(q%2) (bf16) or 4*t32 + 128*q (fp32).
    const int f = kBf16 ? 8 * t32 + 256 * (q >> 1) + 4 * (q & 1) : 4 * t32 + 128 * q;
    *(f32x4_t*)(a.out + grow * kDl + f) = acc[q] * inv;
  }
  if (t32 == 0 && a.lse) a.lse[grow] = nan ? NAN : (M + __log2f(lloc)) * kLn2;
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
  const int64_t groups = (int64_t)a.batch * ((a.max_rows_per_seq + kCombineRows - 1) / kCombineRows);
  if (groups == 0) return 0;
  if (dtype == MLA_DTYPE_BF16)
    hipLaunchKernelGGL(mla_verify_combine_kernel<__bf16>, dim3((unsigned)groups), dim3(kCombineThreads), 0,
                       (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(mla_verify_combine_kernel<float>, dim3((unsigned)groups), dim3(kCombineThreads), 0,
                       (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_tree_masks(const int32_t* parents, int32_t batch, int32_t tree_nodes, uint64_t* masks,
                      void* stream) {
  hipLaunchKernelGGL(mla_tree_masks_kernel, dim3(batch), dim3(kTreeMaskThreads), 0, (hipStream_t)stream,
                     parents, tree_nodes, masks);
  return (int)hipGetLastError();
}

}  // namespace mlav
