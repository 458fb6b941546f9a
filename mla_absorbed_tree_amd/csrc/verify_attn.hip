// Tree-verify attention for absorbed-form MLA on gfx950 (MI355X).
//
// Per query row (b, t, h): score(j) = scale * (q_nope . kv_c[j] + q_pe . k_pe[j])
// over the prefix and the node's ancestor-or-self tree tail, softmax, then the
// weighted sum of kv_c (latent-space output) and the log-sum-exp.
//
// Work decomposition: one workgroup per (sequence b, block of query rows, KV
// split). A KV tile of 32 keys (kv_c | k_pe, 1152 B per key in bf16) is staged
// in LDS once and serves every query row of the block: 128 rows (4 waves x 32)
// in bf16, so a head-shared latent is read from L2 once per 128 rows instead
// of once per head (the "64x redundant reads" of a per-head kernel).
//
// Per wave, per 32-key step (bf16):
//   S^T[32 keys x 32 rows] = K[32 x 576] . Q^T      36 x mfma_f32_32x32x16_bf16
//       A = K from LDS (ds_read_b128), B = Q held in VGPRs for the whole split
//   online softmax on S^T in fp32 (exp2 domain), P rounded to bf16
//   O^T[512 x 32 rows] += V^T[512 x 32] . P^T       32 x mfma_f32_32x32x16_bf16
//       A = V^T via ds_read_b64_tr_b16 from the same LDS tile, B = P^T from VGPRs
// O^T lives in 256 accumulation registers per lane (16 blocks of 32x32 fp32).
// The key order inside each 16-deep MFMA step is permuted consistently in P^T
// and V^T so that P^T comes straight from the S^T accumulator layout.
//
// The fp32 instance (parity workloads in fp32) keeps the same structure with
// mfma_f32_32x32x2_f32, one wave of 32 rows, and Q staged in LDS.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernel_params.h"
#include "plan.h"

namespace mlav {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr float kLn2 = 0.693147180559945309f;
// Largest excess (log2 units) of a score over the row's reference max that a
// pass accepts: weights stay below 2^64, far from fp32/bf16 overflow even when
// summed over millions of keys.
constexpr float kOverflowSlack = 64.f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ int shfl_i32(int v, int src_lane) {
  return __builtin_amdgcn_ds_bpermute(src_lane << 2, v);
}
__device__ __forceinline__ float shfl_f32(float v, int src_lane) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(v)));
}
// Value held by the lane in the other half of the wave (lane ^ 32).
__device__ __forceinline__ float swap_halves(float v) { return shfl_f32(v, lane_id() ^ 32); }

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

__global__ void __launch_bounds__(64) mla_tree_masks_kernel(const int32_t* __restrict__ parents, int T,
                                                            uint64_t* __restrict__ masks) {
  const int b = blockIdx.x;
  const uint64_t m = wave_tree_mask(parents + (int64_t)b * T, T);
  if (lane_id() < T) masks[(int64_t)b * T + lane_id()] = m;
}

template <bool kF32>
struct KCfg;
template <>
struct KCfg<false> {
  static constexpr int kWaves = 4;
  static constexpr int kEsz = 2;
};
template <>
struct KCfg<true> {
  static constexpr int kWaves = 1;
  static constexpr int kEsz = 4;
};

template <bool kF32>
struct KLayout {
  static constexpr int kWaves = KCfg<kF32>::kWaves;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRows = 32 * kWaves;
  static constexpr int kEsz = KCfg<kF32>::kEsz;
  // One LDS row per key: kv_c | k_pe, plus 16 B of padding so that the 32
  // keys read by one MFMA operand load start in different banks.
  static constexpr int kRowBytes = kDk * kEsz + 16;
  static constexpr int kTileBytes = kKeysPerTile * kRowBytes;
  static constexpr int kQBytes = kF32 ? 32 * kRowBytes : 0;
  static constexpr int kSmemBytes = kTileBytes + kQBytes;
};

// Stage keys [k0, k0 + 32) of sequence b into LDS (rows past N are zero).
template <bool kF32>
__device__ __forceinline__ void stage_tile(const VerifyArgs& a, char* smem, int kv0, int k0, int N) {
  using L = KLayout<kF32>;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  if constexpr (!kF32) {
    // Wave w stages keys 8w..8w+7: each kv_c row (1 KB) is one 64-lane
    // 16-byte load; the eight 128-byte k_pe rows together are another.
    const int kfirst = wave * 8;
    const int jl = k0 + kfirst + (lane & 7);
    int my_slot = 0;
    if (lane < 8 && jl < N) my_slot = a.kv_indices[kv0 + jl];
    const __bf16* kvc = (const __bf16*)a.kv_c;
    const __bf16* kpe = (const __bf16*)a.k_pe;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int key = kfirst + kk;
      const int slot = __builtin_amdgcn_readlane(my_slot, kk);
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (k0 + key < N) v = *(const u32x4_t*)(kvc + (int64_t)slot * a.kv_c_stride + lane * 8);
      *(u32x4_t*)(smem + key * L::kRowBytes + lane * 16) = v;
    }
    {
      const int kk = lane >> 3, ch = lane & 7;
      const int key = kfirst + kk;
      const int slot = shfl_i32(my_slot, kk);
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (k0 + key < N) v = *(const u32x4_t*)(kpe + (int64_t)slot * a.k_pe_stride + ch * 8);
      *(u32x4_t*)(smem + key * L::kRowBytes + kDl * 2 + ch * 16) = v;
    }
  } else {
    // One wave stages all 32 keys: kv_c rows are 2 KB (two loads each), four
    // 256-byte k_pe rows per load.
    const int jl = k0 + (lane & 31);
    int my_slot = 0;
    if (lane < 32 && jl < N) my_slot = a.kv_indices[kv0 + jl];
    const float* kvc = (const float*)a.kv_c;
    const float* kpe = (const float*)a.k_pe;
#pragma unroll 4
    for (int key = 0; key < kKeysPerTile; ++key) {
      const int slot = __builtin_amdgcn_readlane(my_slot, key);
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (k0 + key < N)
          v = *(const u32x4_t*)(kvc + (int64_t)slot * a.kv_c_stride + part * 256 + lane * 4);
        *(u32x4_t*)(smem + key * L::kRowBytes + part * 1024 + lane * 16) = v;
      }
    }
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int key = g * 4 + (lane >> 4), ch = lane & 15;
      const int slot = shfl_i32(my_slot, key);
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (k0 + key < N) v = *(const u32x4_t*)(kpe + (int64_t)slot * a.k_pe_stride + ch * 4);
      *(u32x4_t*)(smem + key * L::kRowBytes + kDl * 4 + ch * 16) = v;
    }
  }
}

template <bool kF32>
__global__ void __launch_bounds__(KLayout<kF32>::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_verify_attn_kernel(const VerifyArgs a) {
  using L = KLayout<kF32>;
  __shared__ __attribute__((aligned(16))) char smem[L::kSmemBytes];

  // ---- workgroup -> (row block, global split), XCD-aware -------------------
  // Consecutive workgroup ids go to different XCDs; give every row block of one
  // KV chunk the same XCD so the chunk streams through a single L2.
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds;
  const int local = bid / kXcds;
  const int rb = local % a.row_blocks;
  const int c = (local / a.row_blocks) * kXcds + xcd;
  if (c >= a.total_splits) return;
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.split_offset[mid] <= c) lo = mid;
    else hi = mid - 1;
  }
  const int b = lo;
  const int S = a.split_offset[b + 1] - a.split_offset[b];
  const int s = c - a.split_offset[b];

  const int T = a.tree_nodes, H = a.heads;
  const int kv0 = a.kv_indptr[b];
  const int N = a.kv_indptr[b + 1] - kv0;
  const int P = N - T;
  const bool seq_ok = P >= 0;
  const int ntiles = seq_ok ? (N + kKeysPerTile - 1) / kKeysPerTile : 0;
  const int tile_begin = (int)(((int64_t)s * ntiles) / S);
  const int tile_end = (int)(((int64_t)(s + 1) * ntiles) / S);

  // ---- this lane's query row ------------------------------------------------
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;     // which 8-wide k slice / which key quartets
  const int qcol = lane & 31;     // query column of the 32x32 blocks
  const int r_local = rb * L::kRows + wave * 32 + qcol;
  const bool row_ok = r_local < a.rows_per_seq;
  const int r_eff = row_ok ? r_local : a.rows_per_seq - 1;
  const int node = r_eff / H;
  const int64_t grow = (int64_t)b * a.rows_per_seq + r_eff;

  const uint64_t tmask = wave_tree_mask(a.parents + (int64_t)b * T, T);
  const uint32_t anc_lo = (uint32_t)shfl_i32((int)(uint32_t)tmask, node);
  const uint32_t anc_hi = (uint32_t)shfl_i32((int)(uint32_t)(tmask >> 32), node);
  const uint64_t anc = ((uint64_t)anc_hi << 32) | anc_lo;
  const bool node_ok = seq_ok && anc != 0;

  // ---- Q --------------------------------------------------------------------
  bf16x8_t qreg[kF32 ? 1 : 36];
  if constexpr (!kF32) {
    const __bf16* qn = (const __bf16*)a.q_nope + grow * kDl + half * 8;
    const __bf16* qp = (const __bf16*)a.q_pe + grow * kDr + half * 8;
#pragma unroll
    for (int kc = 0; kc < 32; ++kc) qreg[kc] = *(const bf16x8_t*)(qn + kc * 16);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) qreg[32 + kc] = *(const bf16x8_t*)(qp + kc * 16);
  } else {
    // Q rows of the wave into LDS: row qr = [q_nope | q_pe] in fp32.
    char* qs = smem + L::kTileBytes;
    for (int idx = lane; idx < 32 * 144; idx += 64) {
      const int qr = idx / 144, ch = idx % 144;
      const int rr = min(rb * L::kRows + qr, a.rows_per_seq - 1);
      const int64_t gr = (int64_t)b * a.rows_per_seq + rr;
      const float* src = ch < 128 ? (const float*)a.q_nope + gr * kDl + ch * 4
                                  : (const float*)a.q_pe + gr * kDr + (ch - 128) * 4;
      *(u32x4_t*)(qs + qr * L::kRowBytes + ch * 16) = *(const u32x4_t*)src;
    }
  }

  // Softmax state of this lane's row. m_ref is the reference max (log2 units,
  // scale applied): the max of the first tile in which the row sees a key. It
  // never moves during a pass, so O is never rescaled; weights are
  // 2^(s - m_ref). If a later score exceeds m_ref by more than kOverflowSlack,
  // the whole workgroup repeats the split once with m_ref = the exact max of
  // the split (m_max), which cannot overflow.
  f32x16_t oacc[16];
  float m_ref = -INFINITY;
  float m_max = -INFINITY;
  float l_run = 0.f;        // this lane's partial denominator (its 16 keys of each step)

  // Per-lane pieces of the LDS addresses (see the layout notes at the top).
  const char* k_rd = smem + qcol * L::kRowBytes + half * (kF32 ? 4 : 16);
  const int g16 = lane >> 4, i16 = lane & 15;
  const char* v_rd = smem + (4 * half + (i16 >> 2)) * L::kRowBytes + (16 * (g16 & 1) + 4 * (i16 & 3)) * 2;

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
  for (int fb = 0; fb < 16; ++fb)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[fb][i] = 0.f;
  l_run = 0.f;
  bool overflow = false;
  for (int tile = tile_begin; tile < tile_end; ++tile) {
    const int k0 = tile * kKeysPerTile;
    __syncthreads();
    stage_tile<kF32>(a, smem, kv0, k0, N);
    __syncthreads();

    // ---- S^T = K . Q^T ------------------------------------------------------
    // Issued in batches of four MFMAs with the next batch's LDS reads in
    // flight; the scheduling barriers keep the compiler from hoisting every
    // read at once (which would not fit next to Q and O in registers).
    f32x16_t sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
    if constexpr (!kF32) {
      bf16x8_t kf[2][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) kf[0][j] = *(const bf16x8_t*)(k_rd + j * 32);
#pragma unroll
      for (int kb = 0; kb < 9; ++kb) {
        if (kb + 1 < 9) {
#pragma unroll
          for (int j = 0; j < 4; ++j) kf[(kb + 1) & 1][j] = *(const bf16x8_t*)(k_rd + (4 * (kb + 1) + j) * 32);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb & 1][j], qreg[4 * kb + j], sacc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      const float* kp = (const float*)k_rd;
      const float* qp = (const float*)(smem + L::kTileBytes + qcol * L::kRowBytes) + half;
#pragma unroll 8
      for (int kc = 0; kc < kDk / 2; ++kc)
        sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kp[2 * kc], qp[2 * kc], sacc, 0, 0, 0);
    }

    // ---- scale, tree mask, softmax weights -----------------------------------
    // Register i of this lane holds key (i/4)*8 + 4*half + i%4 of the tile.
    float sv[16];
    const bool no_mask = k0 + kKeysPerTile <= P;
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = k0 + (i >> 2) * 8 + half * 4 + (i & 3);
      // Branch-free: prefix keys are visible, tail key P+u iff bit u of anc.
      const bool tail_bit = ((anc >> ((j - P) & 63)) & 1ull) != 0;
      const bool vis = no_mask | (j < P) | ((j < N) & tail_bit);
      sv[i] = vis ? sacc[i] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sv[i]);
    }
    mx = fmaxf(mx, swap_halves(mx));
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

    // ---- O^T += V^T . P^T -----------------------------------------------------
    if constexpr (!kF32) {
      bf16x8_t pk[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) pk[u][jj] = (__bf16)sv[8 * u + jj];
      // 8 batches: (u, four output blocks); V^T operands via transpose reads.
      i16x4_t vf[2][4][2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vf[0][j][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(v_rd + j * 64));
        vf[0][j][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(v_rd + 8 * L::kRowBytes + j * 64));
      }
#pragma unroll
      for (int bt = 0; bt < 8; ++bt) {
        const int u = bt >> 2, fb0 = (bt & 3) * 4;
        if (bt + 1 < 8) {
          const int un = (bt + 1) >> 2, fbn = ((bt + 1) & 3) * 4;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            vf[(bt + 1) & 1][j][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4_t*)(v_rd + (16 * un) * L::kRowBytes + (fbn + j) * 64));
            vf[(bt + 1) & 1][j][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4_t*)(v_rd + (16 * un + 8) * L::kRowBytes + (fbn + j) * 64));
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const i16x8_t v01 = __builtin_shufflevector(vf[bt & 1][j][0], vf[bt & 1][j][1], 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[fb0 + j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, v01), pk[u],
                                                                  oacc[fb0 + j], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int fb = 0; fb < 16; ++fb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = (i >> 2) * 8 + 4 * half + (i & 3);
          const float v = ((const float*)(smem + key * L::kRowBytes))[32 * fb + qcol];
          oacc[fb] = __builtin_amdgcn_mfma_f32_32x32x2f32(v, sv[i], oacc[fb], 0, 0, 0);
        }
      }
    }
  }

  if (!__syncthreads_or(overflow)) break;
  m_ref = m_max;
  }

  // ---- epilogue ---------------------------------------------------------------
  // Accumulator register i of block fb holds feature 32*fb + (i/4)*8 + 4*half + i%4.
  const float l_tot = l_run + swap_halves(l_run);
  if (!row_ok) return;
  if (S == 1) {
    const float inv = node_ok ? 1.f / l_tot : NAN;
    float* orow = a.out + grow * kDl + 4 * half;
#pragma unroll
    for (int fb = 0; fb < 16; ++fb)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        f32x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = oacc[fb][4 * gi + e] * inv;
        *(f32x4_t*)(orow + 32 * fb + 8 * gi) = v;
      }
    if (half == 0 && a.lse) a.lse[grow] = node_ok ? (m_ref + __log2f(l_tot)) * kLn2 : NAN;
  } else {
    const int64_t prow = (int64_t)c * a.rows_per_seq + r_eff;
    float* po = a.part_o + prow * kDl + 4 * half;
#pragma unroll
    for (int fb = 0; fb < 16; ++fb)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        f32x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = oacc[fb][4 * gi + e];
        *(f32x4_t*)(po + 32 * fb + 8 * gi) = v;
      }
    if (half == 0) {
      a.part_ml[2 * prow] = node_ok ? m_ref : NAN;
      a.part_ml[2 * prow + 1] = node_ok ? l_tot : NAN;
    }
  }
}

// Merge the split partials of one query row (a workgroup of 128 lanes, 4
// features per lane): M = max m_c, w_c = 2^(m_c - M), L = sum w_c l_c,
// out = sum w_c O_c / L, lse = (M + log2 L) ln 2. Empty splits (m = -inf) add
// nothing; a NaN partial (invalid tree) makes the row NaN.
constexpr int kCombineThreads = 128;
constexpr int kCombineStage = 256;

__global__ void __launch_bounds__(kCombineThreads) mla_verify_combine_kernel(const VerifyArgs a) {
  __shared__ float wsh[kCombineStage];
  __shared__ float red[kCombineThreads / 64];
  const int64_t grow = blockIdx.x;
  const int b = (int)(grow / a.rows_per_seq);
  const int r = (int)(grow % a.rows_per_seq);
  const int s0 = a.split_offset[b];
  const int S = a.split_offset[b + 1] - s0;
  if (S <= 1) return;
  const int tid = threadIdx.x;
  const int lane = lane_id(), wave = tid >> 6;
  const float* ml = a.part_ml + 2 * ((int64_t)s0 * a.rows_per_seq + r);
  const int64_t ml_stride = 2 * (int64_t)a.rows_per_seq;

  float mloc = -INFINITY;
  int nan = 0;
  for (int cc = tid; cc < S; cc += kCombineThreads) {
    const float m = ml[cc * ml_stride];
    nan |= m != m;
    mloc = fmaxf(mloc, m);
  }
  for (int off = 32; off > 0; off >>= 1) {
    mloc = fmaxf(mloc, shfl_f32(mloc, lane ^ off));
    nan |= shfl_i32(nan, lane ^ off);
  }
  __shared__ int nan_sh[kCombineThreads / 64];
  if (lane == 0) {
    red[wave] = mloc;
    nan_sh[wave] = nan;
  }
  __syncthreads();
  float M = red[0];
  nan = nan_sh[0];
  for (int w = 1; w < kCombineThreads / 64; ++w) {
    M = fmaxf(M, red[w]);
    nan |= nan_sh[w];
  }
  __syncthreads();

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float lloc = 0.f;
  const float* po = a.part_o + ((int64_t)s0 * a.rows_per_seq + r) * kDl + 4 * tid;
  const int64_t po_stride = (int64_t)a.rows_per_seq * kDl;
  for (int base = 0; base < S; base += kCombineStage) {
    const int cnt = min(kCombineStage, S - base);
    __syncthreads();
    for (int cc = tid; cc < cnt; cc += kCombineThreads) {
      const float m = ml[(base + cc) * ml_stride];
      const float l = ml[(base + cc) * ml_stride + 1];
      const float w = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
      wsh[cc] = w;
      lloc += w * l;
    }
    __syncthreads();
#pragma unroll 8
    for (int cc = 0; cc < cnt; ++cc) {
      const float w = wsh[cc];
      if (w != 0.f) {
        const f32x4_t v = *(const f32x4_t*)(po + (base + cc) * po_stride);
        acc += w * v;
      }
    }
  }
  for (int off = 32; off > 0; off >>= 1) lloc += shfl_f32(lloc, lane ^ off);
  if (lane == 0) red[wave] = lloc;
  __syncthreads();
  float Lsum = 0.f;
  for (int w = 0; w < kCombineThreads / 64; ++w) Lsum += red[w];
  const float inv = nan ? NAN : 1.f / Lsum;
  *(f32x4_t*)(a.out + grow * kDl + 4 * tid) = acc * inv;
  if (tid == 0 && a.lse) a.lse[grow] = nan ? NAN : (M + __log2f(Lsum)) * kLn2;
}

int launch_verify_attention(const VerifyArgs& a, int dtype, int64_t grid_blocks, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (dtype == MLA_DTYPE_BF16)
    hipLaunchKernelGGL(mla_verify_attn_kernel<false>, dim3((unsigned)grid_blocks),
                       dim3(KLayout<false>::kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(mla_verify_attn_kernel<true>, dim3((unsigned)grid_blocks),
                       dim3(KLayout<true>::kThreads), 0, st, a);
  return (int)hipGetLastError();
}

int launch_verify_combine(const VerifyArgs& a, void* stream) {
  const int64_t rows = (int64_t)a.batch * a.rows_per_seq;
  hipLaunchKernelGGL(mla_verify_combine_kernel, dim3((unsigned)rows), dim3(kCombineThreads), 0,
                     (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_tree_masks(const int32_t* parents, int32_t batch, int32_t tree_nodes, uint64_t* masks,
                      void* stream) {
  hipLaunchKernelGGL(mla_tree_masks_kernel, dim3(batch), dim3(64), 0, (hipStream_t)stream, parents,
                     tree_nodes, masks);
  return (int)hipGetLastError();
}

}  // namespace mlav
