// Host-side validation, KV-split schedule and workspace layout.
#include "plan.h"

#include <algorithm>
#include <cstdio>

namespace mlav {

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

std::string fmt(const char* f, long long a = 0, long long b = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, f, a, b);
  return buf;
}

// Launch-time model of the attention kernel, in units of one workgroup's key
// tile. Split groups are dealt round-robin to the XCDs, all row blocks of a
// group on one XCD and in order (as map_block does); each XCD runs one
// workgroup per compute unit at a time and hands the next one, in dispatch
// order, to the first unit that frees up. A workgroup costs its group's tiles
// plus a fixed start-up (Q and tree loads, pipeline fill, epilogue). Split
// partials add their write and the combine's read at HBM speed.
constexpr double kWgOverheadTiles = 4.0;
constexpr double kTileSeconds = 1.75e-6;      // one tile of one 128-row workgroup (measured)
constexpr double kHbmBytesPerSecond = 5.0e12; // sustained partial write/read rate

// S_b splits of sequence b cover its tiles in near-equal ranges (split s:
// tiles s*T/S .. (s+1)*T/S - 1), and each split group runs `group`
// consecutive splits in one workgroup per row block.
double estimate_launch(const std::vector<int64_t>& tiles, const std::vector<int64_t>& row_blocks,
                       const std::vector<int32_t>& splits, int rows_per_block, int dtype, int64_t group = 1) {
  const int cus_per_xcd = kComputeUnits / kXcds;
  std::vector<std::vector<double>> free_at(kXcds, std::vector<double>(cus_per_xcd, 0.0));
  int64_t cg = 0;
  double partial_bytes = 0.0;
  // (m, l, s0, s1) record and O: scaled fp16 for bf16 problems, fp32 for fp32
  const double part_row_bytes = dtype == MLA_DTYPE_BF16 ? kDl * 2 + 16 : kDl * 4 + 16;
  for (size_t b = 0; b < tiles.size(); ++b) {
    const int64_t S = splits[b];
    const int64_t G = (S + group - 1) / group;
    if (G > 1) partial_bytes += double(G) * double(row_blocks[b]) * rows_per_block * part_row_bytes;
    for (int64_t c = 0; c < G; ++c, ++cg) {
      const int64_t s0 = c * group, s1 = std::min(S, s0 + group);
      const int64_t nt = s1 * tiles[b] / S - s0 * tiles[b] / S;
      std::vector<double>& cu = free_at[cg % kXcds];
      for (int64_t rb = 0; rb < row_blocks[b]; ++rb) {
        auto it = std::min_element(cu.begin(), cu.end());
        *it += double(nt) + kWgOverheadTiles;
      }
    }
  }
  double makespan = 0.0;
  for (const auto& cu : free_at) makespan = std::max(makespan, *std::max_element(cu.begin(), cu.end()));
  return makespan * kTileSeconds + 2.0 * partial_bytes / kHbmBytesPerSecond;
}

// Group size for forced split counts: the number of consecutive splits one
// workgroup runs, chosen by the same estimate. For each group count G of the
// longest sequence (S splits), from one group upwards, the candidate is the
// smallest size that gives G groups, ceil(S / G), so that the groups come out
// as even as they can; a candidate with more groups must beat the best so far
// by 1% (ties keep fewer groups and fewer partials). Candidates whose
// workgroups exceed kMaxSearchWorkgroups beyond the first are not tried, as
// for automatic splits.
int64_t choose_group(const std::vector<int64_t>& tiles, const std::vector<int64_t>& row_blocks,
                     const std::vector<int32_t>& splits, int rows_per_block, int dtype) {
  constexpr int64_t kMaxSearchWorkgroups = 16 * kComputeUnits;
  const int64_t max_s = splits.empty() ? 1 : std::max<int64_t>(1, *std::max_element(splits.begin(), splits.end()));
  int64_t best_g = max_s, first_n = -1, last_g = -1;
  double best_t = -1.0;
  for (int64_t G = 1; G <= max_s; ++G) {
    const int64_t g = (max_s + G - 1) / G;
    if (g == last_g) continue;  // the same partition of the longest sequence
    last_g = g;
    int64_t n = 0;
    for (size_t b = 0; b < splits.size(); ++b) n += (splits[b] + g - 1) / g * row_blocks[b];
    if (first_n < 0) first_n = n;
    else if (n > first_n + kMaxSearchWorkgroups) break;
    const double t = estimate_launch(tiles, row_blocks, splits, rows_per_block, dtype, g);
    if (best_t < 0.0 || t < 0.99 * best_t) {
      best_t = t;
      best_g = g;
    }
  }
  return best_g;
}

// Automatic split counts: candidate chunk lengths ceil(max_tiles / k),
// k = 1, 2, ..., no shorter than kMinChunkTiles (a split's partial costs
// about a few tiles); S_b = ceil(tiles_b / chunk), each candidate also tried
// with its total raised to a multiple of the XCD count. The estimate decides;
// a candidate must beat the best so far by 1% (ties keep fewer splits).
// Shorter chunks only add workgroups, so the search stops at the first
// candidate with more than kMaxSearchWorkgroups of them (beyond one split per
// sequence): by then the chip runs many even rounds and finer chunks buy
// little, while each estimate costs time in proportion to the workgroups.
std::vector<int32_t> choose_auto_splits(const std::vector<int64_t>& tiles,
                                        const std::vector<int64_t>& row_blocks, int rows_per_block, int dtype) {
  constexpr int64_t kMinChunkTiles = 8;
  constexpr int64_t kMaxCandidates = 512;
  constexpr int64_t kMaxSearchWorkgroups = 16 * kComputeUnits;
  int64_t first_n = -1;
  const int64_t max_tiles = tiles.empty() ? 0 : *std::max_element(tiles.begin(), tiles.end());
  std::vector<int32_t> best(tiles.size(), 0), cand(tiles.size(), 0);
  double best_t = -1.0;
  int64_t last_chunk = -1;
  for (int64_t k = 1; k <= kMaxCandidates; ++k) {
    const int64_t chunk = std::max<int64_t>(kMinChunkTiles, (max_tiles + k - 1) / k);
    if (chunk == last_chunk) {
      if (chunk == kMinChunkTiles) break;
      continue;
    }
    last_chunk = chunk;
    int64_t n = 0;
    for (size_t b = 0; b < tiles.size(); ++b) {
      cand[b] = tiles[b] > 0 ? int32_t(std::max<int64_t>(1, (tiles[b] + chunk - 1) / chunk)) : 0;
      n += int64_t(cand[b]) * row_blocks[b];
    }
    if (first_n < 0) first_n = n;
    else if (n > first_n + kMaxSearchWorkgroups) break;
    const double t = estimate_launch(tiles, row_blocks, cand, rows_per_block, dtype);
    if (best_t < 0.0 || t < 0.99 * best_t) {
      best_t = t;
      best = cand;
    }
    // The same candidate with its split count raised to a multiple of the
    // XCD count (one more split at a time for the sequence whose splits are
    // longest), so that every XCD gets as many split groups.
    std::vector<int32_t> even = cand;
    int64_t total = 0;
    for (int32_t x : even) total += x;
    bool grown = false;
    while (total % kXcds != 0) {
      size_t arg = tiles.size();
      int64_t longest = 0;
      for (size_t b = 0; b < tiles.size(); ++b) {
        // no chunk below kMinChunkTiles
        if (even[b] == 0 || (tiles[b] + even[b]) / (even[b] + 1) < kMinChunkTiles) continue;
        const int64_t len = (tiles[b] + even[b] - 1) / even[b];
        if (len > longest) longest = len, arg = b;
      }
      if (arg == tiles.size()) break;  // no sequence can take another split
      ++even[arg];
      ++total;
      grown = true;
    }
    if (grown) {
      const double te = estimate_launch(tiles, row_blocks, even, rows_per_block, dtype);
      if (te < 0.99 * best_t) {
        best_t = te;
        best = even;
      }
    }
  }
  return best;
}

}  // namespace

mla_status build_plan(const mla_verify_problem& p, Plan& plan, std::string& err) {
  if (p.batch < 1 || p.batch > MLA_VERIFY_MAX_BATCH) {
    err = fmt("batch %lld outside 1..%lld", p.batch, MLA_VERIFY_MAX_BATCH);
    return MLA_ERR_INVALID_ARG;
  }
  if (p.num_heads < 1) {
    err = fmt("num_heads %lld < 1", p.num_heads);
    return MLA_ERR_INVALID_ARG;
  }
  if (p.tree_nodes < 1 || p.tree_nodes > MLA_VERIFY_MAX_TREE) {
    err = fmt("tree_nodes %lld outside 1..%lld", p.tree_nodes, MLA_VERIFY_MAX_TREE);
    return p.tree_nodes > MLA_VERIFY_MAX_TREE ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  }
  if (p.tree_len_host) {
    for (int b = 0; b < p.batch; ++b)
      if (p.tree_len_host[b] < 0 || p.tree_len_host[b] > p.tree_nodes) {
        err = fmt("tree_len_host[%lld] = %lld is outside 0..tree_nodes", b, p.tree_len_host[b]);
        return MLA_ERR_INVALID_ARG;
      }
  }
  if (p.d_latent != kDl || p.d_rope != kDr) {
    err = fmt("d_latent/d_rope %lld/%lld: only 512/64 is supported", p.d_latent, p.d_rope);
    return MLA_ERR_UNSUPPORTED;
  }
  if (p.dtype != MLA_DTYPE_F32 && p.dtype != MLA_DTYPE_BF16) {
    err = fmt("unknown dtype %lld", p.dtype);
    return MLA_ERR_INVALID_ARG;
  }
  if (p.kv_c_row_stride < kDl || p.kv_c_row_stride % 8 != 0) {
    err = fmt("kv_c_row_stride %lld must be >= 512 and a multiple of 8", p.kv_c_row_stride);
    return MLA_ERR_INVALID_ARG;
  }
  if (p.k_pe_row_stride < kDr || p.k_pe_row_stride % 8 != 0) {
    err = fmt("k_pe_row_stride %lld must be >= 64 and a multiple of 8", p.k_pe_row_stride);
    return MLA_ERR_INVALID_ARG;
  }
  if (p.num_splits < 0) {
    err = fmt("num_splits %lld < 0", p.num_splits);
    return MLA_ERR_INVALID_ARG;
  }
  if (!p.kv_len_host) {
    err = "kv_len_host is NULL";
    return MLA_ERR_INVALID_ARG;
  }
  const int64_t rows_per_seq = int64_t(p.tree_nodes) * p.num_heads;
  if (rows_per_seq > (int64_t(1) << 24)) {
    err = fmt("tree_nodes * num_heads = %lld is too large", rows_per_seq);
    return MLA_ERR_INVALID_ARG;
  }
  std::vector<int32_t> tree_len(p.batch);
  for (int b = 0; b < p.batch; ++b) tree_len[b] = p.tree_len_host ? p.tree_len_host[b] : p.tree_nodes;
  int32_t max_tree = 0;
  for (int b = 0; b < p.batch; ++b) max_tree = std::max(max_tree, tree_len[b]);

  plan = Plan();
  plan.batch = p.batch;
  plan.heads = p.num_heads;
  plan.tree_nodes = p.tree_nodes;
  plan.dtype = p.dtype;
  plan.kv_c_stride = p.kv_c_row_stride;
  plan.k_pe_stride = p.k_pe_row_stride;
  plan.max_rows_per_seq = max_tree * p.num_heads;
  plan.rows_per_block = p.dtype == MLA_DTYPE_BF16 ? kRowsPerBlockBf16 : kRowsPerBlockF32;
  plan.row_blocks = (plan.max_rows_per_seq + plan.rows_per_block - 1) / plan.rows_per_block;
  plan.tree_len = tree_len;
  plan.node_offset.assign(p.batch + 1, 0);
  for (int b = 0; b < p.batch; ++b) plan.node_offset[b + 1] = plan.node_offset[b] + tree_len[b];
  if (int64_t(plan.node_offset[p.batch]) * p.num_heads > (int64_t(1) << 30)) {
    err = "total tree nodes * num_heads is too large";
    return MLA_ERR_INVALID_ARG;
  }

  // Work of a sequence: its key tiles times its row blocks (a sequence
  // without tree nodes has none and gets no split).
  plan.kv_len.resize(p.batch);
  std::vector<int64_t> tiles(p.batch), row_blocks(p.batch);
  for (int b = 0; b < p.batch; ++b) {
    const int32_t n = p.kv_len_host[b];
    if (n < tree_len[b]) {
      err = fmt("kv_len_host[%lld] = %lld is smaller than the sequence's tree", b, n);
      return MLA_ERR_INVALID_ARG;
    }
    plan.kv_len[b] = n;
    row_blocks[b] = (int64_t(tree_len[b]) * p.num_heads + plan.rows_per_block - 1) / plan.rows_per_block;
    tiles[b] = row_blocks[b] > 0 ? (int64_t(n) + kKeysPerTile - 1) / kKeysPerTile : 0;
  }

  // Split schedule. Forced: S_b = min(num_splits, tiles_b). Automatic: the
  // chunk length (in tiles, at least kMinChunkTiles) whose estimated launch
  // time is smallest (choose_auto_splits).
  plan.splits.resize(p.batch);
  if (p.num_splits > 0) {
    for (int b = 0; b < p.batch; ++b)
      plan.splits[b] = int32_t(std::min<int64_t>(p.num_splits, tiles[b]));
  } else {
    plan.splits = choose_auto_splits(tiles, row_blocks, plan.rows_per_block, p.dtype);
  }
  plan.split_offset.assign(p.batch + 1, 0);
  for (int b = 0; b < p.batch; ++b) {
    plan.split_offset[b + 1] = plan.split_offset[b] + plan.splits[b];
    plan.max_splits = std::max(plan.max_splits, plan.splits[b]);
  }
  plan.total_splits = plan.split_offset[p.batch];
  // Many short splits (a forced split count) would make thousands of
  // workgroups that each pay the fixed start-up and tail; instead one
  // workgroup runs several consecutive splits (a split group), as many as the
  // launch-time estimate favours. Its splits share one reference max, so
  // their partials merge by a plain sum, done in the kernel's accumulators:
  // the group writes one partial, and the combine merges the groups. The bf16
  // kernel only (the fp32 kernel runs one split per workgroup); automatic
  // splits are already sized for the chip (one split each).
  plan.group = 1;
  if (p.dtype == MLA_DTYPE_BF16 && p.num_splits > 0)
    plan.group = int32_t(choose_group(tiles, row_blocks, plan.splits, plan.rows_per_block, p.dtype));
  plan.group = std::min(plan.group, std::max(1, plan.max_splits));
  plan.group_offset.assign(p.batch + 1, 0);
  for (int b = 0; b < p.batch; ++b)
    plan.group_offset[b + 1] = plan.group_offset[b] + (plan.splits[b] + plan.group - 1) / plan.group;
  plan.total_groups = plan.group_offset[p.batch];
  for (int b = 0; b < p.batch; ++b) {
    const int32_t g = plan.group_offset[b + 1] - plan.group_offset[b];
    plan.max_groups = std::max(plan.max_groups, g);
    if (g > 1) {
      plan.combine = true;
      plan.partial_rows += int64_t(g) * plan.tree_len[b] * p.num_heads;
    }
  }
  plan.chunk_groups = (plan.total_groups + kXcds - 1) / kXcds;
  plan.grid_blocks = int64_t(plan.chunk_groups) * kXcds * plan.row_blocks;
  if (plan.grid_blocks > (int64_t(1) << 31) - 1) {
    err = "launch grid too large";
    return MLA_ERR_UNSUPPORTED;
  }

  // The per-sequence status words come first, then the split partials.
  plan.ws_status = 0;
  size_t off = align_up(size_t(p.batch) * sizeof(int32_t), 256);
  if (plan.combine) {
    // One partial per split group; rows padded to whole row blocks (the bf16
    // kernel stores unconditionally, padding rows included).
    const size_t part_rows = size_t(plan.total_groups) * size_t(plan.row_blocks) * size_t(plan.rows_per_block);
    plan.ws_part_ml = off;
    off = align_up(off + part_rows * 4 * sizeof(float), 256);
    plan.ws_part_o = off;
    const size_t part_elem = p.dtype == MLA_DTYPE_BF16 ? 2 : sizeof(float);
    off = align_up(off + part_rows * kDl * part_elem, 256);
  }
  plan.ws_bytes = off;
  return MLA_OK;
}

}  // namespace mlav
