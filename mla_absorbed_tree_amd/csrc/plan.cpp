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
  int64_t work = 0, busy_row_blocks = 0;
  for (int b = 0; b < p.batch; ++b) {
    const int32_t n = p.kv_len_host[b];
    if (n < tree_len[b]) {
      err = fmt("kv_len_host[%lld] = %lld is smaller than the sequence's tree", b, n);
      return MLA_ERR_INVALID_ARG;
    }
    plan.kv_len[b] = n;
    row_blocks[b] = (int64_t(tree_len[b]) * p.num_heads + plan.rows_per_block - 1) / plan.rows_per_block;
    tiles[b] = row_blocks[b] > 0 ? (int64_t(n) + kKeysPerTile - 1) / kKeysPerTile : 0;
    work += row_blocks[b] * tiles[b];
    busy_row_blocks += tiles[b] > 0 ? row_blocks[b] : 0;
  }

  // Split schedule. Forced: S_b = min(num_splits, tiles_b). Automatic: pick a
  // chunk length (in tiles) so that the launch holds about one workgroup per
  // compute unit, but never chunks shorter than kMinChunkTiles (a split's
  // partial write costs about as much as a few tiles of compute).
  constexpr int64_t kMinChunkTiles = 8;
  plan.splits.resize(p.batch);
  if (p.num_splits > 0) {
    for (int b = 0; b < p.batch; ++b)
      plan.splits[b] = int32_t(std::min<int64_t>(p.num_splits, tiles[b]));
  } else {
    if (busy_row_blocks >= kComputeUnits) {
      for (int b = 0; b < p.batch; ++b) plan.splits[b] = tiles[b] > 0 ? 1 : 0;
    } else {
      const int64_t chunk = std::max<int64_t>(kMinChunkTiles, (work + kComputeUnits - 1) / kComputeUnits);
      for (int b = 0; b < p.batch; ++b)
        plan.splits[b] = tiles[b] > 0 ? int32_t(std::max<int64_t>(1, (tiles[b] + chunk - 1) / chunk)) : 0;
    }
    // Every KV chunk runs on one XCD (its row blocks share that XCD's L2):
    // with fewer chunks than XCDs some XCDs would idle, so split the longest
    // sequences further (while chunks stay at least kMinChunkTiles long).
    for (;;) {
      int64_t total = 0;
      for (int b = 0; b < p.batch; ++b) total += plan.splits[b];
      if (total >= kXcds) break;
      int best = -1;
      for (int b = 0; b < p.batch; ++b) {
        if (tiles[b] == 0 || tiles[b] / (plan.splits[b] + 1) < kMinChunkTiles) continue;
        if (best < 0 || tiles[b] * plan.splits[best] > tiles[best] * plan.splits[b]) best = b;
      }
      if (best < 0) break;
      ++plan.splits[best];
    }
  }
  plan.split_offset.assign(p.batch + 1, 0);
  for (int b = 0; b < p.batch; ++b) {
    plan.split_offset[b + 1] = plan.split_offset[b] + plan.splits[b];
    plan.max_splits = std::max(plan.max_splits, plan.splits[b]);
    if (plan.splits[b] > 1) plan.combine = true;
  }
  plan.total_splits = plan.split_offset[p.batch];
  // Many short splits (a forced split count) would make thousands of
  // workgroups that each pay the fixed start-up and tail; instead one
  // workgroup runs several consecutive splits, aiming at about one workgroup
  // per compute unit. The bf16 kernel only (the fp32 kernel runs one split).
  plan.group = 1;
  if (p.dtype == MLA_DTYPE_BF16) {
    int64_t split_row_blocks = 0;
    for (int b = 0; b < p.batch; ++b) split_row_blocks += int64_t(plan.splits[b]) * row_blocks[b];
    plan.group = int32_t(std::max<int64_t>(1, split_row_blocks / kComputeUnits));
  }
  plan.group = std::min(plan.group, std::max(1, plan.max_splits));
  plan.group_offset.assign(p.batch + 1, 0);
  for (int b = 0; b < p.batch; ++b)
    plan.group_offset[b + 1] = plan.group_offset[b] + (plan.splits[b] + plan.group - 1) / plan.group;
  plan.total_groups = plan.group_offset[p.batch];
  plan.chunk_groups = (plan.total_groups + kXcds - 1) / kXcds;
  plan.grid_blocks = int64_t(plan.chunk_groups) * kXcds * plan.row_blocks;
  if (plan.grid_blocks > (int64_t(1) << 31) - 1) {
    err = "launch grid too large";
    return MLA_ERR_UNSUPPORTED;
  }

  size_t off = 256;  // status flags live in the first 256 bytes
  plan.ws_status = 0;
  if (plan.combine) {
    // Partial rows per split padded to whole row blocks (the bf16 kernel
    // stores unconditionally, padding rows included).
    const size_t part_rows = size_t(plan.total_splits) * size_t(plan.row_blocks) * size_t(plan.rows_per_block);
    plan.ws_part_ml = off;
    off = align_up(off + part_rows * 2 * sizeof(float), 256);
    plan.ws_part_o = off;
    const size_t part_elem = p.dtype == MLA_DTYPE_BF16 ? 2 : sizeof(float);
    off = align_up(off + part_rows * kDl * part_elem, 256);
  }
  plan.ws_bytes = off;
  return MLA_OK;
}

}  // namespace mlav
