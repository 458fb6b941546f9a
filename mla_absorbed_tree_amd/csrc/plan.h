// Host-side launch plan of the tree-verify attention (no HIP calls here).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/mla_verify.h"

namespace mlav {

// Geometry shared by the planner and the kernels.
constexpr int kDl = 512;
constexpr int kDr = 64;
constexpr int kDk = kDl + kDr;
constexpr int kXcds = 8;                 // MI355X: workgroups are dealt round-robin to 8 XCDs
constexpr int kKeysPerTile = 32;         // keys staged in LDS per step
constexpr int kRowsPerBlockBf16 = 128;   // 4 waves x 32 query rows
constexpr int kRowsPerBlockF32 = 32;     // 1 wave x 32 query rows
constexpr int kComputeUnits = 256;

struct Plan {
  int32_t batch = 0, heads = 0, tree_nodes = 0, dtype = 0;
  int64_t kv_c_stride = 0, k_pe_stride = 0;
  int32_t max_rows_per_seq = 0; // largest T_b * H
  int32_t rows_per_block = 0;
  int32_t row_blocks = 0;       // ceil(max_rows_per_seq / rows_per_block)
  std::vector<int32_t> tree_len;     // T_b
  std::vector<int32_t> node_offset;  // [batch + 1] prefix sums of T_b (packed trees)
  std::vector<int32_t> kv_len;  // N_b from the host copy
  std::vector<int32_t> splits;  // S_b
  std::vector<int32_t> split_offset;  // [batch + 1] prefix sums of S_b
  int32_t total_splits = 0, max_splits = 0;
  // A workgroup runs `group` consecutive splits of one sequence for one row
  // block: one stream of key tiles against one reference max, merged in its
  // accumulators, one partial per group.
  int32_t group = 1;
  std::vector<int32_t> group_offset;  // [batch + 1] prefix sums of ceil(S_b / group)
  int32_t total_groups = 0;
  int32_t max_groups = 0;       // largest group count of one sequence
  int64_t partial_rows = 0;     // sum over sequences with > 1 group of groups * T_b * H
  int32_t chunk_groups = 0;     // ceil(total_groups / kXcds)
  int64_t grid_blocks = 0;      // attention launch
  bool combine = false;         // some sequence has more than one split group
  // Workspace layout (byte offsets from the workspace start).
  size_t ws_status = 0;         // int32 [batch] status words (MLA_VERIFY_STATUS_*)
  // Per (split group, row), rows padded to row_blocks * rows_per_block per group:
  size_t ws_part_ml = 0;        // float4 (m in log2 units, l, s_0, s_1)
  size_t ws_part_o = 0;         // [512] unnormalised O: fp32, or scaled fp16 for bf16 problems
  size_t ws_bytes = 0;
};

// Validates `p` and fills `plan`. On error returns a status and sets `err`.
mla_status build_plan(const mla_verify_problem& p, Plan& plan, std::string& err);

}  // namespace mlav
