// Argument block of the tree-verify kernels (passed by value as kernel arguments).
#pragma once

#include <cstdint>

#include "../../include/mla_verify.h"

namespace mlav {

// Trees are packed: sequence b owns tree nodes node_offset[b] ..
// node_offset[b+1]-1 (b*T when every tree has T nodes), and query row
// (node_offset[b] + t) * H + h.
struct VerifyArgs {
  const void* q_nope;          // [nodes, H, 512]
  const void* q_pe;            // [nodes, H, 64]
  const void* kv_c;            // slot s at kv_c + s * kv_c_stride
  const void* k_pe;            // slot s at k_pe + s * k_pe_stride
  const int32_t* kv_indptr;    // [B + 1]
  const int32_t* kv_indices;   // page table, page_size = 1
  const int32_t* parents;      // [nodes], node indices local to the sequence
  // Device tree offsets [B + 1] read at run time, or nullptr (node_offset
  // below). Sequence b's device size must lie in 0..its planned size
  // node_offset[b+1] - node_offset[b]; a sequence outside that is skipped.
  const int32_t* tree_indptr;
  float* out;                  // [nodes, H, 512]
  float* lse;                  // [nodes, H] or nullptr
  // Partials, one per split group [total_groups, part_rows, 512] (when some
  // sequence has several groups; group_offset[b] is sequence b's first):
  // unnormalised O = sum of 2^(s - m) v, fp32 for fp32 problems; for bf16
  // problems fp16, feature half f scaled by 1 / s_f of the row's record.
  // Rows past a sequence's T_b * H are padding (never read).
  void* part_o;
  float* part_ml;              // [total_groups, part_rows, 4]  (m in log2 units, l, s_0, s_1)
  int32_t* status;             // [batch] per-sequence status words (MLA_VERIFY_STATUS_*)
  int64_t kv_c_stride;         // elements
  int64_t k_pe_stride;         // elements
  float scale_log2;            // softmax scale * log2(e)
  int32_t batch;
  int32_t heads;
  int32_t max_rows_per_seq;    // largest T_b * H
  int32_t part_rows;           // row_blocks * rows per workgroup (>= max_rows_per_seq)
  int32_t row_blocks;          // workgroups along the rows of the largest tree
  int32_t total_splits;
  int32_t group;                                   // consecutive splits per workgroup
  int32_t max_groups;                              // largest split-group count of one sequence
  // The per-sequence tables. Batches of up to MLA_VERIFY_ARG_TABLE_BATCH
  // carry them here, in the kernel-argument block (three tables of
  // MLA_VERIFY_ARG_TABLE_BATCH + 1 words, about 3 KB of the 4 KB a launch's
  // arguments may take); larger batches read them from device memory that
  // mla_verify_plan_stage_tables filled: dev_tables = [split_offset |
  // group_offset | node_offset], batch + 1 words each (nullptr otherwise).
  const int32_t* dev_tables;
  int32_t split_offset[MLA_VERIFY_ARG_TABLE_BATCH + 1];  // first global split of sequence b
  int32_t group_offset[MLA_VERIFY_ARG_TABLE_BATCH + 1];  // first split group (and partial) of sequence b
  int32_t node_offset[MLA_VERIFY_ARG_TABLE_BATCH + 1];   // first tree node of sequence b
};

// Launchers (defined in the HIP translation unit). Return the launch error.
int launch_verify_attention(const VerifyArgs& a, int dtype, int64_t grid_blocks, void* stream);
int launch_verify_combine(const VerifyArgs& a, int dtype, void* stream);
// Host -> device copy of a plan's per-sequence tables (enqueued on stream).
int copy_tables_to_device(void* dst, const void* src, size_t bytes, void* stream);
// Built-in workspace of mla_verify_run_noalloc (defined with the kernels):
// its size, and its device address on the current device (0 on success, else
// the hipError_t of locating it).
size_t noalloc_scratch_bytes();
int noalloc_scratch(void** ptr);
int launch_tree_masks(const int32_t* parents, int32_t batch, int32_t tree_nodes, uint64_t* masks,
                      void* stream);  // masks [batch, tree_nodes, ceil(tree_nodes / 64)]
// indptr NULL: trees of T nodes each; else packed trees of at most T nodes.
int launch_tree_accept(const int32_t* parents, const int32_t* draft, const int32_t* target,
                       const int32_t* root_target, const int32_t* indptr, int32_t batch, int32_t T,
                       int32_t* accept_len, int32_t* accept_path, int32_t* bonus, void* stream);

}  // namespace mlav
