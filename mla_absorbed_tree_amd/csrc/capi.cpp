// extern "C" entry points of libmlaverify: argument checks, plan objects and
// the launch sequence. Device work happens only inside the launchers.
#include <climits>
#include <cstdint>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/mla_kv_compact.h"
#include "../../include/mla_tree_accept.h"
#include "../../include/mla_verify.h"
#include "kernel_params.h"
#include "kv_compact_params.h"
#include "plan.h"

struct mla_verify_plan_s {
  mlav::Plan plan;
  // Batches above MLA_VERIFY_ARG_TABLE_BATCH: the per-sequence tables,
  // [split_offset | group_offset | node_offset], as staged on the host and
  // the caller's device copy (set by mla_verify_plan_stage_tables).
  std::vector<int32_t> tables;
  const int32_t* dev_tables = nullptr;
};

namespace {

thread_local std::string g_last_error;

mla_status fail(mla_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

mla_status mla_verify_plan(const mla_verify_problem* problem, mla_verify_plan_t* out,
                           size_t* workspace_bytes) {
  g_last_error.clear();
  if (!problem || !out || !workspace_bytes) return fail(MLA_ERR_INVALID_ARG, "NULL argument to mla_verify_plan");
  *out = nullptr;
  auto* h = new (std::nothrow) mla_verify_plan_s;
  if (!h) return fail(MLA_ERR_INVALID_ARG, "out of host memory");
  std::string err;
  const mla_status st = mlav::build_plan(*problem, h->plan, err);
  if (st != MLA_OK) {
    delete h;
    return fail(st, err);
  }
  if (problem->batch > MLA_VERIFY_ARG_TABLE_BATCH) {
    const mlav::Plan& p = h->plan;
    h->tables.reserve(3 * size_t(p.batch + 1));
    h->tables.insert(h->tables.end(), p.split_offset.begin(), p.split_offset.end());
    h->tables.insert(h->tables.end(), p.group_offset.begin(), p.group_offset.end());
    h->tables.insert(h->tables.end(), p.node_offset.begin(), p.node_offset.end());
  }
  *out = h;
  *workspace_bytes = h->plan.ws_bytes;
  return MLA_OK;
}

mla_status mla_verify_plan_stage_tables(mla_verify_plan_t plan, void* tables, size_t tables_bytes, void* stream) {
  g_last_error.clear();
  if (!plan) return fail(MLA_ERR_INVALID_ARG, "plan is NULL");
  if (plan->tables.empty()) return MLA_OK;  // the tables travel in the launch arguments
  const size_t need = plan->tables.size() * sizeof(int32_t);
  if (!tables || tables_bytes < need)
    return fail(MLA_ERR_INVALID_ARG, "the plan's tables need " + std::to_string(need) + " bytes of device memory");
  if ((reinterpret_cast<uintptr_t>(tables) & 3u) != 0) return fail(MLA_ERR_INVALID_ARG, "tables must be 4-byte aligned");
  const int e = mlav::copy_tables_to_device(tables, plan->tables.data(), need, stream);
  if (e != 0) return fail(MLA_ERR_HIP, "copying the tables failed (hipError " + std::to_string(e) + ")");
  plan->dev_tables = static_cast<const int32_t*>(tables);
  return MLA_OK;
}

mla_status mla_verify_plan_get_info(mla_verify_plan_t plan, mla_verify_plan_info* info) {
  if (!plan || !info) return fail(MLA_ERR_INVALID_ARG, "NULL argument to mla_verify_plan_get_info");
  const mlav::Plan& p = plan->plan;
  info->total_splits = p.total_splits;
  info->max_splits = p.max_splits;
  info->rows_per_block = p.rows_per_block;
  info->keys_per_tile = mlav::kKeysPerTile;
  info->grid_blocks = int32_t(p.grid_blocks);
  info->uses_combine = p.combine ? 1 : 0;
  info->splits_per_workgroup = p.group;
  info->total_groups = p.total_groups;
  info->workspace_bytes = p.ws_bytes;
  info->table_bytes = plan->tables.size() * sizeof(int32_t);
  info->partial_rows = p.partial_rows;
  return MLA_OK;
}

}  // extern "C"

namespace {

// Checks the run arguments and fills the kernel argument block.
mla_status prepare(mla_verify_plan_t plan, const void* q_nope, const void* q_pe, const void* kv_c,
                   const void* k_pe, const int32_t* kv_indptr, const int32_t* kv_indices,
                   const int32_t* tree_parents, float scale, float* out, float* lse,
                   void* workspace, size_t workspace_bytes, bool need_inputs, mlav::VerifyArgs& a,
                   const int32_t* tree_indptr = nullptr) {
  if (!plan) return fail(MLA_ERR_INVALID_ARG, "plan is NULL");
  const mlav::Plan& p = plan->plan;
  // A batch without any tree node has no query rows: its q, parent and output
  // buffers are empty and may be NULL.
  const bool rows = p.node_offset[p.batch] > 0;
  if (need_inputs && (!kv_c || !k_pe || !kv_indptr || !kv_indices || (rows && (!q_nope || !q_pe || !tree_parents))))
    return fail(MLA_ERR_INVALID_ARG, "NULL device pointer");
  if (!out && rows) return fail(MLA_ERR_INVALID_ARG, "out is NULL");
  if (need_inputs && (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(kv_c) || !aligned16(k_pe)))
    return fail(MLA_ERR_INVALID_ARG, "q_nope, q_pe, kv_c and k_pe must be 16-byte aligned");
  if (!aligned16(out)) return fail(MLA_ERR_INVALID_ARG, "out must be 16-byte aligned");
  if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes))
    return fail(MLA_ERR_WORKSPACE, "workspace of " + std::to_string(workspace_bytes) +
                                       " bytes is smaller than the plan's " + std::to_string(p.ws_bytes));
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MLA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  // The kernels work with scale * log2(e), which must be finite too.
  if (need_inputs && !(scale > 0.f && scale < 2.3e38f))
    return fail(MLA_ERR_INVALID_ARG, "scale must be positive and finite (below 2.3e38)");

  std::memset(&a, 0, sizeof a);
  a.q_nope = q_nope;
  a.q_pe = q_pe;
  a.kv_c = kv_c;
  a.k_pe = k_pe;
  a.kv_indptr = kv_indptr;
  a.kv_indices = kv_indices;
  a.parents = tree_parents;
  a.tree_indptr = tree_indptr;
  a.out = out;
  a.lse = lse;
  char* ws = static_cast<char*>(workspace);
  a.part_o = p.combine ? static_cast<void*>(ws + p.ws_part_o) : nullptr;
  a.part_ml = p.combine ? reinterpret_cast<float*>(ws + p.ws_part_ml) : nullptr;
  a.status = reinterpret_cast<int32_t*>(ws + p.ws_status);
  a.kv_c_stride = p.kv_c_stride;
  a.k_pe_stride = p.k_pe_stride;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.batch = p.batch;
  a.heads = p.heads;
  a.max_rows_per_seq = p.max_rows_per_seq;
  a.part_rows = p.row_blocks * p.rows_per_block;
  a.row_blocks = p.row_blocks;
  a.total_splits = p.total_splits;
  a.group = p.group;
  a.max_groups = p.max_groups;
  if (p.batch > MLA_VERIFY_ARG_TABLE_BATCH) {
    if (!plan->dev_tables)
      return fail(MLA_ERR_INVALID_ARG, "a plan of " + std::to_string(p.batch) +
                                           " sequences needs its tables staged with mla_verify_plan_stage_tables");
    a.dev_tables = plan->dev_tables;
  } else {
    a.dev_tables = nullptr;
    for (int b = 0; b <= p.batch; ++b) a.split_offset[b] = p.split_offset[b];
    for (int b = 0; b <= p.batch; ++b) a.group_offset[b] = p.group_offset[b];
    for (int b = 0; b <= p.batch; ++b) a.node_offset[b] = p.node_offset[b];
  }
  return MLA_OK;
}

mla_status launch_attend(const mlav::Plan& p, const mlav::VerifyArgs& a, void* stream) {
  const int e = mlav::launch_verify_attention(a, p.dtype, p.grid_blocks, stream);
  if (e != 0) return fail(MLA_ERR_HIP, "attention launch failed (hipError " + std::to_string(e) + ")");
  return MLA_OK;
}

mla_status launch_combine(const mlav::Plan& p, const mlav::VerifyArgs& a, void* stream) {
  if (!p.combine) return MLA_OK;
  const int e = mlav::launch_verify_combine(a, p.dtype, stream);
  if (e != 0) return fail(MLA_ERR_HIP, "combine launch failed (hipError " + std::to_string(e) + ")");
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_verify_run(mla_verify_plan_t plan, const void* q_nope, const void* q_pe,
                          const void* kv_c, const void* k_pe, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* tree_parents, float scale,
                          float* out, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream) {
  g_last_error.clear();
  mlav::VerifyArgs a;
  mla_status st = prepare(plan, q_nope, q_pe, kv_c, k_pe, kv_indptr, kv_indices, tree_parents, scale,
                          out, lse, workspace, workspace_bytes, true, a);
  if (st != MLA_OK) return st;
  st = launch_attend(plan->plan, a, stream);
  if (st != MLA_OK) return st;
  return launch_combine(plan->plan, a, stream);
}

mla_status mla_verify_run_varlen(mla_verify_plan_t plan, const void* q_nope, const void* q_pe,
                                 const void* kv_c, const void* k_pe, const int32_t* kv_indptr,
                                 const int32_t* kv_indices, const int32_t* tree_indptr,
                                 const int32_t* tree_parents, float scale, float* out, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!tree_indptr) return fail(MLA_ERR_INVALID_ARG, "tree_indptr is NULL");
  mlav::VerifyArgs a;
  mla_status st = prepare(plan, q_nope, q_pe, kv_c, k_pe, kv_indptr, kv_indices, tree_parents, scale,
                          out, lse, workspace, workspace_bytes, true, a, tree_indptr);
  if (st != MLA_OK) return st;
  st = launch_attend(plan->plan, a, stream);
  if (st != MLA_OK) return st;
  return launch_combine(plan->plan, a, stream);
}

mla_status mla_verify_run_noalloc(mla_verify_plan_t plan, const void* q_nope, const void* q_pe,
                                  const void* kv_c, const void* k_pe, const int32_t* kv_indptr,
                                  const int32_t* kv_indices, const int32_t* tree_parents, float scale,
                                  float* out, float* lse, void* stream) {
  g_last_error.clear();
  if (!plan) return fail(MLA_ERR_INVALID_ARG, "plan is NULL");
  const size_t need = plan->plan.ws_bytes, cap = mlav::noalloc_scratch_bytes();
  if (need > cap)
    return fail(MLA_ERR_WORKSPACE, "the plan needs " + std::to_string(need) +
                                       " bytes of workspace; the built-in buffer of mla_verify_run_noalloc holds " +
                                       std::to_string(cap));
  void* ws = nullptr;
  const int e = mlav::noalloc_scratch(&ws);
  if (e != 0) return fail(MLA_ERR_HIP, "locating the built-in workspace failed (hipError " + std::to_string(e) + ")");
  return mla_verify_run(plan, q_nope, q_pe, kv_c, k_pe, kv_indptr, kv_indices, tree_parents, scale, out, lse, ws,
                        cap, stream);
}

mla_status mla_verify_attend(mla_verify_plan_t plan, const void* q_nope, const void* q_pe,
                             const void* kv_c, const void* k_pe, const int32_t* kv_indptr,
                             const int32_t* kv_indices, const int32_t* tree_parents, float scale,
                             float* out, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream) {
  g_last_error.clear();
  mlav::VerifyArgs a;
  const mla_status st = prepare(plan, q_nope, q_pe, kv_c, k_pe, kv_indptr, kv_indices, tree_parents,
                                scale, out, lse, workspace, workspace_bytes, true, a);
  if (st != MLA_OK) return st;
  return launch_attend(plan->plan, a, stream);
}

mla_status mla_verify_combine(mla_verify_plan_t plan, float* out, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  mlav::VerifyArgs a;
  const mla_status st = prepare(plan, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                0.f, out, lse, workspace, workspace_bytes, false, a);
  if (st != MLA_OK) return st;
  return launch_combine(plan->plan, a, stream);
}

mla_status mla_verify_tree_masks(const int32_t* tree_parents, int32_t batch, int32_t tree_nodes,
                                 uint64_t* masks, void* stream) {
  g_last_error.clear();
  if (!tree_parents || !masks) return fail(MLA_ERR_INVALID_ARG, "NULL device pointer");
  if (batch < 1 || tree_nodes < 1 || tree_nodes > MLA_VERIFY_MAX_TREE)
    return fail(MLA_ERR_INVALID_ARG,
                "batch must be >= 1 and tree_nodes in 1.." + std::to_string(MLA_VERIFY_MAX_TREE));
  const int e = mlav::launch_tree_masks(tree_parents, batch, tree_nodes, masks, stream);
  if (e != 0) return fail(MLA_ERR_HIP, "tree mask launch failed (hipError " + std::to_string(e) + ")");
  return MLA_OK;
}

mla_status mla_kv_compact(int32_t dtype, int32_t batch, int64_t total_tokens, const void* kv_c,
                          const void* k_pe, int64_t kv_c_row_stride, int64_t k_pe_row_stride,
                          const int32_t* kv_indptr, const int32_t* kv_indices, void* dst_kv_c,
                          void* dst_k_pe, int64_t dst_kv_c_row_stride, int64_t dst_k_pe_row_stride,
                          int32_t dst_base, int32_t* new_kv_indices, void* stream) {
  g_last_error.clear();
  if (dtype != MLA_DTYPE_BF16 && dtype != MLA_DTYPE_F32)
    return fail(MLA_ERR_INVALID_ARG, "dtype must be MLA_DTYPE_F32 or MLA_DTYPE_BF16");
  if (batch < 1 || batch > MLA_VERIFY_MAX_BATCH)
    return fail(MLA_ERR_INVALID_ARG, "batch must be in 1.." + std::to_string(MLA_VERIFY_MAX_BATCH));
  if (total_tokens < 0) return fail(MLA_ERR_INVALID_ARG, "total_tokens < 0");
  if (dst_base < 0 || int64_t(dst_base) + total_tokens > int64_t(INT32_MAX))
    return fail(MLA_ERR_INVALID_ARG, "dst_base + total_tokens must fit in int32 (dst_base >= 0)");
  if (kv_c_row_stride < 512 || k_pe_row_stride < 64 || dst_kv_c_row_stride < 512 ||
      dst_k_pe_row_stride < 64 || kv_c_row_stride % 8 || k_pe_row_stride % 8 ||
      dst_kv_c_row_stride % 8 || dst_k_pe_row_stride % 8)
    return fail(MLA_ERR_INVALID_ARG, "row strides must be >= 512 (kv_c) / 64 (k_pe) and multiples of 8");
  if (!kv_c || !k_pe || !kv_indptr || !kv_indices || !dst_kv_c || !dst_k_pe || !new_kv_indices)
    return fail(MLA_ERR_INVALID_ARG, "NULL device pointer");
  if (!aligned16(kv_c) || !aligned16(k_pe) || !aligned16(dst_kv_c) || !aligned16(dst_k_pe))
    return fail(MLA_ERR_INVALID_ARG, "kv_c, k_pe and the destination pool must be 16-byte aligned");
  if (new_kv_indices == kv_indices) return fail(MLA_ERR_INVALID_ARG, "new_kv_indices may not alias kv_indices");
  if (total_tokens == 0) return MLA_OK;
  const int64_t es = dtype == MLA_DTYPE_BF16 ? 2 : 4;
  mlav::KvCompactArgs a{};
  a.kv_c = kv_c;
  a.k_pe = k_pe;
  a.kv_indptr = kv_indptr;
  a.kv_indices = kv_indices;
  a.dst_kv_c = dst_kv_c;
  a.dst_k_pe = dst_k_pe;
  a.new_indices = new_kv_indices;
  a.kv_c_stride_bytes = kv_c_row_stride * es;
  a.k_pe_stride_bytes = k_pe_row_stride * es;
  a.dst_kv_c_stride_bytes = dst_kv_c_row_stride * es;
  a.dst_k_pe_stride_bytes = dst_k_pe_row_stride * es;
  a.total = total_tokens;
  a.batch = batch;
  a.dst_base = dst_base;
  const int e = mlav::launch_kv_compact(a, int(es), stream);
  if (e != 0) return fail(MLA_ERR_HIP, "kv compaction launch failed (hipError " + std::to_string(e) + ")");
  return MLA_OK;
}

mla_status mla_tree_accept(const int32_t* tree_parents, const int32_t* draft_tokens,
                           const int32_t* target_tokens, const int32_t* root_targets, int32_t batch,
                           int32_t tree_nodes, int32_t* accept_len, int32_t* accept_path,
                           int32_t* bonus_token, void* stream) {
  g_last_error.clear();
  if (!tree_parents || !draft_tokens || !target_tokens || !root_targets || !accept_len || !accept_path ||
      !bonus_token)
    return fail(MLA_ERR_INVALID_ARG, "NULL device pointer");
  if (batch < 1 || tree_nodes < 1 || tree_nodes > MLA_TREE_ACCEPT_MAX_TREE)
    return fail(MLA_ERR_INVALID_ARG,
                "batch must be >= 1 and tree_nodes in 1.." + std::to_string(MLA_TREE_ACCEPT_MAX_TREE));
  const int e = mlav::launch_tree_accept(tree_parents, draft_tokens, target_tokens, root_targets, nullptr,
                                         batch, tree_nodes, accept_len, accept_path, bonus_token, stream);
  if (e != 0) return fail(MLA_ERR_HIP, "tree acceptance launch failed (hipError " + std::to_string(e) + ")");
  return MLA_OK;
}

mla_status mla_tree_accept_packed(const int32_t* tree_parents, const int32_t* draft_tokens,
                                  const int32_t* target_tokens, const int32_t* root_targets,
                                  const int32_t* tree_indptr, int32_t batch, int32_t max_tree_nodes,
                                  int32_t* accept_len, int32_t* accept_path, int32_t* bonus_token,
                                  void* stream) {
  g_last_error.clear();
  if (!tree_indptr || !root_targets || !accept_len || !bonus_token)
    return fail(MLA_ERR_INVALID_ARG, "NULL device pointer");
  if (max_tree_nodes > 0 && (!tree_parents || !draft_tokens || !target_tokens || !accept_path))
    return fail(MLA_ERR_INVALID_ARG, "NULL device pointer");
  if (batch < 1 || max_tree_nodes < 0 || max_tree_nodes > MLA_TREE_ACCEPT_MAX_TREE)
    return fail(MLA_ERR_INVALID_ARG, "batch must be >= 1 and max_tree_nodes in 0.." +
                                         std::to_string(MLA_TREE_ACCEPT_MAX_TREE));
  const int e = mlav::launch_tree_accept(tree_parents, draft_tokens, target_tokens, root_targets, tree_indptr,
                                         batch, max_tree_nodes, accept_len, accept_path, bonus_token, stream);
  if (e != 0) return fail(MLA_ERR_HIP, "tree acceptance launch failed (hipError " + std::to_string(e) + ")");
  return MLA_OK;
}

mla_status mla_verify_plan_destroy(mla_verify_plan_t plan) {
  delete plan;
  return MLA_OK;
}

const char* mla_verify_status_string(mla_status status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_verify_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
