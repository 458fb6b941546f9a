// Host fuzz driver for libmlaverify's planner and C-ABI argument checks, built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizer.py. The kernel launchers are stubs that check the
// argument block they receive (workspace regions inside the workspace, offset
// tables consistent with the plan) instead of launching anything.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/mla_kv_compact.h"
#include "../../include/mla_tree_accept.h"
#include "../../include/mla_verify.h"
#include "../../mla_absorbed_tree_amd/csrc/kernel_params.h"
#include "../../mla_absorbed_tree_amd/csrc/kv_compact_params.h"

namespace {

uintptr_t g_ws = 0;
size_t g_ws_bytes = 0;
long g_launches = 0, g_failures = 0;

void check(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "check failed: %s\n", what);
    ++g_failures;
  }
}

// splitmix64
uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next() {
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
int64_t uni(int64_t lo, int64_t hi) { return lo + int64_t(next() % uint64_t(hi - lo + 1)); }

// What the stubbed table copy received: the device address and the bytes.
const void* g_tables_dev = nullptr;
std::vector<int32_t> g_tables_host;

void check_args(const mlav::VerifyArgs& a) {
  check(a.batch >= 1 && a.batch <= MLA_VERIFY_MAX_BATCH, "batch");
  check(reinterpret_cast<uintptr_t>(a.status) == g_ws, "status words at workspace offset 0");
  // Tables in the arguments up to MLA_VERIFY_ARG_TABLE_BATCH, else the staged copy.
  check((a.dev_tables != nullptr) == (a.batch > MLA_VERIFY_ARG_TABLE_BATCH), "table location");
  if (a.dev_tables)
    check(a.dev_tables == g_tables_dev && g_tables_host.size() == 3 * size_t(a.batch + 1), "staged tables");
  auto tab = [&](int t, int i) {
    if (a.dev_tables) return g_tables_host[size_t(t) * (a.batch + 1) + i];
    return t == 0 ? a.split_offset[i] : t == 1 ? a.group_offset[i] : a.node_offset[i];
  };
  int max_groups = 0;
  for (int b = 0; b < a.batch; ++b) {
    check(tab(0, b) <= tab(0, b + 1), "split offsets monotone");
    check(tab(1, b) <= tab(1, b + 1), "group offsets monotone");
    check(tab(2, b) <= tab(2, b + 1), "node offsets monotone");
    max_groups = std::max(max_groups, tab(1, b + 1) - tab(1, b));
  }
  check(a.max_groups == max_groups, "max_groups");
  check(a.part_rows >= a.max_rows_per_seq, "partial rows cover every sequence");
  if (a.part_o) {
    const size_t rows = size_t(tab(1, a.batch)) * size_t(a.part_rows);  // one per split group
    const uintptr_t o = reinterpret_cast<uintptr_t>(a.part_o), ml = reinterpret_cast<uintptr_t>(a.part_ml);
    check(ml >= g_ws + 4 * size_t(a.batch), "partials after the status words");
    check(ml + rows * 16 <= o, "(m, l, s0, s1) before O");
    check(o + rows * 512 * 2 <= g_ws + g_ws_bytes, "O inside the workspace");  // fp16 lower bound
  }
}

}  // namespace

namespace mlav {
int launch_verify_attention(const VerifyArgs& a, int, int64_t grid_blocks, void*) {
  ++g_launches;
  check(grid_blocks >= 0, "grid");
  if (grid_blocks == 0) return 0;  // every tree empty: the real launcher enqueues nothing
  check_args(a);
  return 0;
}
int launch_verify_combine(const VerifyArgs& a, int, void*) {
  check_args(a);
  return 0;
}
int launch_tree_masks(const int32_t*, int32_t, int32_t, uint64_t*, void*) { return 0; }
int launch_tree_accept(const int32_t*, const int32_t*, const int32_t*, const int32_t*, const int32_t*, int32_t,
                       int32_t, int32_t*, int32_t*, int32_t*, void*) {
  return 0;
}
int launch_kv_compact(const KvCompactArgs& a, int es, void*) {
  check(es == 2 || es == 4, "element size");
  check(a.total > 0, "total");
  return 0;
}
int copy_tables_to_device(void* dst, const void* src, size_t bytes, void*) {
  check(bytes % 4 == 0, "table bytes");
  g_tables_dev = dst;
  g_tables_host.assign(static_cast<const int32_t*>(src), static_cast<const int32_t*>(src) + bytes / 4);
  return 0;
}
size_t noalloc_scratch_bytes() { return size_t(MLA_VERIFY_NOALLOC_WORKSPACE_BYTES); }
int noalloc_scratch(void** ptr) {
  *ptr = reinterpret_cast<void*>(g_ws);
  return 0;
}
}  // namespace mlav

int main(int argc, char** argv) {
  const long iters = argc > 1 ? std::atol(argv[1]) : 3000;
  void* const fake = reinterpret_cast<void*>(uintptr_t(1) << 40);  // never dereferenced
  long planned = 0;
  for (long it = 0; it < iters; ++it) {
    // Mostly valid problems (so the plans and runs are exercised), each field
    // with a small chance of an invalid value.
    const bool bad = uni(0, 4) == 0;
    auto pick = [&](int64_t lo, int64_t hi, int64_t blo, int64_t bhi) { return bad && uni(0, 5) == 0 ? uni(blo, bhi) : uni(lo, hi); };
    mla_verify_problem p{};
    p.batch = int32_t(pick(1, uni(0, 3) ? 16 : uni(0, 3) ? 256 : 1200, -2, MLA_VERIFY_MAX_BATCH + 2));
    p.num_heads = int32_t(pick(1, 130, -1, 0));
    p.tree_nodes = int32_t(pick(1, uni(0, 1) ? 64 : 256, -1, 300));
    p.d_latent = int32_t(pick(512, 512, 500, 520));
    p.d_rope = int32_t(pick(64, 64, 60, 70));
    p.dtype = int32_t(pick(0, 1, -1, 2));
    p.num_splits = int32_t(uni(0, 3) ? pick(0, 8, -1, -1) : pick(0, 600, -1, -1));
    const int64_t strides_c[] = {512, 576, 1024, 513, 8, 0};
    const int64_t strides_p[] = {64, 576, 128, 65, 8, 0};
    p.kv_c_row_stride = strides_c[pick(0, 2, 3, 5)];
    p.k_pe_row_stride = strides_p[pick(0, 2, 3, 5)];
    const int nb = p.batch > 0 ? p.batch : 1;
    std::vector<int32_t> kv(nb), tl(nb);
    const int tmax = p.tree_nodes > 0 ? p.tree_nodes : 1;
    for (int b = 0; b < nb; ++b) {
      tl[b] = int32_t(uni(0, 2000) ? uni(0, tmax) : uni(-2, tmax + 3));
      kv[b] = int32_t(uni(0, 2000) ? uni(tmax, tmax + (uni(0, 3) ? 5000 : 300000)) : uni(-1, tmax + 2));
    }
    p.kv_len_host = pick(0, 0, 1, 1) ? nullptr : kv.data();
    p.tree_len_host = uni(0, 1) ? tl.data() : nullptr;

    mla_verify_plan_t plan = nullptr;
    size_t ws_bytes = 0;
    const mla_status st = mla_verify_plan(&p, &plan, &ws_bytes);
    if (st != MLA_OK) {
      check(plan == nullptr, "no plan on failure");
      check(std::strlen(mla_verify_last_error()) > 0, "error message");
      continue;
    }
    ++planned;
    mla_verify_plan_info info{};
    check(mla_verify_plan_get_info(plan, &info) == MLA_OK, "info");
    check(info.workspace_bytes == ws_bytes && ws_bytes >= 4 * size_t(p.batch), "workspace size");
    g_ws = uintptr_t(1) << 41;
    g_ws_bytes = ws_bytes;
    void* ws = reinterpret_cast<void*>(g_ws);
    const int32_t* ip = static_cast<const int32_t*>(fake);
    float* fo = static_cast<float*>(fake);
    // Batches above MLA_VERIFY_ARG_TABLE_BATCH run only once their tables are staged.
    check(info.table_bytes == (p.batch > MLA_VERIFY_ARG_TABLE_BATCH ? 12 * size_t(p.batch + 1) : 0), "table bytes");
    void* const tables = reinterpret_cast<void*>(uintptr_t(1) << 42);
    if (info.table_bytes > 0) {
      check(mla_verify_run(plan, fake, fake, fake, fake, ip, ip, ip, 0.07f, fo, fo, ws, ws_bytes, nullptr) ==
                MLA_ERR_INVALID_ARG,
            "run before the tables are staged");
      check(mla_verify_plan_stage_tables(plan, tables, info.table_bytes - 4, nullptr) == MLA_ERR_INVALID_ARG,
            "short table buffer");
    }
    check(mla_verify_plan_stage_tables(plan, tables, info.table_bytes, nullptr) == MLA_OK, "stage tables");
    const mla_status r = mla_verify_run(plan, fake, fake, fake, fake, ip, ip, ip, 0.07f, fo, fo, ws, ws_bytes, nullptr);
    check(r == MLA_OK, "run with valid arguments");
    check(mla_verify_run(plan, fake, fake, fake, fake, ip, ip, ip, 0.07f, fo, fo, ws, ws_bytes - 1, nullptr) ==
              MLA_ERR_WORKSPACE,
          "short workspace rejected");
    check(mla_verify_run(plan, fake, fake, fake, fake, ip, ip, ip, -1.f, fo, fo, ws, ws_bytes, nullptr) ==
              MLA_ERR_INVALID_ARG,
          "negative scale rejected");
    check(mla_verify_run_varlen(plan, fake, fake, fake, fake, ip, ip, ip, ip, 0.07f, fo, fo, ws, ws_bytes,
                                nullptr) == MLA_OK,
          "varlen run");
    const mla_status na = mla_verify_run_noalloc(plan, fake, fake, fake, fake, ip, ip, ip, 0.07f, fo, fo, nullptr);
    check(na == (ws_bytes <= size_t(MLA_VERIFY_NOALLOC_WORKSPACE_BYTES) ? MLA_OK : MLA_ERR_WORKSPACE), "noalloc");
    check(mla_verify_plan_destroy(plan) == MLA_OK, "destroy");
  }
  // Argument checks of the other entry points.
  for (long it = 0; it < iters; ++it) {
    const int32_t b = int32_t(uni(-1, 300)), t = int32_t(uni(-1, 300));
    const int64_t n = uni(-1, 1 << 20);
    void* f = uni(0, 9) ? fake : nullptr;
    mla_kv_compact(int32_t(uni(-1, 2)), b, n, f, fake, int64_t(uni(0, 3) ? 512 : uni(0, 600)), 64, static_cast<const int32_t*>(fake),
                   static_cast<const int32_t*>(fake), fake, fake, 512, 64, int32_t(uni(-1, 1000)),
                   static_cast<int32_t*>(f), nullptr);
    mla_tree_accept(static_cast<const int32_t*>(f), static_cast<const int32_t*>(fake),
                    static_cast<const int32_t*>(fake), static_cast<const int32_t*>(fake), b, t,
                    static_cast<int32_t*>(fake), static_cast<int32_t*>(fake), static_cast<int32_t*>(fake), nullptr);
    mla_tree_accept_packed(static_cast<const int32_t*>(f), static_cast<const int32_t*>(fake),
                           static_cast<const int32_t*>(fake), static_cast<const int32_t*>(fake),
                           static_cast<const int32_t*>(fake), b, t, static_cast<int32_t*>(fake),
                           static_cast<int32_t*>(fake), static_cast<int32_t*>(fake), nullptr);
    mla_verify_tree_masks(static_cast<const int32_t*>(f), b, t, static_cast<uint64_t*>(fake), nullptr);
    mla_verify_status_string(mla_status(uni(-6, 1)));
  }
  std::printf("iterations %ld planned %ld launches %ld failures %ld\n", iters, planned, g_launches, g_failures);
  return g_failures == 0 && planned > 0 ? 0 : 1;
}
