/*
 * libmlaverify — tree-verify attention for absorbed-form MLA on MI355X (gfx950).
 *
 * The operation (from the pages this library follows):
 *   - Each cache token j holds a latent kv_c[j] (Dl = 512) and a decoupled RoPE
 *     key k_pe[j] (Dr = 64), shared by every head; the query is already
 *     multiplied into latent space ("absorbed"), so query row (b, t, h) brings
 *     q_nope (512) and q_pe (64).  ["Ground Truth in Silicon" page, "The Message
 *     in Full" (the reference docstring) and "Input Knowledge Required", item 2]
 *   - score(j) = scale * (q_nope . kv_c[j] + q_pe . k_pe[j]).
 *   - Visible keys of tree node t of sequence b: the whole prefix plus the
 *     tree-tail tokens of t and of its ancestors.  ["Reading the Reference"
 *     page, "Output Knowledge Created by This Message": prefix visibility +
 *     tree-tail visibility; "Ground Truth in Silicon" page, "Input Knowledge
 *     Required", item 3]
 *   - out = softmax(score) . kv_c over the visible keys (latent-space output;
 *     the caller applies W_UV), lse = natural-log log-sum-exp of the scaled
 *     scores.  ["Ground Truth in Silicon" page, "Output Knowledge Created",
 *     item 1: output aggregation]
 *   - Long sequences are cut into KV splits whose partial results are merged by
 *     log-sum-exp (flash-decode).  ["The Information-Gathering Pivot" page,
 *     "The Context: A Multi-Phase Kernel Integration"]
 *
 * Conventions for every entry point:
 *   - Device pointers point to memory of the current HIP device; host pointers
 *     are marked "host".  The caller owns every buffer and the stream; the
 *     library owns only the plan object (host memory).
 *   - No entry point throws.  Each returns an mla_status; on failure
 *     mla_verify_last_error() (thread-local) describes the first problem found.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 */
#ifndef MLA_VERIFY_H_
#define MLA_VERIFY_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1, /* bad size, NULL pointer, misaligned stride ... */
  MLA_ERR_UNSUPPORTED = -2, /* a valid request the library does not implement */
  MLA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than the plan needs */
  MLA_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} mla_status;

typedef enum { MLA_DTYPE_F32 = 0, MLA_DTYPE_BF16 = 1 } mla_dtype;

/* Opaque. Immutable after mla_verify_plan() (and, for batches above
   MLA_VERIFY_ARG_TABLE_BATCH, after mla_verify_plan_stage_tables()); safe to
   share between threads from then on. */
typedef struct mla_verify_plan_s* mla_verify_plan_t;

typedef struct {
  int32_t batch;            /* B sequences, 1..MLA_VERIFY_MAX_BATCH */
  int32_t num_heads;        /* H >= 1 */
  int32_t tree_nodes;       /* T nodes per sequence, 1..MLA_VERIFY_MAX_TREE; with
                               tree_len_host, an upper bound of every T_b */
  int32_t d_latent;         /* must be 512 */
  int32_t d_rope;           /* must be 64 */
  int32_t dtype;            /* mla_dtype of q_nope, q_pe, kv_c and k_pe; out/lse are fp32 */
  const int32_t* kv_len_host; /* host [batch]: N_b = P_b + T_b tokens of sequence b (>= T_b).
                                 Read during the call only; sizes the split schedule
                                 (the lengths a run sees may differ, see mla_verify_run). */
  int32_t num_splits;       /* 0 = planner's choice; > 0 forces that many KV splits
                               for every sequence (capped at its number of key tiles) */
  int64_t kv_c_row_stride;  /* elements between consecutive kv_c slots (>= 512, multiple of 8) */
  int64_t k_pe_row_stride;  /* elements between consecutive k_pe slots (>= 64, multiple of 8) */
  const int32_t* tree_len_host; /* host [batch]: T_b, the tree nodes of sequence b, each in
                                   0..tree_nodes (0: the sequence has no query this step),
                                   or NULL: every sequence has tree_nodes nodes. Read during
                                   the call only; fixed for the plan's runs. Every node
                                   of the draft tree is a query of the verify step, and
                                   the pages put no limit on how many there are ["Ground
                                   Truth in Silicon" page, "Input Knowledge Required",
                                   item 3]. */
} mla_verify_problem;

/* Sequences per plan. */
#define MLA_VERIFY_MAX_BATCH 65536
/* The per-sequence split, split-group and node offset tables (3 x (batch + 1)
   int32) travel in each launch's argument block for batches up to this size
   (the block may hold 4 KB). Larger batches keep them in device memory that
   the caller provides once, through mla_verify_plan_stage_tables(). */
#define MLA_VERIFY_ARG_TABLE_BATCH 256
/* Ancestor masks are four 64-bit words per node. */
#define MLA_VERIFY_MAX_TREE 256

/* Per-sequence status words: int32 [batch] at byte offset 0 of the workspace,
   written by the device on every run that has at least one tree node
   (mla_verify_run, mla_verify_run_varlen, mla_verify_attend); 0 = the
   sequence's tree and lengths are valid, else an OR of these bits.  They are
   stored with plain vector stores, never cleared in between, so capturing a
   run in a graph captures them too. */
#define MLA_VERIFY_STATUS_BAD_PARENT 1 /* a parent outside -1..node-1: the rows of
                                           every node whose ancestor chain meets it
                                           are NaN (out and lse) */
#define MLA_VERIFY_STATUS_SHORT_KV 2   /* N_b < T_b on the device: every row of the
                                           sequence is NaN */
#define MLA_VERIFY_STATUS_TREE_RANGE 4 /* mla_verify_run_varlen: tree_indptr entries
                                           out of range; no row of the sequence is
                                           written */

typedef struct {
  int32_t total_splits;     /* sum over sequences of the KV splits */
  int32_t max_splits;       /* largest split count of one sequence */
  int32_t rows_per_block;   /* query rows one workgroup processes */
  int32_t keys_per_tile;    /* keys staged in LDS per step */
  int32_t grid_blocks;      /* workgroups of the attention launch */
  int32_t uses_combine;     /* 1 when a split-combine launch follows */
  int32_t splits_per_workgroup; /* consecutive splits one workgroup runs (row block fixed),
                                   merged in its accumulators into one partial */
  int32_t total_groups;     /* sum over sequences of their split groups */
  size_t workspace_bytes;   /* same value mla_verify_plan() returned */
  size_t table_bytes;       /* device bytes mla_verify_plan_stage_tables() needs:
                               12 * (batch + 1) when batch > MLA_VERIFY_ARG_TABLE_BATCH,
                               else 0 (the tables travel in the launch arguments) */
  int64_t partial_rows;     /* (group, query row) partials one run writes and the
                               combine reads back: sum over sequences with more
                               than one group of groups * T_b * num_heads */
} mla_verify_plan_info;

/*
 * Validate a problem and build its launch plan (host only; no device work).
 * Checks: sizes above, dtype, strides, kv_len_host[b] >= tree_nodes.
 * On success *out receives a new plan and *workspace_bytes the device
 * workspace mla_verify_run() needs (bytes, 256-byte aligned start required).
 */
mla_status mla_verify_plan(const mla_verify_problem* problem, mla_verify_plan_t* out,
                           size_t* workspace_bytes);

/* Describe a plan (host only). */
mla_status mla_verify_plan_get_info(mla_verify_plan_t plan, mla_verify_plan_info* info);

/*
 * Batches above MLA_VERIFY_ARG_TABLE_BATCH only: copy the plan's per-sequence
 * tables (split, split-group and node offsets, int32 [3][batch + 1]) into
 * caller-owned device memory and have every later run of the plan read them
 * there. Call it once after mla_verify_plan() and before the plan's first
 * run, from one thread: it enqueues one host-to-device copy on `stream` and
 * records `tables` in the plan (not for graph capture; the runs it enables
 * are). Runs on other streams must be ordered after that copy by the caller.
 *   tables        device, >= table_bytes of mla_verify_plan_get_info(), 4-byte
 *                 aligned; owned by the caller, left unchanged and alive as long
 *                 as the plan runs.
 *   tables_bytes  its size.
 * For a plan whose tables fit the launch arguments it does nothing and
 * returns MLA_OK. Runs of a larger plan fail with MLA_ERR_INVALID_ARG until it
 * has been called.
 */
mla_status mla_verify_plan_stage_tables(mla_verify_plan_t plan, void* tables, size_t tables_bytes,
                                        void* stream);

/*
 * Tree-verify attention of one batch (device work on `stream`, asynchronous).
 *
 * Trees are packed: with node_off[b] = T_0 + ... + T_{b-1} (b*T when
 * tree_len_host is NULL), tree node t of sequence b is packed node
 * node_off[b] + t, and nodes = node_off[batch] in all.
 *   q_nope      device [nodes, H, 512] of dtype, row-major; row node_off[b] + t, head h
 *   q_pe        device [nodes, H, 64]  of dtype, row-major
 *   kv_c        device, slot s at kv_c + s*kv_c_row_stride, 512 elements
 *   k_pe        device, slot s at k_pe + s*k_pe_row_stride, 64 elements
 *               (kv_c and k_pe may interleave inside one 576-wide buffer)
 *   kv_indptr   device int32 [batch+1]; kv_indptr[0] = 0 and
 *               N_b = kv_indptr[b+1] - kv_indptr[b] >= T_b.  N_b may differ from
 *               the plan's kv_len_host[b] (one plan, or one captured graph,
 *               serves decode steps whose lengths change on the device): each
 *               sequence keeps the plan's split count over its actual length,
 *               and a split left without keys contributes nothing.
 *   kv_indices  device int32 [kv_indptr[batch]]: slot of logical position j of
 *               sequence b at kv_indices[kv_indptr[b] + j] (page_size = 1).
 *               Positions 0..P_b-1 are the prefix, P_b..P_b+T_b-1 the tree nodes.
 *               The library does not know the pool's size: every entry must be
 *               a slot of kv_c and k_pe (0 <= s < slots), or the kernels read
 *               outside them.
 *   tree_parents device int32 [nodes]: parent of packed node node_off[b] + t as
 *               a node index of the same tree, -1 = child of the last prefix
 *               token; parent[t] < t.  A node whose parent chain is invalid gets
 *               NaN output rows and lse.
 *   scale       softmax scale applied to the summed dot products; positive
 *               and below 2.3e38, so that scale * log2(e) is finite
 *               (MLA_ERR_INVALID_ARG otherwise)
 *   out         device fp32 [nodes, H, 512]
 *   lse         device fp32 [nodes, H] (natural log) or NULL
 *   workspace   device, >= workspace_bytes of the plan, 256-byte aligned.  Holds
 *               the status words (MLA_VERIFY_STATUS_*, int32 [batch] at offset
 *               0) and the split-group partials between the two launches; concurrent
 *               runs need separate workspaces.
 * No allocation, no host synchronisation, no memset and no host reads of
 * device data: the call only enqueues kernels, so it can be captured in a HIP
 * graph and replayed across decode steps (the pages' verify kernel was made
 * capture-safe for the serving loop's CUDA-graph capture: "The
 * Information-Gathering Pivot" page, "Input Knowledge and Assumptions" and
 * "The Significance of the Transition").
 * A plan whose trees are all empty (nodes = 0) enqueues nothing; q_nope, q_pe,
 * tree_parents, out and lse may then be NULL.
 */
mla_status mla_verify_run(mla_verify_plan_t plan, const void* q_nope, const void* q_pe,
                          const void* kv_c, const void* k_pe, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* tree_parents, float scale,
                          float* out, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * mla_verify_run with the tree packing read on the device, so that one plan
 * (or one captured graph) serves decode steps whose tree sizes change:
 *   tree_indptr device int32 [batch+1]: sequence b's nodes are packed nodes
 *               tree_indptr[b] .. tree_indptr[b+1]-1 of q_nope, q_pe,
 *               tree_parents, out and lse (sized for tree_indptr[batch] nodes).
 *               Its size T_b must lie in 0..the plan's size for b (its
 *               tree_len_host entry, or tree_nodes), which fixes the row
 *               blocks. A sequence whose size or offset is out of range is
 *               skipped: none of its rows are written.
 * Every other argument, the NaN rule for invalid parents and the capture
 * rules are those of mla_verify_run.
 */
mla_status mla_verify_run_varlen(mla_verify_plan_t plan, const void* q_nope, const void* q_pe,
                                 const void* kv_c, const void* k_pe, const int32_t* kv_indptr,
                                 const int32_t* kv_indices, const int32_t* tree_indptr,
                                 const int32_t* tree_parents, float scale, float* out, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_verify_run for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * launches, with the workspace taken from a buffer built into the library,
 * MLA_VERIFY_NOALLOC_WORKSPACE_BYTES per GPU, which each GPU the library runs on
 * holds from the first call on it until the process ends.  The arguments are
 * those of mla_verify_run without the workspace.  A plan whose workspace_bytes
 * exceeds the buffer is rejected with MLA_ERR_WORKSPACE before any device work.
 * The call allocates nothing (its first call on a device locates that device's
 * buffer).  Every call on one GPU uses the same buffer, which keeps the last
 * call's status words and partials (nothing in it has to start at zero), so
 * calls that overlap on one GPU race: calls on one stream are ordered, calls on
 * different streams or threads must be ordered by the caller.  The status words
 * of these calls are not readable by the caller (use mla_verify_run for them).
 * A plan of more than MLA_VERIFY_ARG_TABLE_BATCH sequences still needs its
 * tables staged (mla_verify_plan_stage_tables, once, in caller memory).
 */
#define MLA_VERIFY_NOALLOC_WORKSPACE_BYTES (64u << 20)
mla_status mla_verify_run_noalloc(mla_verify_plan_t plan, const void* q_nope, const void* q_pe,
                                  const void* kv_c, const void* k_pe, const int32_t* kv_indptr,
                                  const int32_t* kv_indices, const int32_t* tree_parents, float scale,
                                  float* out, float* lse, void* stream);

/*
 * The two halves of mla_verify_run, for callers that schedule or time them
 * separately. mla_verify_attend takes exactly the arguments of mla_verify_run
 * and enqueues the attention kernel. One workgroup runs a split group:
 * splits_per_workgroup consecutive KV splits of one row block, which share
 * one reference max, so their merge is a plain sum kept in the workgroup's
 * accumulators. Sequences with a single split group write out/lse directly;
 * the others leave one partial per split group in the workspace: an fp32
 * record per row (m, l and two scales), and the group's unnormalised output
 * O = l * o_group: fp32 for fp32 problems; for bf16 problems fp16 times a
 * power of two per row and feature half (its inverse is one of the record's
 * scales), which moves the result by at most
 * 2^-12 of that half's largest |o_group| (bf16 storage would move each
 * element by up to 2^-9 of itself, about 8e-3 where a row's weight sits on
 * a few keys with latent values near 4).
 * mla_verify_combine then merges those partials by log-sum-exp into out/lse
 * (it enqueues nothing when no sequence has more than one split group,
 * uses_combine = 0). Calling attend and
 * then combine on one stream with the same workspace equals mla_verify_run.
 */
mla_status mla_verify_attend(mla_verify_plan_t plan, const void* q_nope, const void* q_pe,
                             const void* kv_c, const void* k_pe, const int32_t* kv_indptr,
                             const int32_t* kv_indices, const int32_t* tree_parents, float scale,
                             float* out, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream);

mla_status mla_verify_combine(mla_verify_plan_t plan, float* out, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * Ancestor-or-self bitmask of every tree node (device work on `stream`).
 *   tree_parents device int32 [batch, tree_nodes], as in mla_verify_run
 *   tree_nodes   1..MLA_VERIFY_MAX_TREE; W = ceil(tree_nodes / 64) words per node
 *   masks        device uint64 [batch, tree_nodes, W]; bit u % 64 of word u / 64
 *                of node (b, t) is set iff node u is t or an ancestor of t.  All
 *                words 0 mark an invalid parent chain (parent >= node or < -1
 *                somewhere on it).
 * This is the mask mla_verify_run applies to the tree-tail keys.
 */
mla_status mla_verify_tree_masks(const int32_t* tree_parents, int32_t batch, int32_t tree_nodes,
                                 uint64_t* masks, void* stream);

mla_status mla_verify_plan_destroy(mla_verify_plan_t plan);

/* Static string naming a status code. */
const char* mla_verify_status_string(mla_status status);

/* Thread-local description of the last failure on this thread ("" if none). */
const char* mla_verify_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_VERIFY_H_ */
