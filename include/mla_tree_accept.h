/*
 * libmlaverify — token acceptance over a verified draft tree (gfx950).
 *
 * The pages list token acceptance among the kernels of the speculative-decoding
 * engine next to tree-verify attention and tree construction ["Ground Truth in
 * Silicon" page, "Input Knowledge Required", item 1] but do not define it.
 * This entry point takes the plainest reading, greedy acceptance along the tree:
 *
 *   Node t of sequence b carries the draft token draft[b, t]. After the
 *   verify pass the target model's greedy next token is known after every
 *   node's path (target[b, t]) and after the last prefix token
 *   (root_target[b]). Node t is accepted when its own draft token equals the
 *   target's token after its parent (root_target for a node whose parent is
 *   -1) and its parent is accepted. The accepted nodes form rooted paths; the
 *   result is the deepest accepted node t* (ties: the smallest node index):
 *     accept_len[b]          = depth of t* (nodes on its root path), 0 if no
 *                              node is accepted
 *     accept_path[b, 0..T-1] = the nodes of that path from the root down, then
 *                              -1
 *     bonus_token[b]         = target[b, t*], or root_target[b] when
 *                              accept_len is 0 (the token the target emits
 *                              after the accepted draft)
 *   A node with an invalid parent chain (parent >= node or < -1 on its root
 *   path, as in mla_verify_run) is never accepted.
 *
 * Conventions as in mla_verify.h. Declared here, defined in libmlaverify.
 */
#ifndef MLA_TREE_ACCEPT_H_
#define MLA_TREE_ACCEPT_H_

#include <stdint.h>

#include "mla_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Largest tree the acceptance kernels handle (the verify limit). */
#define MLA_TREE_ACCEPT_MAX_TREE MLA_VERIFY_MAX_TREE

/*
 *   tree_parents  device int32 [batch, T], as for mla_verify_run
 *   draft_tokens  device int32 [batch, T]
 *   target_tokens device int32 [batch, T]: target's greedy token after node t
 *   root_targets  device int32 [batch]: target's token after the last prefix
 *                 token of sequence b
 *   batch >= 1, T = tree_nodes in 1..MLA_TREE_ACCEPT_MAX_TREE
 *   accept_len    device int32 [batch], written
 *   accept_path   device int32 [batch, T], written
 *   bonus_token   device int32 [batch], written
 * One wave per sequence for T <= 64, one 256-lane workgroup per sequence
 * above; asynchronous, allocates nothing (graph-capturable).
 * Errors: MLA_ERR_INVALID_ARG (NULL pointer, bad sizes; nothing launched),
 * MLA_ERR_HIP if the launch fails.
 */
mla_status mla_tree_accept(const int32_t* tree_parents, const int32_t* draft_tokens,
                           const int32_t* target_tokens, const int32_t* root_targets, int32_t batch,
                           int32_t tree_nodes, int32_t* accept_len, int32_t* accept_path,
                           int32_t* bonus_token, void* stream);

/*
 * The same acceptance over packed trees, one size per sequence (the layout of
 * mla_verify_run with tree_len_host): sequence b owns nodes
 * tree_indptr[b] .. tree_indptr[b+1]-1 of the flat arrays.
 *   tree_indptr    device int32 [batch+1], tree_indptr[0] = 0, non-decreasing
 *   tree_parents, draft_tokens, target_tokens
 *                  device int32 [tree_indptr[batch]]; parents are node indices
 *                  of the same tree (-1 = child of the last prefix token)
 *   root_targets   device int32 [batch]
 *   max_tree_nodes 0..MLA_TREE_ACCEPT_MAX_TREE, at least every T_b; sizes the
 *                  launch (64 lanes per sequence up to 64, else 256)
 *   accept_len     device int32 [batch], written; -1 marks a sequence whose
 *                  device entries are out of range: a size outside
 *                  0..max_tree_nodes, a negative offset, or a tree that ends
 *                  past tree_indptr[batch] (its path slots are then not written)
 *   accept_path    device int32 [tree_indptr[batch]], written: sequence b's
 *                  path from its root down at tree_indptr[b], then -1 up to T_b
 *   bonus_token    device int32 [batch], written (root_targets[b] for an empty
 *                  tree or a rejected size)
 * The rule, conventions and errors are those of mla_tree_accept. An empty tree
 * accepts nothing (accept_len 0). The arrays of the nodes may be NULL when
 * max_tree_nodes is 0.
 */
mla_status mla_tree_accept_packed(const int32_t* tree_parents, const int32_t* draft_tokens,
                                  const int32_t* target_tokens, const int32_t* root_targets,
                                  const int32_t* tree_indptr, int32_t batch, int32_t max_tree_nodes,
                                  int32_t* accept_len, int32_t* accept_path, int32_t* bonus_token,
                                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_TREE_ACCEPT_H_ */
