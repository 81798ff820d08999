/*
 * oracle.h - TEST INFRASTRUCTURE ONLY. A plain, slow fp64 CPU oracle for
 * tree-verify attention and acceptance. Only the tests, the smoke check and
 * the bench's CPU-baseline leg may load it; the product library never does.
 * It shares no code, header or constant table with the GPU library.
 *
 * Status codes (same numbering as the library's public status enum, restated
 * here on purpose so the two stay independent):
 *   0 OK, 1 invalid argument, 2 invalid tree, 3 unsupported, 4 workspace, 5 runtime.
 *
 * Parity pins for every function are in tests/test_oracle_*.py; none of the
 * functions here is pinned by page-printed values (the pages print no worked
 * example), so each is pinned by closed forms, brute force, library routines
 * on special cases and statistical identities instead.
 */
#ifndef TV_ORACLE_H
#define TV_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  TVO_OK = 0,
  TVO_ERR_INVALID_ARG = 1,
  TVO_ERR_INVALID_TREE = 2,
  TVO_ERR_UNSUPPORTED = 3,
  TVO_ERR_WORKSPACE = 4,
  TVO_ERR_RUNTIME = 5
};

/* Node counts: tree_sizes [B] (nullable, NULL = every sequence has N nodes)
 * gives sequence b n_b nodes, 1 <= n_b <= N <= 128; nodes n_b..N-1 are
 * absent: their parents, tokens, logits rows and K/V are never read, mask
 * rows are 0 with depth -1, attention rows are NaN, argmax rows -1. */

/* Ancestor-or-self mask and depth of every node (EAGLE-2 deep-dive page,
 * tree-mask assembly in its reference code): bit j of mask[b][i][j/64]
 * (bit position j%64, least significant bit = node 0) is set iff j is met on
 * the walk i, parent[i], parent[parent[i]], ... ; depth[i] = (#set bits) - 1. */
int tvo_build_mask(const int32_t *parents, const int32_t *tree_sizes, int32_t B, int32_t N, uint64_t *mask,
                   int32_t *depth);

/* Tree-masked paged GQA attention in fp64 for the listed rows.
 * rows: [n_rows][3] triples (b, i, h), or NULL for every row in [B][N][Hq]
 * order. out: [n_rows][D] doubles. tree_mask NULL = every tree node visible. */
int tvo_attention(const uint16_t *q, const uint16_t *k_pages, const uint16_t *v_pages, int64_t num_pages,
                  const int32_t *page_table, int32_t maxp, const int32_t *prefix_lens, int32_t max_prefix_len,
                  const uint64_t *tree_mask, const int32_t *tree_sizes, int32_t B, int32_t N, int32_t Hq,
                  int32_t Hkv, int32_t D, float sm_scale, const int32_t *rows, int64_t n_rows, double *out,
                  int nthreads);

/* Greedy acceptance: longest root path of matching nodes, lexicographically
 * smallest on ties; accept_len counts the bonus token. */
int tvo_accept_greedy(const float *target_logits, const int32_t *draft_tokens, const int32_t *parents,
                      const int32_t *tree_sizes, int32_t B, int32_t N, int32_t V, int32_t *accept_len, int32_t *path,
                      int32_t *bonus, int32_t *target_argmax, int nthreads);

/* Stochastic acceptance on a chain or tree: from the root, test the current
 * node's children in id order, child c accepted iff u[c-1] < pi(t_c)/q_c(t_c)
 * with pi = p_node at first and, after each rejected sibling, the normalised
 * residual max(0, pi - q_c); when no child is accepted, draw the next token
 * from pi by inverse CDF with u[N-1]. margins [B][N] (nullable): |u - a| for
 * each tested node c at [c-1], distance of the final draw to the nearest CDF
 * boundary relative to the total mass at [N-1], +inf where unused. */
int tvo_accept_stochastic(const float *target_logits, const float *draft_logits, const int32_t *draft_tokens,
                          const int32_t *parents, const int32_t *tree_sizes, const float *uniforms, int32_t B,
                          int32_t N, int32_t V,
                          float temperature, int32_t *accept_len, int32_t *path, int32_t *bonus, double *margins,
                          int nthreads);

/* Accepted-path KV commit (EAGLE-2 page, third pillar: no KV-cache pollution;
 * Sonar page, MTP schedule: next token inserted on the device). Committed
 * position L+m receives the K/V of path node v_m (all KV heads, read before
 * written); new_prefix_lens[b] = L + len; emitted [B][N] (nullable) =
 * draft_tokens at v_1..v_{len-1}, then the bonus, -1 padded; next_root[b] =
 * bonus. k_pages and v_pages are updated in place. Bad sequences are left
 * unchanged (length L, root -1, emitted -1) and make the call return 1. */
int tvo_commit(uint16_t *k_pages, uint16_t *v_pages, int64_t num_pages, const int32_t *page_table, int32_t maxp,
               const int32_t *prefix_lens, int32_t max_prefix_len, const int32_t *draft_tokens,
               const int32_t *path, const int32_t *accept_len, const int32_t *bonus, int32_t B, int32_t N,
               int32_t Hkv, int32_t D, int32_t *new_prefix_lens, int32_t *emitted, int32_t *next_root);

/* Dynamic draft-tree construction (EAGLE-2 page, dynamic-tree algorithm and
 * its reference code): best-first by cumulative score from the root's
 * top-k_root proposals; a created node shallower than max_depth queues its
 * top-k children whose cumulative score is > threshold; N nodes at most.
 * cand_tokens / cand_probs [B][N][k]: row i = proposals of the node created
 * i-th. Outputs [B][N] (depth, mask, scores, n_nodes nullable); unused slots
 * are padding (parent -1, root token, depth 0, self mask, score 0). */
int tvo_build_tree(const int32_t *root_tokens, const int32_t *cand_tokens, const float *cand_probs, int32_t B,
                   int32_t N, int32_t k, int32_t k_root, float threshold, int32_t max_depth, int32_t *parents,
                   int32_t *tokens, int32_t *depth, uint64_t *mask, double *scores, int32_t *n_nodes);

/* tau = (1/M) sum_j n_accepted(j) over M verification cycles (EAGLE-3 page,
 * tree acceptance rate definition); 0 when M = 0. */
double tvo_tau(const int32_t *accept_len, int64_t M);

#ifdef __cplusplus
}
#endif
#endif
