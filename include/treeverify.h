/*
 * treeverify.h - C ABI of libtreeverify: the verification pass of tree
 * speculative decoding (EAGLE-2 / EAGLE-3 style) on one AMD Instinct MI355X.
 *
 * Sources, by page title:
 *  [EAGLE-2 page]  "EAGLE-2 심층 아키텍처: 특징 공간(Feature Space) 자동회귀와 동적
 *                  초안 트리..." (techknowgenie) - third pillar (one target
 *                  forward verifies every tree node through a 2D tree mask
 *                  injected into the attention kernel; the longest accepted
 *                  path is kept), the reference code's tree-mask loop, the
 *                  benchmark discussion (rejection sampling keeps the output
 *                  lossless) and the production note on indexing tree masks
 *                  directly over paged KV memory.
 *  [Sonar page]    "Accelerating Sonar through speculation" (Perplexity) -
 *                  four stages of speculative sampling (longest acceptable
 *                  prefix; the target's logits at the mismatch or the end give
 *                  one more token), draft-target acceptance by comparing full
 *                  distributions, and the device-side insertion that avoids a
 *                  CPU-GPU sync on the accepted length.
 *  [EAGLE-3 page]  "論文解説: EAGLE-3 - Training-Time Test-Scaling..." - tau,
 *                  the mean number of tokens accepted per draft/verify cycle.
 *
 * Conventions for every call
 *  - Pointers are DEVICE pointers unless marked (host). The caller allocates
 *    and owns every buffer, workspaces included; the library never allocates
 *    device memory in these calls (only tv_create does: 64 bytes of
 *    counters and flags plus 256 KB of per-sequence arrival counters).
 *  - Calls are asynchronous on the context's HIP stream, except tv_tau and
 *    tv_device_error, which synchronise that stream.
 *  - Host-detected errors return a status and launch nothing; outputs are
 *    left untouched.
 *  - Device-detected bad data (a parent not earlier than its child, a page id
 *    outside [0, num_pages), a token outside [0, V), a prefix length outside
 *    [0, max_prefix_len]) sets a sticky
 *    per-context flag read by tv_device_error; the affected outputs are
 *    written as NaN (attention) or -1 (masks: 0 with depth -1; acceptance).
 *  - Tree numbering: node ids are topological (parent[i] < i), as in the
 *    EAGLE-2 page's reference code which numbers nodes in creation order.
 *    Node 0 is the root: the last verified token, counted in the tree.
 *  - Tree sizes: N <= 128 node slots per sequence; masks have W =
 *    ceil(N / 64) words per row. tree_sizes int32 [B] (nullable; NULL =
 *    every sequence has N nodes) gives sequence b n_b nodes, 1 <= n_b <= N;
 *    slots n_b..N-1 are absent: their parents, tokens, logits rows and K/V
 *    are never read; mask rows are written 0 with depth -1, attention rows
 *    are not written, argmax rows are -1. A count outside [1, N] sets the
 *    sticky TV_ERR_INVALID_ARG (that sequence's outputs as for bad data).
 *  - A context is not thread-safe; use one per thread. Its calls run in
 *    issue order even across tv_set_stream (see there).
 */
#ifndef TREEVERIFY_H
#define TREEVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tv_status {
  TV_OK = 0,
  TV_ERR_INVALID_ARG = 1,  /* bad scalar, NULL pointer, bad page id / token / prefix length */
  TV_ERR_INVALID_TREE = 2, /* parent[b][i] outside {-1} U [0, i), or accept root with a parent */
  TV_ERR_UNSUPPORTED = 3,  /* shape outside what the kernels implement (N > 128, D not 64/128) */
  TV_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than the *_workspace_bytes figure */
  TV_ERR_HIP = 5           /* HIP runtime error (launch failure, bad device) */
} tv_status;

typedef enum tv_dtype { TV_F32 = 0, TV_BF16 = 1 } tv_dtype;

typedef enum tv_accept_mode { TV_GREEDY = 0, TV_STOCHASTIC = 1 } tv_accept_mode;

typedef struct tv_ctx tv_ctx;

/* Creates a context on `device` bound to `hip_stream` (a hipStream_t; NULL =
 * the default stream). Allocates, zeroed, 64 bytes of device memory for the
 * tau counters and the sticky error flag and 256 KB of per-sequence arrival
 * counters that small greedy tv_accept calls use (each call leaves them
 * zero), plus one HIP event. *ctx is host memory. */
tv_status tv_create(tv_ctx **ctx, int device, void *hip_stream);
tv_status tv_destroy(tv_ctx *ctx);
/* Rebinds the context to another stream of the same device. Work already
 * queued on the previous stream is ordered before later calls (an event
 * recorded there that the new stream waits for), so the context's device
 * counters are never used by two calls at once. The previous stream must
 * still exist when this is called; rebinding to the same stream does
 * nothing. */
tv_status tv_set_stream(tv_ctx *ctx, void *hip_stream);

/* Ancestor-or-self bitmask of every tree node ([EAGLE-2 page], reference
 * code, tree-mask assembly: a node's row marks the node, then each parent up
 * to the root).
 *   parents     int32 [B][N]: parent id, or -1 for a root (forests allowed).
 *   tree_sizes  int32 [B] or NULL: node counts (see the conventions above).
 *   mask        uint64 [B][N][W], W = ceil(N/64): bit j (position j % 64 of
 *               word j / 64, least significant bit = node 0) of row (b, i)
 *               is set iff j is i or an ancestor of i.
 *   depth       int32 [B][N] or NULL: number of ancestors (root = 0); a
 *               node's position id would be prefix_len + depth.
 * Requires 0 <= N <= 128, B >= 0. Bad parents among the present nodes:
 * sticky TV_ERR_INVALID_TREE and that sequence's rows are written as mask 0,
 * depth -1. */
tv_status tv_build_mask(tv_ctx *ctx, const int32_t *parents, const int32_t *tree_sizes, int32_t B, int32_t N,
                        uint64_t *mask, int32_t *depth);

/* Dynamic draft-tree construction ([EAGLE-2 page], dynamic-tree algorithm
 * section and its reference code's builder). A node's cumulative score is the
 * product of the draft probabilities on its root path (root = 1). The queue
 * starts with the root's first k_root proposals (queued whatever their
 * score); repeatedly the queued candidate with the highest score becomes the
 * next node (ids in creation order, so parents come first; on equal scores
 * the candidate queued first); a node whose depth is below max_depth then
 * queues those of its k proposals whose cumulative score is > threshold (the
 * reference code's strict test), in slot order. Construction stops at N
 * nodes (root included) or when the queue is empty.
 *   root_tokens  int32 [B]: node 0's token (the last verified token)
 *   cand_tokens  int32 [B][N][k], cand_probs fp32 [B][N][k]: row i holds the
 *                draft head's top-k proposals (token, probability) for the
 *                node created i-th (row 0: the root); rows of nodes that are
 *                never created or never expanded are not read for scores
 *   threshold    fp32, compared in fp64 with the fp64 product of fp32 scores
 *   parents, tokens  int32 [B][N]: the tree, in the layout tv_build_mask,
 *                tv_attention and tv_accept take
 *   depth int32 [B][N], mask uint64 [B][N][W] (ancestor-or-self bits as
 *                tv_build_mask writes them), scores fp64 [B][N] (cumulative),
 *                n_nodes int32 [B]: all nullable
 * Slots past n_nodes of a short tree are padding: parent -1, the root's
 * token, depth 0, mask = the slot's own bit, score 0 (never accepted).
 * Requires 1 <= N <= 128, 1 <= k_root <= k <= 32, max_depth >= 1, threshold
 * not NaN. A sequence with a NaN or negative probability anywhere in its
 * table is written as padding with n_nodes 0 and sets the sticky
 * TV_ERR_INVALID_ARG. */
tv_status tv_build_tree(tv_ctx *ctx, const int32_t *root_tokens, const int32_t *cand_tokens, const float *cand_probs,
                        int32_t B, int32_t N, int32_t k, int32_t k_root, float threshold, int32_t max_depth,
                        int32_t *parents, int32_t *tokens, int32_t *depth, uint64_t *mask, double *scores,
                        int32_t *n_nodes);

/* Workspace (bytes) tv_attention needs for these host scalars: partial
 * results when one sequence's keys are split over several workgroups (per
 * row and split: the normalised partial output in fp16, or in fp32 for rows
 * whose values exceed 4 in magnitude, and its fp32 maximum and sum), or,
 * for many short row groups (at most 32 query rows per KV head, more
 * (sequence, KV head) units than CUs), the order in which the units are
 * dispatched (longest prefix first; B * Hkv int32). The plan depends only on
 * these arguments and the device's CU count, and results do not depend on
 * the dispatch order, so repeated calls are bitwise reproducible. May be 0;
 * its contents need no initialisation. Also 0 for shapes tv_attention
 * refuses (N > 128, max_prefix_len > 2^30). */
size_t tv_attention_workspace_bytes(tv_ctx *ctx, int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t max_prefix_len);

/* Tree-masked attention over a paged GQA KV cache ([EAGLE-2 page], third
 * pillar and the production note on paged tree masks).
 * For sequence b, present node i < n_b, query head h (KV head g = h / (Hq/Hkv)):
 *   keys  = prefix tokens t in [0, L_b) and tree tokens t = L_b + j for every
 *           present j whose bit is set in tree_mask[b][i] (all present j when
 *           tree_mask is NULL: the unmasked baseline);
 *   s_t   = sm_scale * <q, k_t>,  out = sum_t softmax(s)_t v_t.
 * Token t of sequence b lives in page page_table[b][t / 16], slot t % 16.
 *   q            bf16 [B][N][Hq][D]
 *   k_pages      bf16 [num_pages][Hkv][16][D]; v_pages likewise. The tree
 *                nodes' own K/V are already written at positions L_b..L_b+N-1.
 *   page_table   int32 [B][maxp]; entries past a sequence's last page unused
 *   prefix_lens  int32 [B], L_b in [0, max_prefix_len] (root excluded)
 *   max_prefix_len (host) bound used for planning; maxp * 16 >= max_prefix_len + N
 *   tree_mask    uint64 [B][N][W] as written by tv_build_mask, or NULL
 *   tree_sizes   int32 [B] or NULL: node counts; rows of absent nodes are not
 *                written and their keys are never read
 *   out          [B][N][Hq][D] in out_dtype (TV_F32 or TV_BF16)
 *   workspace    >= tv_attention_workspace_bytes(...) bytes (may be NULL if 0)
 * Requires D in {64, 128}, Hq % Hkv == 0, 0 <= N <= 128. Accumulates in fp32.
 * Returns TV_ERR_UNSUPPORTED when max_prefix_len > 2^30 or when the launch
 * would need more than 2^31 - 1 workgroups (B * Hkv * row groups * splits). */
tv_status tv_attention(tv_ctx *ctx, const void *q, const void *k_pages, const void *v_pages, int64_t num_pages,
                       const int32_t *page_table, int32_t maxp, const int32_t *prefix_lens, int32_t max_prefix_len,
                       const uint64_t *tree_mask, const int32_t *tree_sizes, int32_t B, int32_t N, int32_t Hq,
                       int32_t Hkv, int32_t D, float sm_scale, void *out, tv_dtype out_dtype, void *workspace,
                       size_t workspace_bytes);

/* tv_attention for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments (minus the workspace), checks, plan, kernels and results
 * as tv_attention; the plan's split partials or unit order go to a scratch
 * array that the library holds on each device it runs on, from set-up
 * (tv_create) until the process ends: TV_NOALLOC_SCRATCH_BYTES (64 MiB) per
 * device. Allocates nothing itself (no hipMalloc, hipFree or allocating
 * library call); the caller still passes q, the pools, the tables and out.
 * Returns TV_ERR_WORKSPACE, launching nothing, when the plan needs more
 * scratch than that (tv_attention_workspace_bytes(...) tells how much).
 * Every call on one device shares the array, which keeps the last call's
 * contents; nothing in it needs clearing. Calls that overlap on one device
 * (concurrent streams, or two contexts) race on the array: order them on
 * one stream. */
#define TV_NOALLOC_SCRATCH_BYTES (64ull << 20)
tv_status tv_attention_noalloc(tv_ctx *ctx, const void *q, const void *k_pages, const void *v_pages,
                               int64_t num_pages, const int32_t *page_table, int32_t maxp,
                               const int32_t *prefix_lens, int32_t max_prefix_len, const uint64_t *tree_mask,
                               const int32_t *tree_sizes, int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                               float sm_scale, void *out, tv_dtype out_dtype);

/* Workspace (bytes) tv_accept needs: per-row partial vocab reductions, and
 * in stochastic mode two residual rows of V doubles per sequence. */
size_t tv_accept_workspace_bytes(int32_t B, int32_t N, int32_t V, tv_accept_mode mode);

/* Acceptance and bonus token ([EAGLE-2 page], third pillar: longest
 * accepted path; [Sonar page], four stages: n drafts give up to n + 1 tokens,
 * the last from the target's logits after the accepted prefix; draft-target
 * section: acceptance compares the full distributions; [EAGLE-2 page]
 * benchmark discussion: rejection sampling keeps the output distribution).
 *   target_logits  fp32 [B][N][V]: row j = target's next-token logits after node j
 *   draft_logits   fp32 [B][N][V] (stochastic only, else NULL): row i >= 1 =
 *                  the draft distribution that produced node i's token
 *   draft_tokens   int32 [B][N]; [b][0] is the root's token (not verified)
 *   parents        int32 [B][N]; parents[b][0] must be -1
 *   tree_sizes     int32 [B] or NULL: node counts; absent nodes are never
 *                  read or accepted, their argmax rows are -1
 *   uniforms       fp32 [B][N] in [0, 1) (stochastic only, else NULL):
 *                  u[c-1] tests node c, u[N-1] drives the final draw
 *   temperature    > 0; logits are divided by it (stochastic only)
 *   accept_len     int32 [B]: root + accepted nodes = accepted drafts + 1
 *                  (counts the bonus token)
 *   path           int32 [B][N]: accepted node ids from the root, -1 padded
 *   bonus_token    int32 [B]
 *   target_argmax  int32 [B][N] or NULL (greedy only): per-row argmax
 * GREEDY: y_j = argmax of row j (fp32 compare, lowest index on ties, NaN
 *   below every number); node c matches iff draft_tokens[c] == y_parent(c);
 *   the longest root path of matching nodes wins, lexicographically smallest
 *   node sequence on ties; bonus = y at its last node.
 * STOCHASTIC (chains and trees): p_j = softmax(target row j / T), q_c =
 *   softmax(draft row c / T) in fp64, where draft row c is the distribution
 *   node c's token was drawn from (for siblings drawn without replacement,
 *   the row with the earlier siblings' tokens removed). The pages give no
 *   rule for several candidates; the single-candidate rule is applied to one
 *   candidate after another: from the root, with pi = p_node, the children c
 *   of the current node are tested in id order, c accepted iff
 *   u[c-1] < pi(t_c) / q_c(t_c); an accepted child becomes the current node
 *   (pi = p_c); a rejected one replaces pi by max(0, pi - q_c) normalised
 *   (unchanged if its mass is 0) before the next sibling. When no child is
 *   accepted, the next token is the inverse-CDF draw from pi (token order,
 *   theta = u[N-1] * total mass, smallest token whose running sum exceeds
 *   theta; the last token of positive mass if rounding finds none). On a
 *   chain this is: accept while u[i-1] < p_{i-1}(t_i) / q_i(t_i), then draw
 *   from max(0, p - q) at the rejection (p if its mass is 0), or from
 *   p_{N-1} when every draft is accepted.
 * Adds sum(accept_len) and B to the context's tau counters. Requires
 * 1 <= N <= 128 when B > 0, V >= 1, and B * N * ceil(V / C) <= 2^24 - 1
 * with C = 16384 in GREEDY mode and 8192 in STOCHASTIC mode (one 256-thread
 * workgroup per row and C-token chunk on a 1-D grid), and in STOCHASTIC mode
 * also B <= 2^23 - 1 (one 512-thread workgroup per sequence); larger calls
 * return TV_ERR_UNSUPPORTED.
 * In STOCHASTIC mode a small batch splits each sequence's vocabulary over
 * several workgroups that exchange partial sums and wait for each other
 * (bounded); the grid fits the device when nothing else runs on it. Two
 * such calls running at the same time on one device (two contexts on
 * different streams) can each hold part of the device; a workgroup that
 * waits past the bound marks its sequence -1 (accept_len, bonus, path) and
 * sets the sticky TV_ERR_HIP. Order concurrent stochastic calls on one
 * stream. */
tv_status tv_accept(tv_ctx *ctx, const float *target_logits, const float *draft_logits, const int32_t *draft_tokens,
                    const int32_t *parents, const int32_t *tree_sizes, const float *uniforms, int32_t B, int32_t N,
                    int32_t V,
                    tv_accept_mode mode, float temperature, int32_t *accept_len, int32_t *path, int32_t *bonus_token,
                    int32_t *target_argmax, void *workspace, size_t workspace_bytes);

/* Accepted-path KV commit and next-input insertion ([EAGLE-2 page], third
 * pillar: only the accepted path may stay in the target's KV cache;
 * [Sonar page], MTP schedule: the next target input is inserted by a kernel
 * after the input shift, so the host never waits for the accepted length).
 * For sequence b with L = prefix_lens[b] and n = accept_len[b]:
 *   - for m in [1, n) and every KV head, the K and V rows at position
 *     L + path[b][m] are moved to position L + m (all rows are read before
 *     any is written; rows with path[b][m] == m stay put; positions
 *     L+n..L+N-1 keep stale data, outside the new prefix);
 *   - new_prefix_lens[b] = L + n (root and accepted drafts are now prefix);
 *   - emitted[b] = draft_tokens[b][path[b][1..n-1]], then bonus_token[b],
 *     padded with -1 (the tokens this cycle produced);
 *   - next_root[b] = bonus_token[b] (node 0 of the next tree).
 *   k_pages, v_pages  bf16 [num_pages][Hkv][16][D], updated in place
 *   page_table, prefix_lens, max_prefix_len, maxp: as for tv_attention
 *   draft_tokens      int32 [B][N]
 *   path, accept_len, bonus_token: as written by tv_accept; path[b][0] = 0
 *                     and path[b][0..n) strictly increasing below N
 *                     (parents are not re-checked)
 *   new_prefix_lens, next_root  int32 [B]; emitted int32 [B][N] or NULL
 * The outputs must not overlap any input; pages holding positions
 * L..L+N-1 of one sequence must belong to that sequence alone (sequences are
 * committed concurrently). A sequence with L outside [0, max_prefix_len],
 * n outside [1, N], a bad path, a negative bonus or a page id outside
 * [0, num_pages) at a touched position is left unchanged (new length L,
 * next root -1, emitted -1) and sets the sticky TV_ERR_INVALID_ARG.
 * Requires D in {64, 128}, 1 <= N <= 128 when B > 0, maxp * 16 >=
 * max_prefix_len + N; max_prefix_len > 2^30 returns TV_ERR_UNSUPPORTED. */
tv_status tv_commit(tv_ctx *ctx, void *k_pages, void *v_pages, int64_t num_pages, const int32_t *page_table,
                    int32_t maxp, const int32_t *prefix_lens, int32_t max_prefix_len, const int32_t *draft_tokens,
                    const int32_t *path, const int32_t *accept_len, const int32_t *bonus_token, int32_t B, int32_t N,
                    int32_t Hkv, int32_t D, int32_t *new_prefix_lens, int32_t *emitted, int32_t *next_root);

/* tau = (sum of accept_len) / (number of sequences verified) since the last
 * reset ([EAGLE-3 page], tree acceptance rate); 0 when no cycle was counted.
 * tau and cycles are host pointers (cycles may be NULL). Synchronises. */
tv_status tv_tau(tv_ctx *ctx, double *tau, uint64_t *cycles);
tv_status tv_tau_reset(tv_ctx *ctx);

/* Reads and clears the sticky device error flag into *code (host). Synchronises. */
tv_status tv_device_error(tv_ctx *ctx, int32_t *code);

const char *tv_status_string(tv_status s);

/* Node budget of a draft tree for the current concurrency ([EAGLE-2 page],
 * production guideline on switching by batch size: past about 32 concurrent
 * requests verification becomes compute-bound, so the tree shrinks
 * 64 -> 32 -> 16, and past a batch of 64 speculation is switched off). Host
 * only; needs no context or GPU. The page gives the two thresholds and the
 * three sizes; the reading taken here:
 *   concurrency <= 32        max_nodes
 *   32 < concurrency <= 48   max_nodes / 2   (the page places the second
 *   48 < concurrency <= 64   max_nodes / 4    step nowhere; the midpoint)
 *   concurrency > 64         1 (the root alone: a plain decode step, which
 *                            the same calls run with N = 1)
 * never below 1. Returns -1 if concurrency < 0 or max_nodes is outside
 * [1, 128]. A caller passes the budget as N to tv_build_tree, or as the
 * tree_sizes entries of buffers laid out for max_nodes. */
int32_t tv_tree_budget(int32_t concurrency, int32_t max_nodes);

#ifdef __cplusplus
}
#endif
#endif
