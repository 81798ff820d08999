/*
 * oracle.c - TEST INFRASTRUCTURE ONLY: the plain fp64 CPU oracle.
 *
 * Only tests/, the smoke check and the bench's cpu_baseline leg may load this
 * file's library. It is written for a reader checking it against the pages by
 * eye: straight loops, fp64 arithmetic, no blocking or fusion. Work is split
 * over threads only across independent rows, which changes no result.
 *
 * Sources (titles of the pages this follows):
 *  [EAGLE-2 page] "EAGLE-2 심층 아키텍처 ..." (techknowgenie) - the three
 *     pillars (tree mask injected into the attention kernel, longest accepted
 *     path), the dynamic-tree section, the reference code's tree-mask loop,
 *     and the production note on indexing tree masks over paged memory.
 *  [Sonar page] "Accelerating Sonar through speculation" (Perplexity) - the
 *     four stages of speculative sampling (longest acceptable prefix, bonus
 *     token from the logits at the mismatch or the end), draft-target
 *     acceptance by comparing full distributions.
 *  [EAGLE-3 page] "論文解説: EAGLE-3 ..." - definition of tau.
 * Readings where the pages are silent (scale, GQA grouping, root handling,
 * tie-breaks, the rejection-sampling formula) are stated at each function.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------------ */
/* small helpers                                                            */
/* ------------------------------------------------------------------------ */

static double bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static int resolve_threads(int nthreads) {
  if (nthreads > 0) return nthreads;
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

typedef void (*range_fn)(void *ctx, int64_t lo, int64_t hi);

typedef struct {
  range_fn fn;
  void *ctx;
  int64_t lo, hi;
} range_job;

static void *range_worker(void *p) {
  range_job *j = (range_job *)p;
  j->fn(j->ctx, j->lo, j->hi);
  return NULL;
}

/* Runs fn over [0, n) split into contiguous chunks, one per thread. */
static void parallel_for(int64_t n, int nthreads, range_fn fn, void *ctx) {
  int T = resolve_threads(nthreads);
  if (T > n) T = (int)(n > 0 ? n : 1);
  if (T <= 1) {
    fn(ctx, 0, n);
    return;
  }
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * T);
  range_job *jobs = (range_job *)malloc(sizeof(range_job) * T);
  for (int t = 0; t < T; ++t) {
    jobs[t].fn = fn;
    jobs[t].ctx = ctx;
    jobs[t].lo = n * t / T;
    jobs[t].hi = n * (t + 1) / T;
    pthread_create(&th[t], NULL, range_worker, &jobs[t]);
  }
  for (int t = 0; t < T; ++t) pthread_join(th[t], NULL);
  free(th);
  free(jobs);
}

/* Tree rule shared by every call: parent[b][i] in {-1} U [0, i) (node ids are
 * assigned in creation order on the EAGLE-2 page, so a parent always precedes
 * its child); with need_root, parent[b][0] must be -1. */
/* Node count of sequence b: tree_sizes[b] when given, else N. */
static int32_t nodes_of(const int32_t *tree_sizes, int64_t b, int32_t N) { return tree_sizes ? tree_sizes[b] : N; }

static int check_sizes(const int32_t *tree_sizes, int32_t B, int32_t N) {
  for (int64_t b = 0; tree_sizes && b < B; ++b)
    if (tree_sizes[b] < 1 || tree_sizes[b] > N) return TVO_ERR_INVALID_ARG;
  return TVO_OK;
}

/* parents of the present nodes: -1 or an earlier node (need_root: node 0 has
 * no parent) */
static int check_tree_sized(const int32_t *parents, const int32_t *tree_sizes, int32_t B, int32_t N,
                            int need_root) {
  for (int64_t b = 0; b < B; ++b)
    for (int32_t i = 0; i < nodes_of(tree_sizes, b, N); ++i) {
      int32_t p = parents[b * N + i];
      if (p < -1 || p >= i) return TVO_ERR_INVALID_TREE;
      if (need_root && i == 0 && p != -1) return TVO_ERR_INVALID_TREE;
    }
  return TVO_OK;
}

static int check_tree(const int32_t *parents, int32_t B, int32_t N, int need_root) {
  for (int64_t b = 0; b < B; ++b)
    for (int32_t i = 0; i < N; ++i) {
      int32_t p = parents[b * N + i];
      if (p < -1 || p >= i) return TVO_ERR_INVALID_TREE;
      if (need_root && i == 0 && p != -1) return TVO_ERR_INVALID_TREE;
    }
  return TVO_OK;
}

/* ------------------------------------------------------------------------ */
/* O1: ancestor-or-self mask ([EAGLE-2 page], reference code, tree-mask loop:
 * start at the node itself, mark it, move to its parent, stop past the root) */
/* ------------------------------------------------------------------------ */

int tvo_build_mask(const int32_t *parents, const int32_t *tree_sizes, int32_t B, int32_t N, uint64_t *mask,
                   int32_t *depth) {
  if (B < 0 || N < 0) return TVO_ERR_INVALID_ARG;
  if (N > 128) return TVO_ERR_UNSUPPORTED;
  if ((int64_t)B * N == 0) return TVO_OK;
  if (!parents || !mask) return TVO_ERR_INVALID_ARG;
  int st = check_sizes(tree_sizes, B, N);
  if (st != TVO_OK) return st;
  st = check_tree_sized(parents, tree_sizes, B, N, 0);
  if (st != TVO_OK) return st;
  const int32_t W = (N + 63) / 64;
  for (int64_t b = 0; b < B; ++b) {
    const int32_t n = nodes_of(tree_sizes, b, N);
    for (int32_t i = 0; i < N; ++i) {
      uint64_t *row = mask + ((int64_t)b * N + i) * W;
      for (int32_t w = 0; w < W; ++w) row[w] = 0;
      int32_t d = -1;
      int32_t c = i < n ? i : -1; /* an absent node: empty row, depth -1 */
      while (c != -1) {
        row[c / 64] |= (uint64_t)1 << (c % 64);
        d += 1;
        c = parents[b * N + c];
      }
      if (depth) depth[b * N + i] = d;
    }
  }
  return TVO_OK;
}

/* ------------------------------------------------------------------------ */
/* O2: tree-masked attention over the paged KV cache                        */
/*                                                                          */
/* [EAGLE-2 page], third pillar: every tree node is verified in one target  */
/* forward, seeing only its causal (ancestor) relations through a 2D tree   */
/* mask; production note: the mask is indexed directly over paged memory.   */
/* Readings where the pages are silent:                                     */
/*  - score s_t = sm_scale * <q, k_t>, softmax over the visible keys, output */
/*    sum_t w_t v_t (standard scaled dot-product attention);                */
/*  - GQA: query head h reads KV head h / (Hq/Hkv) (contiguous groups);     */
/*  - the prefix (L_b cached tokens) is visible to every node; tree node j  */
/*    sits at token position L_b + j and is visible to node i iff bit j of */
/*    mask[b][i] is set; node 0 is the root (last verified token, counted   */
/*    in the tree as in the page's code), so prefix_lens exclude it;        */
/*  - token t lives in page page_table[b][t/16] at slot t%16, KV layout     */
/*    [page][kv_head][slot][d].                                             */
/* ------------------------------------------------------------------------ */

typedef struct {
  const uint16_t *q, *kp, *vp;
  int64_t num_pages;
  const int32_t *page_table;
  int32_t maxp;
  const int32_t *prefix_lens;
  const uint64_t *mask;
  const int32_t *tree_sizes;
  int32_t B, N, Hq, Hkv, D;
  double scale;
  const int32_t *rows;
  double *out;
  int32_t max_keys;
} attn_ctx;

static const uint16_t *kv_row(const attn_ctx *a, const uint16_t *base, int64_t b, int32_t g, int64_t t) {
  int64_t page = a->page_table[b * a->maxp + t / 16];
  int64_t slot = t % 16;
  return base + ((page * a->Hkv + g) * 16 + slot) * a->D;
}

static void attn_rows(void *vctx, int64_t lo, int64_t hi) {
  const attn_ctx *a = (const attn_ctx *)vctx;
  int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (a->max_keys > 0 ? a->max_keys : 1));
  double *s = (double *)malloc(sizeof(double) * (a->max_keys > 0 ? a->max_keys : 1));
  double *qd = (double *)malloc(sizeof(double) * a->D);
  const int32_t W = (a->N + 63) / 64;
  const int32_t G = a->Hq / a->Hkv;
  for (int64_t r = lo; r < hi; ++r) {
    int64_t b, i, h;
    if (a->rows) {
      b = a->rows[3 * r];
      i = a->rows[3 * r + 1];
      h = a->rows[3 * r + 2];
    } else {
      b = r / ((int64_t)a->N * a->Hq);
      i = (r / a->Hq) % a->N;
      h = r % a->Hq;
    }
    const int32_t g = (int32_t)(h / G);
    const int64_t L = a->prefix_lens[b];
    const uint16_t *qr = a->q + ((b * a->N + i) * a->Hq + h) * a->D;
    for (int32_t d = 0; d < a->D; ++d) qd[d] = bf16_to_double(qr[d]);

    const int32_t n = nodes_of(a->tree_sizes, b, a->N);
    double *o = a->out + r * a->D;
    if (i >= n) { /* an absent node has no output */
      for (int32_t d = 0; d < a->D; ++d) o[d] = NAN;
      continue;
    }
    /* visible key positions: the whole prefix, then the present tree nodes on the mask */
    int64_t nk = 0;
    for (int64_t t = 0; t < L; ++t) keys[nk++] = t;
    for (int32_t j = 0; j < n; ++j) {
      int visible = 1;
      if (a->mask) visible = (int)((a->mask[(b * a->N + i) * W + j / 64] >> (j % 64)) & 1u);
      if (visible) keys[nk++] = L + j;
    }

    double m = -INFINITY;
    for (int64_t n = 0; n < nk; ++n) {
      const uint16_t *kr = kv_row(a, a->kp, b, g, keys[n]);
      double dot = 0.0;
      for (int32_t d = 0; d < a->D; ++d) dot += qd[d] * bf16_to_double(kr[d]);
      s[n] = a->scale * dot;
      if (s[n] > m) m = s[n];
    }
    double Z = 0.0;
    for (int64_t n = 0; n < nk; ++n) {
      s[n] = exp(s[n] - m);
      Z += s[n];
    }
    for (int32_t d = 0; d < a->D; ++d) o[d] = 0.0;
    for (int64_t n = 0; n < nk; ++n) {
      const uint16_t *vr = kv_row(a, a->vp, b, g, keys[n]);
      const double w = s[n] / Z;
      for (int32_t d = 0; d < a->D; ++d) o[d] += w * bf16_to_double(vr[d]);
    }
    if (nk == 0)
      for (int32_t d = 0; d < a->D; ++d) o[d] = NAN;
  }
  free(keys);
  free(s);
  free(qd);
}

int tvo_attention(const uint16_t *q, const uint16_t *k_pages, const uint16_t *v_pages, int64_t num_pages,
                  const int32_t *page_table, int32_t maxp, const int32_t *prefix_lens, int32_t max_prefix_len,
                  const uint64_t *tree_mask, const int32_t *tree_sizes, int32_t B, int32_t N, int32_t Hq,
                  int32_t Hkv, int32_t D, float sm_scale, const int32_t *rows, int64_t n_rows, double *out,
                  int nthreads) {
  /* argument rules (same as the library's) */
  if (B < 0 || N < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || num_pages < 0 || maxp < 0 || max_prefix_len < 0)
    return TVO_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return TVO_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return TVO_ERR_UNSUPPORTED;
  if (N > 128) return TVO_ERR_UNSUPPORTED;
  if (!isfinite(sm_scale)) return TVO_ERR_INVALID_ARG;
  if ((int64_t)B * N == 0) return TVO_OK;
  if ((int64_t)maxp * 16 < (int64_t)max_prefix_len + N) return TVO_ERR_INVALID_ARG;
  if (!q || !k_pages || !v_pages || !page_table || !prefix_lens || !out) return TVO_ERR_INVALID_ARG;
  /* data rules: node counts within [1, N], prefix lengths within
   * [0, max_prefix_len], every page the sequence touches inside [0, num_pages) */
  if (check_sizes(tree_sizes, B, N) != TVO_OK) return TVO_ERR_INVALID_ARG;
  for (int64_t b = 0; b < B; ++b) {
    int32_t L = prefix_lens[b];
    if (L < 0 || L > max_prefix_len) return TVO_ERR_INVALID_ARG;
    int64_t np = ((int64_t)L + nodes_of(tree_sizes, b, N) + 15) / 16;
    for (int64_t p = 0; p < np; ++p) {
      int32_t id = page_table[b * maxp + p];
      if (id < 0 || id >= num_pages) return TVO_ERR_INVALID_ARG;
    }
  }
  if (!rows) n_rows = (int64_t)B * N * Hq;
  for (int64_t r = 0; rows && r < n_rows; ++r)
    if (rows[3 * r] < 0 || rows[3 * r] >= B || rows[3 * r + 1] < 0 || rows[3 * r + 1] >= N || rows[3 * r + 2] < 0 ||
        rows[3 * r + 2] >= Hq)
      return TVO_ERR_INVALID_ARG;

  attn_ctx a;
  a.q = q;
  a.kp = k_pages;
  a.vp = v_pages;
  a.num_pages = num_pages;
  a.page_table = page_table;
  a.maxp = maxp;
  a.prefix_lens = prefix_lens;
  a.mask = tree_mask;
  a.tree_sizes = tree_sizes;
  a.B = B;
  a.N = N;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.scale = (double)sm_scale;
  a.rows = rows;
  a.out = out;
  a.max_keys = max_prefix_len + N;
  parallel_for(n_rows, nthreads, attn_rows, &a);
  return TVO_OK;
}

/* ------------------------------------------------------------------------ */
/* O3: greedy acceptance                                                    */
/*                                                                          */
/* [EAGLE-2 page]: the draft proposes tokens by argmax, and the verifier     */
/* compares the target's logits with the draft tokens and keeps the longest */
/* accepted path. [Sonar page], four stages: the longest acceptable prefix  */
/* is kept and the logits at the mismatch (or after the last accepted token)*/
/* give one more token, so n drafts yield up to n + 1 tokens.               */
/* Readings:                                                                */
/*  - y_j = argmax_x logits[b][j][x] in fp32, lowest x on ties, NaN below   */
/*    every number;                                                         */
/*  - node c >= 1 matches iff draft_tokens[b][c] == y_{parent[c]};          */
/*  - result: the longest root path of matching nodes, lexicographically    */
/*    smallest node sequence on ties; accept_len = path nodes (root + k     */
/*    accepted) = k + 1, so it counts the bonus token y_{last};             */
/*  - path[b] = [0, v_1, .., v_k, -1 ...].                                  */
/* ------------------------------------------------------------------------ */

/* NaN-aware "greater than": a NaN never wins, and anything beats a NaN. */
static int f32_greater(float a, float b) {
  if (isnan(a)) return 0;
  if (isnan(b)) return 1;
  return a > b;
}

typedef struct {
  const float *logits;
  int64_t V;
  int32_t *y;
} argmax_ctx;

static void argmax_rows(void *vctx, int64_t lo, int64_t hi) {
  const argmax_ctx *a = (const argmax_ctx *)vctx;
  for (int64_t r = lo; r < hi; ++r) {
    const float *row = a->logits + r * a->V;
    int64_t best = 0;
    for (int64_t x = 1; x < a->V; ++x)
      if (f32_greater(row[x], row[best])) best = x;
    a->y[r] = (int32_t)best;
  }
}

static int check_tokens(const int32_t *tok, const int32_t *tree_sizes, int32_t B, int32_t N, int32_t V) {
  for (int64_t b = 0; b < B; ++b)
    for (int32_t i = 1; i < nodes_of(tree_sizes, b, N); ++i)
      if (tok[b * N + i] < 0 || tok[b * N + i] >= V) return TVO_ERR_INVALID_ARG;
  return TVO_OK;
}

int tvo_accept_greedy(const float *target_logits, const int32_t *draft_tokens, const int32_t *parents,
                      const int32_t *tree_sizes, int32_t B, int32_t N, int32_t V, int32_t *accept_len, int32_t *path,
                      int32_t *bonus, int32_t *target_argmax, int nthreads) {
  if (B < 0 || V <= 0) return TVO_ERR_INVALID_ARG;
  if (B == 0) return TVO_OK;
  if (N < 1) return TVO_ERR_INVALID_ARG;
  if (N > 128) return TVO_ERR_UNSUPPORTED;
  if (!target_logits || !draft_tokens || !parents || !accept_len || !path || !bonus) return TVO_ERR_INVALID_ARG;
  int st = check_sizes(tree_sizes, B, N);
  if (st != TVO_OK) return st;
  st = check_tree_sized(parents, tree_sizes, B, N, 1);
  if (st != TVO_OK) return st;
  st = check_tokens(draft_tokens, tree_sizes, B, N, V);
  if (st != TVO_OK) return st;

  int32_t *y = (int32_t *)malloc(sizeof(int32_t) * (size_t)B * N);
  argmax_ctx ac = {target_logits, V, y};
  parallel_for((int64_t)B * N, nthreads, argmax_rows, &ac);

  int32_t best[128], next[128];
  for (int64_t b = 0; b < B; ++b) {
    const int32_t n = nodes_of(tree_sizes, b, N);
    const int32_t *par = parents + b * N;
    const int32_t *tok = draft_tokens + b * N;
    int32_t *yb = y + b * N;
    for (int32_t i = n; i < N; ++i) yb[i] = -1; /* absent nodes have no row */
    /* bottom-up: best[i] = most matching nodes on a path below i,
     * next[i] = the lowest child reaching it */
    for (int32_t i = n - 1; i >= 0; --i) {
      best[i] = 0;
      next[i] = -1;
      for (int32_t c = i + 1; c < n; ++c) {
        if (par[c] != i) continue;
        if (tok[c] != yb[i]) continue;
        if (1 + best[c] > best[i]) {
          best[i] = 1 + best[c];
          next[i] = c;
        }
      }
    }
    int32_t *pb = path + b * N;
    for (int32_t i = 0; i < N; ++i) pb[i] = -1;
    int32_t v = 0, k = 0;
    pb[0] = 0;
    while (next[v] >= 0) {
      v = next[v];
      pb[++k] = v;
    }
    accept_len[b] = k + 1;
    bonus[b] = yb[v];
    if (target_argmax)
      for (int32_t i = 0; i < N; ++i) target_argmax[b * N + i] = yb[i];
  }
  free(y);
  return TVO_OK;
}

/* ------------------------------------------------------------------------ */
/* O4: stochastic acceptance on a chain or a tree                           */
/*                                                                          */
/* [Sonar page], draft-target section: acceptance compares the full draft   */
/* and target distributions, and the target always adds one token after the */
/* accepted drafts. [EAGLE-2 page], benchmark discussion: verification is   */
/* rejection sampling, so the output follows the target's distribution      */
/* exactly (lossless). The pages cite Leviathan et al. and Chen et al. (and */
/* SpecInfer for trees) but print no formula; the plainest reading is their */
/* standard rule, applied to one candidate after another:                   */
/*  - p_j = softmax(target row j / T), q_c = softmax(draft row c / T), fp64;*/
/*    draft row c is the distribution node c's token was drawn from;        */
/*  - the walk starts at the root with pi = p_0; the children c of the      */
/*    current node are tested in increasing id order: c is accepted iff     */
/*    u[c-1] < pi(t_c) / q_c(t_c) (a ratio >= 1 always accepts, u < 1);     */
/*  - an accepted child becomes the current node, with pi = p_c;            */
/*  - a rejected child replaces pi by the residual max(0, pi - q_c),        */
/*    normalised, before the next sibling is tested (a residual of mass 0   */
/*    leaves pi unchanged);                                                 */
/*  - when no child of the current node is accepted (or it has none), the   */
/*    next token is drawn from pi by inverse CDF in token order with        */
/*    theta = u[N-1] * (sum of pi's unnormalised weights): the smallest x   */
/*    whose running sum exceeds theta, or the last x with positive weight  */
/*    if rounding leaves none.                                              */
/* On a chain this is the single-candidate rule: accept node i iff          */
/* u[i-1] < p_{i-1}(t_i) / q_i(t_i), and at the first rejection draw from   */
/* max(0, p_{i-1} - q_i) (from p_{i-1} if that is 0), or from p_{N-1} when  */
/* every draft is accepted.                                                 */
/* ------------------------------------------------------------------------ */

typedef struct {
  const float *logits;
  int64_t V;
  double T; /* temperature; z = logit / T */
  double *m, *Z;
} softmax_ctx;

static void softmax_stats(void *vctx, int64_t lo, int64_t hi) {
  const softmax_ctx *a = (const softmax_ctx *)vctx;
  for (int64_t r = lo; r < hi; ++r) {
    const float *row = a->logits + r * a->V;
    double m = -INFINITY;
    for (int64_t x = 0; x < a->V; ++x) {
      double z = (double)row[x] / a->T;
      if (z > m) m = z;
    }
    double Z = 0.0;
    for (int64_t x = 0; x < a->V; ++x) Z += exp((double)row[x] / a->T - m);
    a->m[r] = m;
    a->Z[r] = Z;
  }
}

static double prob(const float *row, int64_t x, double T, double m, double Z) {
  return exp((double)row[x] / T - m) / Z;
}

/* Inverse-CDF draw from weights w(x) (given by the callback) with theta = u * W. */
typedef double (*weight_fn)(const void *ctx, int64_t x);

static int32_t inverse_cdf(weight_fn w, const void *ctx, int64_t V, double u, double *margin_out) {
  double W = 0.0;
  for (int64_t x = 0; x < V; ++x) W += w(ctx, x);
  double theta = u * W;
  double cum = 0.0;
  int32_t pick = -1, last_pos = -1;
  double margin = INFINITY;
  for (int64_t x = 0; x < V; ++x) {
    double wx = w(ctx, x);
    cum += wx;
    if (wx > 0.0) last_pos = (int32_t)x;
    double dist = fabs(cum - theta);
    if (dist < margin) margin = dist;
    if (pick < 0 && cum > theta) pick = (int32_t)x;
  }
  if (pick < 0) pick = last_pos;
  if (margin_out) *margin_out = W > 0.0 ? margin / W : 0.0;
  return pick;
}

typedef struct {
  const float *prow, *qrow;
  double T, mp, Zp, mq, Zq;
} resid_ctx;

static double array_w(const void *vc, int64_t x) { return ((const double *)vc)[x]; }

static double target_w(const void *vc, int64_t x) {
  const resid_ctx *c = (const resid_ctx *)vc;
  return prob(c->prow, x, c->T, c->mp, c->Zp);
}

int tvo_accept_stochastic(const float *target_logits, const float *draft_logits, const int32_t *draft_tokens,
                          const int32_t *parents, const int32_t *tree_sizes, const float *uniforms, int32_t B,
                          int32_t N, int32_t V,
                          float temperature, int32_t *accept_len, int32_t *path, int32_t *bonus, double *margins,
                          int nthreads) {
  if (B < 0 || V <= 0) return TVO_ERR_INVALID_ARG;
  if (!(temperature > 0.0f) || !isfinite(temperature)) return TVO_ERR_INVALID_ARG;
  if (B == 0) return TVO_OK;
  if (N < 1) return TVO_ERR_INVALID_ARG;
  if (N > 128) return TVO_ERR_UNSUPPORTED;
  if (!target_logits || !draft_logits || !draft_tokens || !parents || !uniforms || !accept_len || !path || !bonus)
    return TVO_ERR_INVALID_ARG;
  int st = check_sizes(tree_sizes, B, N);
  if (st != TVO_OK) return st;
  st = check_tree_sized(parents, tree_sizes, B, N, 1);
  if (st != TVO_OK) return st;
  st = check_tokens(draft_tokens, tree_sizes, B, N, V);
  if (st != TVO_OK) return st;

  const double T = (double)temperature;
  const int64_t R = (int64_t)B * N;
  double *mp = (double *)malloc(sizeof(double) * R), *Zp = (double *)malloc(sizeof(double) * R);
  double *mq = (double *)malloc(sizeof(double) * R), *Zq = (double *)malloc(sizeof(double) * R);
  double *wbuf = (double *)malloc(sizeof(double) * 2 * (size_t)V);
  if (!mp || !Zp || !mq || !Zq || !wbuf) {
    free(mp), free(Zp), free(mq), free(Zq), free(wbuf);
    return TVO_ERR_RUNTIME;
  }
  softmax_ctx sp = {target_logits, V, T, mp, Zp};
  softmax_ctx sq = {draft_logits, V, T, mq, Zq};
  parallel_for(R, nthreads, softmax_stats, &sp);
  parallel_for(R, nthreads, softmax_stats, &sq);

  for (int64_t b = 0; b < B; ++b) {
    const int32_t n = nodes_of(tree_sizes, b, N);
    const int32_t *tok = draft_tokens + b * N;
    const int32_t *par = parents + b * N;
    const float *u = uniforms + b * N;
    double *mg = margins ? margins + b * N : NULL;
    if (mg)
      for (int32_t i = 0; i < N; ++i) mg[i] = INFINITY;
    int32_t *pb = path + b * N;
    for (int32_t i = 0; i < N; ++i) pb[i] = -1;
    pb[0] = 0;
    int32_t k = 0, node = 0;
    /* the distribution the next test and the final draw use: p_node while
     * cur is NULL, else the stored residual cur (unnormalised, mass M) */
    double *cur = NULL, M = 1.0;
    for (;;) {
      const int64_t rp = b * N + node;
      const float *prow = target_logits + rp * V;
      int32_t accepted = -1;
      for (int32_t c = node + 1; c < n; ++c) {
        if (par[c] != node) continue; /* children in increasing id order */
        const int64_t rq = b * N + c;
        const float *qrow = draft_logits + rq * V;
        const double qv = prob(qrow, tok[c], T, mq[rq], Zq[rq]);
        const double pv = cur ? cur[tok[c]] / M : prob(prow, tok[c], T, mp[rp], Zp[rp]);
        const double a = pv / qv;
        if (mg) mg[c - 1] = fabs((double)u[c - 1] - a);
        if ((double)u[c - 1] < a) {
          accepted = c;
          break;
        }
        /* rejected: the next sibling is tested against, and the final draw
         * taken from, the residual max(0, pi - q_c) of the current pi */
        double *nw = cur == wbuf ? wbuf + V : wbuf;
        double Rsum = 0.0;
        for (int64_t x = 0; x < V; ++x) {
          const double d = (cur ? cur[x] / M : prob(prow, x, T, mp[rp], Zp[rp])) - prob(qrow, x, T, mq[rq], Zq[rq]);
          nw[x] = d > 0.0 ? d : 0.0;
          Rsum += nw[x];
        }
        if (Rsum > 0.0) { /* a residual of mass 0 leaves pi unchanged */
          cur = nw;
          M = Rsum;
        }
      }
      if (accepted < 0) break;
      pb[++k] = accepted;
      node = accepted;
      cur = NULL;
      M = 1.0;
    }
    double smargin = INFINITY;
    int32_t pick;
    if (cur) {
      pick = inverse_cdf(array_w, cur, V, (double)u[N - 1], &smargin);
    } else {
      const int64_t rp = b * N + node;
      resid_ctx c = {target_logits + rp * V, NULL, T, mp[rp], Zp[rp], 0.0, 1.0};
      pick = inverse_cdf(target_w, &c, V, (double)u[N - 1], &smargin);
    }
    if (mg) mg[N - 1] = smargin;
    accept_len[b] = k + 1;
    bonus[b] = pick;
  }
  free(wbuf);
  free(mp);
  free(Zp);
  free(mq);
  free(Zq);
  return TVO_OK;
}

/* ------------------------------------------------------------------------ */
/* O5: tau ([EAGLE-3 page], tree acceptance rate): mean accepted tokens per */
/* verification cycle; a cycle is one sequence in one accept call.          */
/* ------------------------------------------------------------------------ */

double tvo_tau(const int32_t *accept_len, int64_t M) {
  if (M <= 0) return 0.0;
  int64_t sum = 0;
  for (int64_t j = 0; j < M; ++j) sum += accept_len[j];
  return (double)sum / (double)M;
}

/* ------------------------------------------------------------------------ */
/* Accepted-path KV commit and next-input insertion.                        */
/*                                                                          */
/* [EAGLE-2 page], third pillar: rejected drafts must not pollute the       */
/* target's KV cache. [Sonar page], MTP schedule: after acceptance the      */
/* target's input is shifted and the next token is inserted on the device, */
/* avoiding a CPU-GPU sync on the accepted length. Readings:                */
/*  - committed position L+m (m = 0..len-1) receives the K/V that node v_m  */
/*    of the accepted path (v_0 = 0 < v_1 < ...) holds at L+v_m, for every  */
/*    KV head; everything is read before anything is written;              */
/*  - the new prefix length is L + len (the root and the accepted drafts);  */
/*  - emitted tokens: draft_tokens[v_1..v_{len-1}], then the bonus, -1 pad; */
/*  - the next root token (the next tree's node 0) is the bonus.            */
/* A sequence whose prefix length, path, bonus or touched pages are invalid */
/* is left unchanged (new length L, next root -1, emitted all -1) and the   */
/* call reports TVO_ERR_INVALID_ARG.                                        */
/* ------------------------------------------------------------------------ */

int tvo_commit(uint16_t *k_pages, uint16_t *v_pages, int64_t num_pages, const int32_t *page_table, int32_t maxp,
               const int32_t *prefix_lens, int32_t max_prefix_len, const int32_t *draft_tokens,
               const int32_t *path, const int32_t *accept_len, const int32_t *bonus, int32_t B, int32_t N,
               int32_t Hkv, int32_t D, int32_t *new_prefix_lens, int32_t *emitted, int32_t *next_root) {
  if (B < 0 || N < 1 || N > 128 || Hkv <= 0 || (D != 64 && D != 128) || maxp < 0 || max_prefix_len < 0 ||
      num_pages < 0)
    return TVO_ERR_INVALID_ARG;
  if (B == 0) return TVO_OK;
  if (!k_pages || !v_pages || !page_table || !prefix_lens || !draft_tokens || !path || !accept_len || !bonus ||
      !new_prefix_lens || !next_root)
    return TVO_ERR_INVALID_ARG;
  int status = TVO_OK;
  uint16_t *tmp = (uint16_t *)malloc(sizeof(uint16_t) * 2 * (size_t)N * (size_t)D);
  if (!tmp) return TVO_ERR_RUNTIME;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t L = prefix_lens[b];
    const int32_t len = accept_len[b];
    const int32_t *pth = path + (int64_t)b * N;
    int ok = L >= 0 && L <= max_prefix_len && (int64_t)L + N <= (int64_t)maxp * 16 && len >= 1 && len <= N &&
             pth[0] == 0 && bonus[b] >= 0;
    for (int32_t m = 1; ok && m < len; ++m) ok = pth[m] > pth[m - 1] && pth[m] < N;
    /* every page the moves touch must exist */
    for (int32_t m = 0; ok && m < len; ++m) {
      const int64_t ts[2] = {(int64_t)L + pth[m], (int64_t)L + m};
      for (int u = 0; u < 2; ++u) {
        const int32_t pid = page_table[(int64_t)b * maxp + ts[u] / 16];
        if (pid < 0 || pid >= num_pages) ok = 0;
      }
    }
    if (!ok) {
      status = TVO_ERR_INVALID_ARG;
      new_prefix_lens[b] = L;
      next_root[b] = -1;
      if (emitted)
        for (int32_t m = 0; m < N; ++m) emitted[(int64_t)b * N + m] = -1;
      continue;
    }
    for (int32_t g = 0; g < Hkv; ++g) {
      /* gather the accepted rows first, then write them to their new places */
      for (int32_t m = 1; m < len; ++m) {
        const int64_t t = (int64_t)L + pth[m];
        const int64_t row = (((int64_t)page_table[(int64_t)b * maxp + t / 16] * Hkv + g) * 16 + t % 16) * D;
        memcpy(tmp + (2 * (size_t)m) * D, k_pages + row, sizeof(uint16_t) * D);
        memcpy(tmp + (2 * (size_t)m + 1) * D, v_pages + row, sizeof(uint16_t) * D);
      }
      for (int32_t m = 1; m < len; ++m) {
        const int64_t t = (int64_t)L + m;
        const int64_t row = (((int64_t)page_table[(int64_t)b * maxp + t / 16] * Hkv + g) * 16 + t % 16) * D;
        memcpy(k_pages + row, tmp + (2 * (size_t)m) * D, sizeof(uint16_t) * D);
        memcpy(v_pages + row, tmp + (2 * (size_t)m + 1) * D, sizeof(uint16_t) * D);
      }
    }
    new_prefix_lens[b] = L + len;
    next_root[b] = bonus[b];
    if (emitted) {
      for (int32_t m = 0; m < N; ++m) emitted[(int64_t)b * N + m] = -1;
      for (int32_t m = 1; m < len; ++m) emitted[(int64_t)b * N + m - 1] = draft_tokens[(int64_t)b * N + pth[m]];
      emitted[(int64_t)b * N + len - 1] = bonus[b];
    }
  }
  free(tmp);
  return status;
}

/* ------------------------------------------------------------------------ */
/* Dynamic draft-tree construction ([EAGLE-2 page], the dynamic-tree        */
/* algorithm section and its reference code's tree builder).                */
/*                                                                          */
/* A node's cumulative score is the product of the draft probabilities on   */
/* its root path (root = 1). The candidate queue starts with the root's     */
/* top-k_root proposals; repeatedly the candidate with the highest score is */
/* made the next node (ids in creation order; ties go to the candidate      */
/* queued first); a node shallower than max_depth then proposes its top-k   */
/* children, and a child is queued only if its cumulative score is above    */
/* the threshold (the reference code's strict test; the prose says "at or  */
/* above"). Construction stops at N nodes (root included) or when the      */
/* queue is empty. Proposal row i of a sequence is what the draft head      */
/* proposes for the node created i-th (row 0: the root); scores are fp64    */
/* products of the fp32 probabilities. Unused slots of a short tree are     */
/* padding: parent -1, the root's token, depth 0, mask = the slot itself,   */
/* score 0. A probability that is NaN or negative makes that sequence all   */
/* padding with n_nodes = 0 and the call return TVO_ERR_INVALID_ARG.        */
/* ------------------------------------------------------------------------ */

int tvo_build_tree(const int32_t *root_tokens, const int32_t *cand_tokens, const float *cand_probs, int32_t B,
                   int32_t N, int32_t k, int32_t k_root, float threshold, int32_t max_depth, int32_t *parents,
                   int32_t *tokens, int32_t *depth, uint64_t *mask, double *scores, int32_t *n_nodes) {
  if (B < 0 || N < 1 || N > 128 || k < 1 || k > 32 || k_root < 1 || k_root > k || max_depth < 1 ||
      !(threshold == threshold))
    return TVO_ERR_INVALID_ARG;
  if (B == 0) return TVO_OK;
  if (!root_tokens || !cand_tokens || !cand_probs || !parents || !tokens) return TVO_ERR_INVALID_ARG;
  const int64_t cap = (int64_t)k_root + (int64_t)(N - 1) * k;
  double *qs = (double *)malloc(sizeof(double) * cap);
  int32_t *qp = (int32_t *)malloc(sizeof(int32_t) * cap), *qt = (int32_t *)malloc(sizeof(int32_t) * cap);
  char *alive = (char *)malloc(cap);
  if (!qs || !qp || !qt || !alive) {
    free(qs), free(qp), free(qt), free(alive);
    return TVO_ERR_RUNTIME;
  }
  int status = TVO_OK;
  for (int64_t b = 0; b < B; ++b) {
    const int32_t *ct = cand_tokens + b * N * k;
    const float *cp = cand_probs + b * N * k;
    int32_t *pa = parents + b * N, *tk = tokens + b * N;
    double sc[128];
    int32_t dp[128];
    int bad = 0;
    for (int64_t j = 0; j < (int64_t)N * k; ++j)
      if (!(cp[j] >= 0.0f)) bad = 1; /* NaN or negative */
    int32_t n = 0;
    if (!bad) {
      int64_t q = 0;
      pa[0] = -1, tk[0] = root_tokens[b], dp[0] = 0, sc[0] = 1.0, n = 1;
      for (int32_t s = 0; s < k_root; ++s) { /* the root's proposals are queued unconditionally */
        qs[q] = sc[0] * (double)cp[s], qp[q] = 0, qt[q] = ct[s], alive[q] = 1, ++q;
      }
      while (n < N) {
        int64_t best = -1;
        for (int64_t j = 0; j < q; ++j) /* strict '>' keeps the earliest queued among equal scores */
          if (alive[j] && (best < 0 || qs[j] > qs[best])) best = j;
        if (best < 0) break;
        alive[best] = 0;
        const int32_t id = n++;
        pa[id] = qp[best], tk[id] = qt[best], dp[id] = dp[qp[best]] + 1, sc[id] = qs[best];
        if (dp[id] < max_depth)
          for (int32_t s = 0; s < k; ++s) {
            const double c = sc[id] * (double)cp[(int64_t)id * k + s];
            if (c > (double)threshold) qs[q] = c, qp[q] = id, qt[q] = ct[(int64_t)id * k + s], alive[q] = 1, ++q;
          }
      }
    } else {
      status = TVO_ERR_INVALID_ARG;
    }
    for (int32_t i = n; i < N; ++i) pa[i] = -1, tk[i] = root_tokens[b], dp[i] = 0, sc[i] = 0.0;
    for (int32_t i = 0; i < N; ++i) {
      if (depth) depth[b * N + i] = dp[i];
      if (scores) scores[b * N + i] = sc[i];
      if (mask) { /* the node and every ancestor, W = ceil(N / 64) words per row */
        const int32_t W = (N + 63) / 64;
        uint64_t *row = mask + (b * N + i) * W;
        for (int32_t w = 0; w < W; ++w) row[w] = 0;
        for (int32_t c = i; c >= 0; c = pa[c]) row[c / 64] |= 1ull << (c % 64);
      }
    }
    if (n_nodes) n_nodes[b] = n;
  }
  free(qs), free(qp), free(qt), free(alive);
  return status;
}
