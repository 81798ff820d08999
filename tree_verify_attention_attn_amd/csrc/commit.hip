// commit.hip - accepted-path KV commit and next-input insertion.
//
// After acceptance only the accepted path may stay in the target's KV cache
// (EAGLE-2 deep-dive page, third pillar: rejected drafts must not pollute the
// cache), and the next target input is produced on the device so the host
// never waits for the accepted length (Sonar page, MTP schedule: a kernel
// inserts the next token after the input shift instead of a CPU-GPU sync).
//
// Tree node j's K/V sits at position L+j. The accepted path v_0 = 0 < v_1 <
// ... < v_{n-1} is compacted to L..L+n-1: row L+m receives row L+v_m. Since
// v_m >= m, only the rows after the path's identity prefix (v_m == m) move.
//
// One workgroup per (sequence, KV head). Thread m checks path entry m and
// puts its source / destination row offsets in LDS; the workgroup loads
// every moved row into registers, waits for all of its loads, meets at a
// barrier, then stores.
// Reading everything first makes overlapping moves (a row that is both a
// source and a destination) safe. Workgroups touch disjoint rows: different
// KV heads, or different sequences (which own the pages of their tree
// positions).
#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kCommitThreads = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte chunk

template <int D>
__global__ void __launch_bounds__(kCommitThreads)
    commit_kernel(u32x4 *__restrict__ k_pages, u32x4 *__restrict__ v_pages, int64_t num_pages,
                  const int32_t *__restrict__ page_table, int maxp, const int32_t *__restrict__ prefix_lens,
                  int max_prefix_len, const int32_t *__restrict__ draft_tokens, const int32_t *__restrict__ path,
                  const int32_t *__restrict__ accept_len, const int32_t *__restrict__ bonus, int N, int Hkv,
                  int32_t *__restrict__ new_prefix_lens, int32_t *__restrict__ emitted, int32_t *__restrict__ next_root,
                  unsigned long long *state) {
  constexpr int CH = D / 8;                                       // 16-byte chunks per row
  constexpr int NPT = (127 * 2 * CH + kCommitThreads - 1) / kCommitThreads;  // chunks per thread, worst case
  __shared__ int s_v[128];                 // path entries
  __shared__ int64_t s_src[128], s_dst[128];  // their source and destination rows, in chunks
  const int b = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
  const int tid = threadIdx.x, m = tid;  // threads 0..127: path entry m

  const int L = prefix_lens[b];
  const int len = accept_len[b];
  const int bon = bonus[b];
  const bool bad0 = L < 0 || L > max_prefix_len || len < 1 || len > N || bon < 0;
  const bool live = !bad0 && m < len;
  const int v = live ? path[static_cast<int64_t>(b) * N + m] : 0;
  if (m < 128) s_v[m] = v;
  __syncthreads();
  const int prev = m >= 1 && m < 128 ? s_v[m - 1] : 0;
  // a valid path has v_m >= m, so no page-table index below L is formed
  bool lane_bad = live && (m == 0 ? v != 0 : (v <= prev || v < m || v >= N));
  if (live && !lane_bad) {
    const int ts = L + v, td = L + m;
    const int ps = page_table[static_cast<int64_t>(b) * maxp + ts / kPage];
    const int pd = page_table[static_cast<int64_t>(b) * maxp + td / kPage];
    lane_bad = ps < 0 || ps >= num_pages || pd < 0 || pd >= num_pages;
    s_src[m] = ((static_cast<int64_t>(ps) * Hkv + g) * kPage + ts % kPage) * CH;
    s_dst[m] = ((static_cast<int64_t>(pd) * Hkv + g) * kPage + td % kPage) * CH;
  }
  const bool bad = bad0 || __syncthreads_or(lane_bad);
  // the path starts with an identity run v_m == m; rows from m0 on move
  const int run = __syncthreads_count(live && v == m);
  const int m0 = bad ? len : run;
  const int total = bad ? 0 : (len - m0) * 2 * CH;

  if (total > 0) {
    // Every thread issues all NPT loads with no branch between them, so they
    // are in flight together; a thread past the end re-reads the last moved
    // chunk (in bounds, same cache line) and stores nothing.
    u32x4 r[NPT];
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int cc = min(tid + kCommitThreads * i, total - 1);
      r[i] = (((cc / CH) & 1) ? v_pages : k_pages)[s_src[m0 + cc / (2 * CH)] + cc % CH];
    }
    // every row of this (sequence, head) is read before any is written
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int c = tid + kCommitThreads * i;
      const int cc = min(c, total - 1);
      if (c < total) (((cc / CH) & 1) ? v_pages : k_pages)[s_dst[m0 + cc / (2 * CH)] + cc % CH] = r[i];
    }
  }

  if (g == 0 && m < N) {
    // emitted: the accepted drafts (path nodes 1..len-1), then the bonus
    if (emitted) {
      int tok = -1;
      if (!bad && m < len - 1) tok = draft_tokens[static_cast<int64_t>(b) * N + s_v[m + 1]];
      if (!bad && m == len - 1) tok = bon;
      emitted[static_cast<int64_t>(b) * N + m] = tok;
    }
    if (m == 0) {
      new_prefix_lens[b] = bad ? L : L + len;
      next_root[b] = bad ? -1 : bon;
      if (bad) raise_error(state, TV_ERR_INVALID_ARG);
    }
  }
}

}  // namespace

tv_status launch_commit(tv_ctx *ctx, void *k_pages, void *v_pages, int64_t num_pages, const int32_t *page_table,
                        int maxp, const int32_t *prefix_lens, int max_prefix_len, const int32_t *draft_tokens,
                        const int32_t *path, const int32_t *accept_len, const int32_t *bonus, int B, int N, int Hkv,
                        int D, int32_t *new_prefix_lens, int32_t *emitted, int32_t *next_root) {
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(B) * Hkv)), block(kCommitThreads);
  auto *k = static_cast<u32x4 *>(k_pages);
  auto *v = static_cast<u32x4 *>(v_pages);
  if (D == 128)
    hipLaunchKernelGGL(commit_kernel<128>, grid, block, 0, ctx->stream, k, v, num_pages, page_table, maxp,
                       prefix_lens, max_prefix_len, draft_tokens, path, accept_len, bonus, N, Hkv, new_prefix_lens,
                       emitted, next_root, ctx->d_state);
  else
    hipLaunchKernelGGL(commit_kernel<64>, grid, block, 0, ctx->stream, k, v, num_pages, page_table, maxp,
                       prefix_lens, max_prefix_len, draft_tokens, path, accept_len, bonus, N, Hkv, new_prefix_lens,
                       emitted, next_root, ctx->d_state);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

}  // namespace tv
