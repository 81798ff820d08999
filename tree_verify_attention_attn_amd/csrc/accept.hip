// accept.hip - acceptance of the draft tree and the bonus token.
//
// Greedy (EAGLE-2 deep-dive page, third pillar: compare the target's logits
// with the draft tokens and keep the longest accepted path; Sonar page, four
// stages: the logits after the accepted prefix give one more token):
//   pass 1  vocab-chunked argmax per (sequence, node) row. Each workgroup
//           reduces a 8192-entry chunk to one packed 64-bit key
//           (order-preserving float bits << 32 | ~index), so a plain max picks
//           the largest value and, among equal values, the lowest index.
//   pass 2  one wavefront per sequence, lane = node: merge the chunk keys,
//           rebuild ancestor masks by pointer doubling, and mark a node ok
//           when every node on its root path matches. The accepted path ends
//           at the deepest ok node; among equally deep ones the
//           lexicographically smallest root path is the one whose ancestor
//           mask has the larger bit-reversed value (node ids increase along a
//           path, so the first differing path element is the lowest
//           differing mask bit). Path, length, bonus and tau counters follow.
// Stochastic (Sonar page, draft-target section: acceptance compares the full
// draft and target distributions; EAGLE-2 page: rejection sampling keeps the
// target distribution), on chains and trees:
//   pass 1  per-chunk max and sum of exp (fp64) of logits / T, target and draft
//   pass 2  one workgroup per sequence: merge the chunk statistics and walk
//           from the root, testing the current node's children in id order
//           (u[c-1] < pi(t_c) / q_c(t_c)); an accepted child becomes the
//           current node with pi = its target row, a rejected one replaces pi
//           by the normalised residual max(0, pi - q_c) for the next sibling.
//           The next token is one inverse-CDF draw from the final pi (or the
//           last rejected sibling's residual) with theta = u[N-1] * mass.
//   Every exponential is fp64 (exp_fast, within a few ulp), so a decision
//   agrees with exact arithmetic whenever its margin exceeds ~1e-15.
#include <math.h>

#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kChunk = 8192;  // vocab entries per pass-1 workgroup
constexpr int kThreads = 256;

__device__ inline uint32_t orderable(float f) {
  if (isnan(f)) return 0u;  // NaN ranks below every number
  // -0 and +0 compare equal in fp32, so they must map to one key (the tie then
  // goes to the lower index)
  const uint32_t u = f == 0.0f ? 0u : __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline unsigned long long pack_key(float v, int x) {
  return (static_cast<unsigned long long>(orderable(v)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(x));
}

__device__ inline unsigned long long umax64(unsigned long long a, unsigned long long b) { return a > b ? a : b; }

template <bool kVec>
__global__ void __launch_bounds__(kThreads) argmax_chunk_kernel(const float *__restrict__ logits, int V, int chunks,
                                                                unsigned long long *__restrict__ keys) {
  __shared__ unsigned long long red[kThreads / 64];
  const int chunk = blockIdx.x;
  const int64_t row = blockIdx.y;
  const float *p = logits + row * V;
  const int x0 = chunk * kChunk;
  const int x1 = min(x0 + kChunk, V);
  unsigned long long best = 0ull;
  if (kVec) {
    // all of the thread's 16-byte loads are issued before any is used
    // (streaming loads: each logit is read once)
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    constexpr int kIt = kChunk / (kThreads * 4);
    f32x4 v[kIt];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int x = x0 + (it * kThreads + threadIdx.x) * 4;
      if (x < x1) v[it] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p + x));
    }
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int x = x0 + (it * kThreads + threadIdx.x) * 4;
      if (x < x1) {
        best = umax64(best, pack_key(v[it][0], x));
        best = umax64(best, pack_key(v[it][1], x + 1));
        best = umax64(best, pack_key(v[it][2], x + 2));
        best = umax64(best, pack_key(v[it][3], x + 3));
      }
    }
  } else {
    for (int x = x0 + threadIdx.x; x < x1; x += kThreads) best = umax64(best, pack_key(p[x], x));
  }
  for (int m = 32; m >= 1; m >>= 1) best = umax64(best, shfl_xor_u64(best, m));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kThreads / 64; ++i) best = umax64(best, red[i]);
    keys[row * chunks + chunk] = best;
  }
}

// One wavefront per sequence; lane = node.
__global__ void __launch_bounds__(256) greedy_path_kernel(const unsigned long long *__restrict__ keys, int chunks,
                                                          const int32_t *__restrict__ draft_tokens,
                                                          const int32_t *__restrict__ parents, int B, int N, int V,
                                                          int32_t *__restrict__ accept_len, int32_t *__restrict__ path,
                                                          int32_t *__restrict__ bonus,
                                                          int32_t *__restrict__ target_argmax,
                                                          unsigned long long *state) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= B) return;
  const bool live = lane < N;
  const int64_t idx = static_cast<int64_t>(b) * N + lane;
  int y = 0;
  if (live) {
    unsigned long long best = 0ull;
    for (int c = 0; c < chunks; ++c) best = umax64(best, keys[idx * chunks + c]);
    y = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best & 0xFFFFFFFFull));
  }
  const int par = live ? parents[idx] : -1;
  const int tok = live ? draft_tokens[idx] : 0;
  const bool bad_tree = live && (par < -1 || par >= lane || (lane == 0 && par != -1));
  const bool bad_tok = live && lane > 0 && (tok < 0 || tok >= V);
  const bool tree_err = __ballot(bad_tree) != 0;
  const bool tok_err = __ballot(bad_tok) != 0;
  if (tree_err || tok_err) {
    if (lane == 0) raise_error(state, tree_err ? TV_ERR_INVALID_TREE : TV_ERR_INVALID_ARG);
    if (live) {
      path[idx] = -1;
      if (target_argmax) target_argmax[idx] = y;
    }
    if (lane == 0) {
      accept_len[b] = -1;
      bonus[b] = -1;
    }
    return;
  }
  // ancestor-or-self masks by pointer doubling (parents precede children)
  unsigned long long anc = live ? (1ull << lane) : 0ull;
  int jump = live ? par : -1;
#pragma unroll
  for (int r = 0; r < 6; ++r) {
    const int src = jump >= 0 ? jump : lane;
    const unsigned long long a_src = shfl_u64(anc, src);
    const int j_src = __shfl(jump, src);
    if (jump >= 0) {
      anc |= a_src;
      jump = j_src;
    }
  }
  // node c >= 1 matches iff its token is the target's argmax at its parent
  const int y_par = __shfl(y, par >= 0 ? par : 0);
  const bool match = live && (lane == 0 || (par >= 0 && tok == y_par));
  const unsigned long long match_bits = __ballot(match);
  const bool ok = live && (anc & 1ull) && ((anc & ~match_bits) == 0ull);
  // deepest ok node; ties -> lexicographically smallest root path
  int depth = ok ? __popcll(anc) : 0;
  int dmax = depth;
  for (int m = 32; m >= 1; m >>= 1) dmax = max(dmax, __shfl_xor(dmax, m));
  unsigned long long key = (ok && depth == dmax) ? __brevll(anc) : 0ull;
  for (int m = 32; m >= 1; m >>= 1) key = umax64(key, shfl_xor_u64(key, m));
  const unsigned long long chosen = __brevll(key);  // the chosen path's node set; always holds node 0
  const int len = __popcll(chosen);
  const int last = 63 - __clzll(static_cast<long long>(chosen));
  const int y_last = __shfl(y, last);
  if (live) {
    // lane p writes the p-th node of the path (the p-th set bit of `chosen`)
    int node = -1;
    if (lane < len) {
      unsigned long long rest = chosen;
      for (int q = 0; q < lane; ++q) rest &= rest - 1ull;
      node = __ffsll(static_cast<long long>(rest)) - 1;
    }
    path[idx] = node;
    if (target_argmax) target_argmax[idx] = y;
  }
  if (lane == 0) {
    accept_len[b] = len;
    bonus[b] = y_last;
    atomicAdd(state + 0, static_cast<unsigned long long>(len));
    atomicAdd(state + 1, 1ull);
  }
}

// ---------------------------------------------------------------- stochastic

// e^x in fp64 for the arguments the acceptance step forms (a scaled logit
// minus a row maximum, so x <= 0). Cody-Waite reduction x = k ln2 + r with
// |r| <= ln2 / 2, ln2 split into a head with 32 significant bits (so k * head
// is exact for every k that occurs) and a tail; e^r from its Taylor series
// to degree 13 (truncation below 2e-18 relative); scaling by 2^k. The result
// is within a few ulp of e^x. Arguments below -745.2, -inf included, give 0.
constexpr double kLog2eD = 1.4426950408889634;
constexpr double kLn2Hi = 0.6931471803691238;
constexpr double kLn2Lo = 1.9082149292705877e-10;

__device__ inline double exp_fast(double x) {
  if (!(x > -745.2)) return 0.0;
  const double k = rint(x * kLog2eD);
  double r = fma(-k, kLn2Hi, x);
  r = fma(-k, kLn2Lo, r);
  double p = 1.6059043836821613e-10;  // 1/13!
  p = fma(p, r, 2.08767569878681e-09);
  p = fma(p, r, 2.505210838544172e-08);
  p = fma(p, r, 2.755731922398589e-07);
  p = fma(p, r, 2.7557319223985893e-06);
  p = fma(p, r, 2.48015873015873e-05);
  p = fma(p, r, 0.0001984126984126984);
  p = fma(p, r, 0.001388888888888889);
  p = fma(p, r, 0.008333333333333333);
  p = fma(p, r, 0.041666666666666664);
  p = fma(p, r, 0.16666666666666666);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  return ldexp(p, static_cast<int>(k));
}

// x / T in fp64 from a precomputed 1/T and one FMA correction step (exact
// when T = 1)
__device__ inline double div_t(double x, double T, double invT) {
  const double q = x * invT;
  return fma(fma(-q, T, x), invT, q);
}

template <bool kVec>
__global__ void __launch_bounds__(kThreads) softmax_chunk_kernel(const float *__restrict__ target,
                                                                 const float *__restrict__ draft, int N, int V,
                                                                 int chunks, double T, double invT,
                                                                 double *__restrict__ stats) {
  __shared__ double red[kThreads / 64];
  const int chunk = blockIdx.x;
  const int64_t row = blockIdx.y;  // b * N + j
  const int which = blockIdx.z;    // 0 = target, 1 = draft
  const int j = static_cast<int>(row % N);
  double *out = stats + ((row * 2 + which) * chunks + chunk) * 2;
  if (which == 1 && j == 0) {  // draft row 0 is never used
    if (threadIdx.x == 0) {
      out[0] = 0.0;
      out[1] = 0.0;
    }
    return;
  }
  const float *p = (which ? draft : target) + row * V;
  const int x0 = chunk * kChunk;
  const int x1 = min(x0 + kChunk, V);
  constexpr int kPer = kChunk / kThreads;  // 32 values per thread, kept in registers
  double z[kPer];
  if (kVec) {
#pragma unroll
    for (int it = 0; it < kPer / 4; ++it) {
      const int x = x0 + (it * kThreads + threadIdx.x) * 4;
      float4 v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (x < x1) v = *reinterpret_cast<const float4 *>(p + x);
      z[it * 4 + 0] = div_t(v.x, T, invT);
      z[it * 4 + 1] = div_t(v.y, T, invT);
      z[it * 4 + 2] = div_t(v.z, T, invT);
      z[it * 4 + 3] = div_t(v.w, T, invT);
    }
  } else {
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
      const int x = x0 + it * kThreads + threadIdx.x;
      z[it] = x < x1 ? div_t(p[x], T, invT) : -INFINITY;
    }
  }
  double mx = -INFINITY;
#pragma unroll
  for (int it = 0; it < kPer; ++it) mx = fmax(mx, z[it]);
  for (int m = 32; m >= 1; m >>= 1) mx = fmax(mx, __shfl_xor(mx, m));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = red[0];
  for (int i = 1; i < kThreads / 64; ++i) mx = fmax(mx, red[i]);
  __syncthreads();
  double zs = 0.0;
#pragma unroll
  for (int it = 0; it < kPer; ++it) zs += exp_fast(z[it] - mx);  // -inf (padding) gives 0
  for (int m = 32; m >= 1; m >>= 1) zs += __shfl_xor(zs, m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = zs;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int i = 0; i < kThreads / 64; ++i) tot += red[i];
    out[0] = mx;
    out[1] = tot;
  }
}

struct RowStat {
  double m, Z, invZ;
};

__device__ inline RowStat merge_stats(const double *stats, int64_t row, int which, int chunks) {
  const double *s = stats + (row * 2 + which) * chunks * 2;
  double M = -INFINITY;
  for (int c = 0; c < chunks; ++c) M = fmax(M, s[2 * c]);
  double Z = 0.0;
  for (int c = 0; c < chunks; ++c) {
    if (s[2 * c + 1] > 0.0) Z += s[2 * c + 1] * exp_fast(s[2 * c] - M);
  }
  return RowStat{M, Z, 1.0 / Z};
}

__device__ inline double prob_at(const float *row, int x, double T, double invT, const RowStat &st) {
  return exp_fast(div_t(row[x], T, invT) - st.m) * st.invZ;
}

constexpr int kPathThreads = 512;
constexpr int kBlk = 16;  // tokens per register block of a row sweep

// The target distribution pi the walk holds: the current node's target row
// (w == nullptr, invM = 1), or a stored residual w[0..V) of mass 1 / invM.
struct Pi {
  const double *w;
  double invM;
};

// One workgroup per sequence, for chains and trees alike. Wavefront 0
// validates the tree, computes for every node c its first test's p(t_c)
// (under its parent's target row) and q_c(t_c), and the children of every
// node as a bit mask. Every thread then runs the same walk from the LDS
// copies: the current node's children are tested in id order; a rejection
// followed by another sibling stores the residual max(0, pi - q_c) of the
// whole row in one of two per-sequence buffers (a sweep by all threads, its
// mass summed in a fixed order), and the next sibling is tested against it.
// The final draw - from the last rejected sibling's residual (built on the
// fly), or from pi itself - sweeps the row once in contiguous token-order
// segments (16-token register blocks, next block's loads issued before the
// current block's exponentials), scans the segment sums in a fixed order,
// and re-sweeps only the segment whose running sum passes theta, one token
// per lane of one wavefront.
template <bool kVec>
__global__ void __launch_bounds__(kPathThreads) stochastic_path_kernel(
    const float *__restrict__ target, const float *__restrict__ draft, const int32_t *__restrict__ draft_tokens,
    const int32_t *__restrict__ parents, const float *__restrict__ uniforms, int B, int N, int V, int chunks,
    double T, double invT, const double *__restrict__ stats, double *__restrict__ wbuf,
    int32_t *__restrict__ accept_len, int32_t *__restrict__ path, int32_t *__restrict__ bonus,
    unsigned long long *state) {
  __shared__ int s_err, s_pick, s_lastpos, s_cross, s_cross_last;
  __shared__ double s_wave[kPathThreads / 64], s_wpre[kPathThreads / 64], s_total, s_cprefix;
  __shared__ double s_pa[64], s_qa[64], s_u[64];
  __shared__ int s_tok[64], s_path[64];
  __shared__ unsigned long long s_child[64];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t base = static_cast<int64_t>(b) * N;
  if (wid == 0) {
    // validation with the same precedence as a serial check: a bad parent
    // anywhere, then a draft token outside [0, V)
    bool tree_bad = false, tok_bad = false;
    int p = -1, t = 0;
    if (lane < N) {
      p = parents[base + lane];
      tree_bad = p < -1 || p >= lane || (lane == 0 && p != -1);
      if (lane >= 1) {
        t = draft_tokens[base + lane];
        tok_bad = t < 0 || t >= V;
      }
      s_u[lane] = static_cast<double>(uniforms[base + lane]);
    }
    const int err = __builtin_amdgcn_ballot_w64(tree_bad) ? TV_ERR_INVALID_TREE
                    : __builtin_amdgcn_ballot_w64(tok_bad) ? TV_ERR_INVALID_ARG
                                                           : 0;
    if (!err && lane >= 1 && lane < N) {
      s_tok[lane] = t;
      if (p >= 0) {  // a node without a parent (forest) is never tested
        const RowStat sp = merge_stats(stats, base + p, 0, chunks);
        const RowStat sq = merge_stats(stats, base + lane, 1, chunks);
        s_pa[lane] = prob_at(target + (base + p) * V, t, T, invT, sp);
        s_qa[lane] = prob_at(draft + (base + lane) * V, t, T, invT, sq);
      }
    }
    for (int n = 0; n < N; ++n) {
      const uint64_t kids = __builtin_amdgcn_ballot_w64(!err && lane >= 1 && lane < N && p == n);
      if (lane == 0) s_child[n] = kids;
    }
    if (lane == 0) {
      s_err = err;
      s_pick = 0x7FFFFFFF;
      s_lastpos = -1;
      s_cross = 0x7FFFFFFF;
      s_path[0] = 0;
    }
  }
  __syncthreads();
  if (s_err) {
    if (tid == 0) {
      raise_error(state, s_err);
      accept_len[b] = -1;
      bonus[b] = -1;
    }
    for (int i = tid; i < N; i += kPathThreads) path[base + i] = -1;
    return;
  }
  // contiguous segment per thread in token order, a multiple of 4 tokens
  const int seg = ((V + 4 * kPathThreads - 1) / (4 * kPathThreads)) * 4;
  const int x0 = min(tid * seg, V), x1 = min(x0 + seg, V);
  double *const buf0 = wbuf + static_cast<int64_t>(b) * 2 * V;
  double *const buf1 = buf0 + V;

  auto load_block = [&](const float *row, int xb, float (&v)[kBlk]) __attribute__((always_inline)) {
    if (kVec) {  // V % 4 == 0 and xb % 4 == 0: a float4 is either all in [x0, x1) or all out
#pragma unroll
      for (int i = 0; i < kBlk / 4; ++i) {
        const int x = xb + 4 * i;
        float4 f = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        if (x < x1) f = *reinterpret_cast<const float4 *>(row + x);
        v[4 * i] = f.x;
        v[4 * i + 1] = f.y;
        v[4 * i + 2] = f.z;
        v[4 * i + 3] = f.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kBlk; ++i) v[i] = xb + i < x1 ? row[xb + i] : -INFINITY;
    }
  };
  auto load_wblock = [&](const double *w, int xb, double (&v)[kBlk]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kBlk; ++i) v[i] = xb + i < x1 ? w[xb + i] : 0.0;
  };
  // weight of one token: pi's weight (the target row's probability, or the
  // stored residual's entry), or, with a sibling's draft row, the residual
  // max(0, pi - q) with pi normalised
  auto weight = [&](const RowStat &sp, const Pi &pi, bool with_q, const RowStat &sq, float pl, double wl,
                    float ql) __attribute__((always_inline)) {
    const double w = pi.w ? wl : exp_fast(div_t(pl, T, invT) - sp.m) * sp.invZ;  // padding (-inf) gives 0
    if (!with_q) return w;
    return fmax(0.0, w * pi.invM - exp_fast(div_t(ql, T, invT) - sq.m) * sq.invZ);
  };
  // one sweep of this thread's segment; optionally stores every weight
  auto sweep = [&](const float *P, const RowStat &sp, const Pi &pi, const float *Q, const RowStat &sq, double *dst,
                   double &local, int &lastpos) __attribute__((always_inline)) {
    local = 0.0;
    lastpos = -1;
    float pv[kBlk], qv[kBlk], pn[kBlk], qn[kBlk];
    double wv[kBlk], wn[kBlk];
    if (pi.w)
      load_wblock(pi.w, x0, wv);
    else
      load_block(P, x0, pv);
    if (Q) load_block(Q, x0, qv);
    for (int xb = x0; xb < x1; xb += kBlk) {
      if (xb + kBlk < x1) {
        if (pi.w)
          load_wblock(pi.w, xb + kBlk, wn);
        else
          load_block(P, xb + kBlk, pn);
        if (Q) load_block(Q, xb + kBlk, qn);
      }
#pragma unroll
      for (int i = 0; i < kBlk; ++i) {
        const double w = weight(sp, pi, Q != nullptr, sq, pv[i], wv[i], qv[i]);
        local += w;
        if (w > 0.0) lastpos = xb + i;
        if (dst && xb + i < x1) dst[xb + i] = w;
      }
#pragma unroll
      for (int i = 0; i < kBlk; ++i) {
        pv[i] = pn[i];
        qv[i] = qn[i];
        wv[i] = wn[i];
      }
    }
  };
  // exclusive prefix of the segment sums and their total: a fixed-order
  // scan within each wavefront, then over the wavefront totals in order
  auto scan = [&](double local, double &prefix, double &total) __attribute__((always_inline)) {
    double incl = local;
    for (int d = 1; d < 64; d <<= 1) {
      const double t = __shfl_up(incl, d);
      if (lane >= d) incl += t;
    }
    double excl = __shfl_up(incl, 1);
    if (lane == 0) excl = 0.0;
    if (lane == 63) s_wave[wid] = incl;
    __syncthreads();
    if (tid == 0) {
      double run = 0.0;
      for (int i = 0; i < kPathThreads / 64; ++i) {
        s_wpre[i] = run;
        run += s_wave[i];
      }
      s_total = run;
    }
    __syncthreads();
    prefix = s_wpre[wid] + excl;
    total = s_total;
    __syncthreads();
  };

  // the walk; every thread takes the same decisions from the same data
  Pi pi{nullptr, 1.0};
  int node = 0, k = 0, pend = -1;
  for (;;) {
    const float *P = target + (base + node) * V;
    const RowStat sp = merge_stats(stats, base + node, 0, chunks);
    uint64_t kids = s_child[node];
    int acc = -1;
    while (kids) {
      const int c = __builtin_ctzll(kids);
      kids &= kids - 1;
      const double a = pi.w ? (pi.w[s_tok[c]] * pi.invM) / s_qa[c] : s_pa[c] / s_qa[c];
      if (s_u[c - 1] < a) {
        acc = c;
        break;
      }
      if (!kids) {  // the last sibling: its residual is built on the fly by the final draw
        pend = c;
        break;
      }
      double *dst = pi.w == buf0 ? buf1 : buf0;
      const RowStat sq = merge_stats(stats, base + c, 1, chunks);
      double local, prefix, total;
      int lastpos;
      sweep(P, sp, pi, draft + (base + c) * V, sq, dst, local, lastpos);
      scan(local, prefix, total);
      if (total > 0.0) pi = Pi{dst, 1.0 / total};  // a residual of mass 0 leaves pi unchanged
    }
    if (acc < 0) break;
    node = acc;
    ++k;
    if (tid == 0) s_path[k] = acc;
    pi = Pi{nullptr, 1.0};
  }

  // the final draw
  const float *P = target + (base + node) * V;
  const float *Q = pend >= 0 ? draft + (base + pend) * V : nullptr;
  const RowStat sp = merge_stats(stats, base + node, 0, chunks);
  const RowStat sq = Q ? merge_stats(stats, base + pend, 1, chunks) : RowStat{0.0, 1.0, 1.0};
  const double u = s_u[N - 1];
  for (int pass = 0; pass < 2; ++pass) {
    const float *Qp = pass == 0 ? Q : nullptr;
    double local, prefix, total;
    int lastpos;
    sweep(P, sp, pi, Qp, sq, nullptr, local, lastpos);
    scan(local, prefix, total);
    if (Qp && !(total > 0.0)) continue;  // no residual mass: draw from pi instead
    const double theta = u * total;
    // the first segment whose running sum passes theta holds the draw
    if (prefix + local > theta) atomicMin(&s_cross, tid);
    if (lastpos >= 0) atomicMax(&s_lastpos, lastpos);
    __syncthreads();
    if (tid == s_cross) {
      s_cprefix = prefix;
      s_cross_last = lastpos;
    }
    __syncthreads();
    // wavefront 0 re-sweeps the crossing segment one token per lane: a
    // fixed-order scan of the weights gives each token's running sum
    const int cross = s_cross;
    if (wid == 0 && cross != 0x7FFFFFFF) {
      const int cx0 = min(cross * seg, V), cx1 = min(cx0 + seg, V);
      double carry = s_cprefix;
      int pick = -1;
      for (int xb = cx0; xb < cx1 && pick < 0; xb += 64) {
        const int x = xb + lane;
        double w = 0.0;
        if (x < cx1)
          w = weight(sp, pi, Qp != nullptr, sq, pi.w ? 0.f : P[x], pi.w ? pi.w[x] : 0.0, Qp ? Qp[x] : 0.f);
        double run = w;
        for (int d = 1; d < 64; d <<= 1) {
          const double t = __shfl_up(run, d);
          if (lane >= d) run += t;
        }
        const uint64_t hit = __builtin_amdgcn_ballot_w64(x < cx1 && carry + run > theta);
        if (hit) pick = xb + __builtin_ctzll(hit);
        carry += __shfl(run, 63);
      }
      const int pk = pick >= 0 ? pick : s_cross_last;  // rounding left no crossing: last positive token
      if (lane == 0 && pk >= 0) s_pick = pk;
    }
    __syncthreads();
    break;
  }
  if (tid == 0) {
    const int pick = s_pick != 0x7FFFFFFF ? s_pick : s_lastpos;
    accept_len[b] = k + 1;
    bonus[b] = pick;
    atomicAdd(state + 0, static_cast<unsigned long long>(k + 1));
    atomicAdd(state + 1, 1ull);
  }
  for (int i = tid; i < N; i += kPathThreads) path[base + i] = i <= k ? s_path[i] : -1;
}

}  // namespace

// stochastic: the chunk statistics, then (256-byte aligned) two residual
// buffers of V doubles per sequence
size_t stats_doubles(int B, int N, int V) {
  const int chunks = (V + kChunk - 1) / kChunk;
  return ((static_cast<size_t>(B) * N * 2 * chunks * 2 + 31) / 32) * 32;
}

size_t accept_ws_bytes(int B, int N, int V, tv_accept_mode mode) {
  const int chunks = (V + kChunk - 1) / kChunk;
  const size_t rows = static_cast<size_t>(B) * N;
  if (mode == TV_GREEDY) return rows * chunks * sizeof(unsigned long long);
  return (stats_doubles(B, N, V) + static_cast<size_t>(B) * 2 * V) * sizeof(double);
}

tv_status launch_accept(tv_ctx *ctx, const float *target_logits, const float *draft_logits,
                        const int32_t *draft_tokens, const int32_t *parents, const float *uniforms, int B, int N,
                        int V, tv_accept_mode mode, float temperature, int32_t *accept_len, int32_t *path,
                        int32_t *bonus, int32_t *target_argmax, void *workspace) {
  const int chunks = (V + kChunk - 1) / kChunk;
  const dim3 blk(kThreads);
  const bool vec = (V % 4) == 0 && (reinterpret_cast<uintptr_t>(target_logits) & 15) == 0 &&
                   (draft_logits == nullptr || (reinterpret_cast<uintptr_t>(draft_logits) & 15) == 0);
  if (mode == TV_GREEDY) {
    auto *keys = static_cast<unsigned long long *>(workspace);
    const dim3 g1(chunks, B * N);
    if (vec)
      hipLaunchKernelGGL(argmax_chunk_kernel<true>, g1, blk, 0, ctx->stream, target_logits, V, chunks, keys);
    else
      hipLaunchKernelGGL(argmax_chunk_kernel<false>, g1, blk, 0, ctx->stream, target_logits, V, chunks, keys);
    if (hipGetLastError() != hipSuccess) return TV_ERR_HIP;
    hipLaunchKernelGGL(greedy_path_kernel, dim3((B + 3) / 4), dim3(256), 0, ctx->stream, keys, chunks, draft_tokens,
                       parents, B, N, V, accept_len, path, bonus, target_argmax, ctx->d_state);
    return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
  }
  auto *stats = static_cast<double *>(workspace);
  double *wbuf = stats + stats_doubles(B, N, V);
  const double T = static_cast<double>(temperature), invT = 1.0 / T;
  const dim3 g1(chunks, B * N, 2);
  if (vec)
    hipLaunchKernelGGL(softmax_chunk_kernel<true>, g1, blk, 0, ctx->stream, target_logits, draft_logits, N, V,
                       chunks, T, invT, stats);
  else
    hipLaunchKernelGGL(softmax_chunk_kernel<false>, g1, blk, 0, ctx->stream, target_logits, draft_logits, N, V,
                       chunks, T, invT, stats);
  if (hipGetLastError() != hipSuccess) return TV_ERR_HIP;
  if (vec)
    hipLaunchKernelGGL(stochastic_path_kernel<true>, dim3(B), dim3(kPathThreads), 0, ctx->stream, target_logits,
                       draft_logits, draft_tokens, parents, uniforms, B, N, V, chunks, T, invT, stats, wbuf,
                       accept_len, path, bonus, ctx->d_state);
  else
    hipLaunchKernelGGL(stochastic_path_kernel<false>, dim3(B), dim3(kPathThreads), 0, ctx->stream, target_logits,
                       draft_logits, draft_tokens, parents, uniforms, B, N, V, chunks, T, invT, stats, wbuf,
                       accept_len, path, bonus, ctx->d_state);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

}  // namespace tv
