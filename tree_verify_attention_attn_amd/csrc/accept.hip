// accept.hip - acceptance of the draft tree and the bonus token.
//
// Greedy (EAGLE-2 deep-dive page, third pillar: compare the target's logits
// with the draft tokens and keep the longest accepted path; Sonar page, four
// stages: the logits after the accepted prefix give one more token):
//   pass 1  vocab-chunked argmax per (sequence, node) row. Each workgroup
//           reduces a 16384-entry chunk to one packed 64-bit key
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
//           When pass 1 has at most kMaxFusedGrid workgroups, both passes
//           are one launch: the workgroup of pass 1 that completes a
//           sequence's last chunk key runs pass 2 for that sequence.
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
//   Every exponential is fp64 (exp_tab, within a few ulp), so a decision
//   agrees with exact arithmetic whenever its margin exceeds ~1e-15.
#include <math.h>

#include <type_traits>

#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kChunk = 8192;  // vocab entries per stochastic pass-1 workgroup
constexpr int kGChunk = 16384;  // vocab entries per greedy argmax workgroup
constexpr int kMaxFusedGrid = 256;  // pass-1 workgroups up to which both greedy passes are one launch
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

__device__ inline int size_of(const int32_t *sizes, int64_t b, int N) { return sizes ? sizes[b] : N; }

// Node count of sequence b. A count outside [1, N] is bad data: every row of
// the sequence is then reduced, and the path logic reports the error.
__device__ inline int present_nodes(const int32_t *sizes, int64_t b, int N) {
  const int nb = sizes ? sizes[b] : N;
  return (nb < 1 || nb > N) ? N : nb;
}

// Argmax key of p[x0, x1) over the workgroup; thread 0 receives it.
template <bool kVec>
__device__ inline unsigned long long block_argmax(const float *p, int x0, int x1, unsigned long long *red) {
  unsigned long long best = 0ull;
  if (kVec) {
    // all of the thread's 16-byte loads are issued before any is used
    // (streaming loads: each logit is read once)
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    constexpr int kIt = kGChunk / (kThreads * 4);
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
  if (threadIdx.x == 0)
    for (int i = 1; i < kThreads / 64; ++i) best = umax64(best, red[i]);
  return best;
}

// Workgroup (row, chunk) = (blockIdx.x / chunks, blockIdx.x % chunks).
template <bool kVec>
__global__ void __launch_bounds__(kThreads) argmax_chunk_kernel(const float *__restrict__ logits,
                                                                const int32_t *__restrict__ sizes, int N, int V,
                                                                int chunks, unsigned long long *__restrict__ keys) {
  __shared__ unsigned long long red[kThreads / 64];
  const int chunk = static_cast<int>(blockIdx.x % static_cast<unsigned>(chunks));
  const int64_t row = blockIdx.x / static_cast<unsigned>(chunks);
  if (row % N >= present_nodes(sizes, row / N, N)) return;  // an absent node: its row is never read
  const int x0 = chunk * kGChunk;
  const unsigned long long best = block_argmax<kVec>(logits + row * V, x0, min(x0 + kGChunk, V), red);
  if (threadIdx.x == 0) keys[row * chunks + chunk] = best;
}

// One wavefront per sequence; lane i holds node i (and node i + 64 when
// H = 2). Ancestor sets are 128-bit (nodes 0..63 in word 0, 64..127 in word 1).
// kCoherent: the keys were published by other workgroups of the same launch
// (device-scope atomic swaps), so they are read with device-scope atomics.
template <int H, bool kCoherent>
__device__ void greedy_path_seq(int b, int lane, unsigned long long *keys, int chunks,
                                const int32_t *__restrict__ draft_tokens, const int32_t *__restrict__ parents,
                                const int32_t *__restrict__ sizes, int N, int V, int32_t *__restrict__ accept_len,
                                int32_t *__restrict__ path, int32_t *__restrict__ bonus,
                                int32_t *__restrict__ target_argmax, unsigned long long *state) {
  const int nb = size_of(sizes, b, N);
  const bool bad_size = nb < 1 || nb > N;
  bool live[H], bad_tree = false, bad_tok = false;
  int y[H], par[H], tok[H];
#pragma unroll
  for (int k = 0; k < H; ++k) {
    const int i = lane + 64 * k;
    const int64_t idx = static_cast<int64_t>(b) * N + i;
    live[k] = !bad_size && i < nb;
    y[k] = -1;
    if (live[k]) {
      // the row's chunk keys, 16 loads in flight at a time
      unsigned long long best = 0ull;
      unsigned long long *kp = keys + idx * chunks;
      for (int c0 = 0; c0 < chunks; c0 += 16) {
        unsigned long long kv[16];
#pragma unroll
        for (int q = 0; q < 16; ++q)
          kv[q] = c0 + q >= chunks ? 0ull : kCoherent ? atomicAdd(kp + c0 + q, 0ull) : kp[c0 + q];
#pragma unroll
        for (int q = 0; q < 16; ++q) best = umax64(best, kv[q]);
      }
      y[k] = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best & 0xFFFFFFFFull));
    }
    par[k] = live[k] ? parents[idx] : -1;
    tok[k] = live[k] ? draft_tokens[idx] : 0;
    bad_tree |= live[k] && (par[k] < -1 || par[k] >= i || (i == 0 && par[k] != -1));
    bad_tok |= live[k] && i > 0 && (tok[k] < 0 || tok[k] >= V);
  }
  const bool tree_err = __ballot(bad_tree) != 0;
  const bool tok_err = __ballot(bad_tok) != 0;
  if (bad_size || tree_err || tok_err) {
    if (lane == 0)
      raise_error(state, bad_size ? TV_ERR_INVALID_ARG : tree_err ? TV_ERR_INVALID_TREE : TV_ERR_INVALID_ARG);
#pragma unroll
    for (int k = 0; k < H; ++k) {
      const int i = lane + 64 * k;
      if (i < N) {
        const int64_t idx = static_cast<int64_t>(b) * N + i;
        path[idx] = -1;
        if (target_argmax) target_argmax[idx] = y[k];
      }
    }
    if (lane == 0) {
      accept_len[b] = -1;
      bonus[b] = -1;
    }
    return;
  }
  // ancestor-or-self sets by pointer doubling (parents precede children):
  // node j's values are in lane j % 64, half j / 64
  unsigned long long a0[H], a1[H];
  int jump[H];
#pragma unroll
  for (int k = 0; k < H; ++k) {
    a0[k] = live[k] && k == 0 ? (1ull << lane) : 0ull;
    a1[k] = live[k] && k == 1 ? (1ull << lane) : 0ull;
    jump[k] = live[k] ? par[k] : -1;
  }
#pragma unroll
  for (int r = 0; r < (H == 1 ? 6 : 7); ++r) {
    unsigned long long n0[H], n1[H];
    int nj[H];
#pragma unroll
    for (int k = 0; k < H; ++k) {
      const int j = jump[k] >= 0 ? jump[k] : lane + 64 * k;
      const int src = j & 63;
      unsigned long long s0 = shfl_u64(a0[0], src), s1 = shfl_u64(a1[0], src);
      int sj = __shfl(jump[0], src);
      if (H == 2) {
        const unsigned long long t0 = shfl_u64(a0[H - 1], src), t1 = shfl_u64(a1[H - 1], src);
        const int tj = __shfl(jump[H - 1], src);
        if (j >= 64) {
          s0 = t0;
          s1 = t1;
          sj = tj;
        }
      }
      n0[k] = a0[k];
      n1[k] = a1[k];
      nj[k] = jump[k];
      if (jump[k] >= 0) {
        n0[k] |= s0;
        n1[k] |= s1;
        nj[k] = sj;
      }
    }
#pragma unroll
    for (int k = 0; k < H; ++k) {
      a0[k] = n0[k];
      a1[k] = n1[k];
      jump[k] = nj[k];
    }
  }
  // node c >= 1 matches iff its token is the target's argmax at its parent
  bool match[H];
#pragma unroll
  for (int k = 0; k < H; ++k) {
    const int pp = par[k] >= 0 ? par[k] : 0;
    int y_par = __shfl(y[0], pp & 63);
    if (H == 2) {
      const int y_hi = __shfl(y[H - 1], pp & 63);
      if (pp >= 64) y_par = y_hi;
    }
    match[k] = live[k] && (lane + 64 * k == 0 || (par[k] >= 0 && tok[k] == y_par));
  }
  const unsigned long long m0 = __ballot(match[0]);
  const unsigned long long m1 = H == 2 ? __ballot(match[H - 1]) : 0ull;
  // deepest ok node (every node on its root path matches); ties -> the
  // lexicographically smallest root path, i.e. the largest bit-reversed set
  // (node ids increase along a path, so the first differing path element is
  // the lowest differing set bit)
  int dmax = 0;
  bool ok[H];
#pragma unroll
  for (int k = 0; k < H; ++k) {
    ok[k] = live[k] && (a0[k] & 1ull) && ((a0[k] & ~m0) == 0ull) && ((a1[k] & ~m1) == 0ull);
    if (ok[k]) dmax = max(dmax, __popcll(a0[k]) + __popcll(a1[k]));
  }
  for (int m = 32; m >= 1; m >>= 1) dmax = max(dmax, __shfl_xor(dmax, m));
  unsigned long long khi = 0ull, klo = 0ull;  // key = (brev(word 0), brev(word 1))
#pragma unroll
  for (int k = 0; k < H; ++k)
    if (ok[k] && static_cast<int>(__popcll(a0[k]) + __popcll(a1[k])) == dmax) {
      const unsigned long long h = __brevll(a0[k]), l = __brevll(a1[k]);
      if (h > khi || (h == khi && l > klo)) {
        khi = h;
        klo = l;
      }
    }
  for (int m = 32; m >= 1; m >>= 1) {
    const unsigned long long oh = shfl_xor_u64(khi, m), ol = shfl_xor_u64(klo, m);
    if (oh > khi || (oh == khi && ol > klo)) {
      khi = oh;
      klo = ol;
    }
  }
  const unsigned long long c0 = __brevll(khi), c1 = __brevll(klo);  // the chosen path's set; holds node 0
  const int len = __popcll(c0) + __popcll(c1);
  const int last = c1 ? 64 + 63 - __clzll(static_cast<long long>(c1)) : 63 - __clzll(static_cast<long long>(c0));
  int y_last = __shfl(y[0], last & 63);
  if (H == 2) {
    const int y_hi = __shfl(y[H - 1], last & 63);
    if (last >= 64) y_last = y_hi;
  }
#pragma unroll
  for (int k = 0; k < H; ++k) {
    const int pos = lane + 64 * k;  // writes the pos-th node of the path (the pos-th set bit)
    if (pos < N) {
      int node = -1;
      if (pos < len) {
        const int n0 = __popcll(c0);
        unsigned long long rest = pos < n0 ? c0 : c1;
        for (int q = pos < n0 ? pos : pos - n0; q > 0; --q) rest &= rest - 1ull;
        node = (pos < n0 ? 0 : 64) + __ffsll(static_cast<long long>(rest)) - 1;
      }
      const int64_t idx = static_cast<int64_t>(b) * N + pos;
      path[idx] = node;
      if (target_argmax) target_argmax[idx] = y[k];
    }
  }
  if (lane == 0) {
    accept_len[b] = len;
    bonus[b] = y_last;
    atomicAdd(state + 0, static_cast<unsigned long long>(len));
    atomicAdd(state + 1, 1ull);
  }
}

// Path pass on its own: one wavefront per sequence.
template <int H>
__global__ void __launch_bounds__(256) greedy_path_kernel(unsigned long long *keys, int chunks,
                                                          const int32_t *__restrict__ draft_tokens,
                                                          const int32_t *__restrict__ parents,
                                                          const int32_t *__restrict__ sizes, int B, int N, int V,
                                                          int32_t *__restrict__ accept_len, int32_t *__restrict__ path,
                                                          int32_t *__restrict__ bonus,
                                                          int32_t *__restrict__ target_argmax,
                                                          unsigned long long *state) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= B) return;
  greedy_path_seq<H, false>(b, threadIdx.x & 63, keys, chunks, draft_tokens, parents, sizes, N, V, accept_len, path,
                            bonus, target_argmax, state);
}

// Both passes in one launch. Each workgroup publishes its chunk key with a
// device-scope atomic swap, waits for the swap to complete, and counts itself
// in on its sequence's arrival counter; the workgroup that arrives last (all
// of the sequence's present rows times chunks) resets the counter to zero and
// runs the path logic in its first wavefront. No workgroup waits for another.
template <bool kVec, int H>
__global__ void __launch_bounds__(kThreads) argmax_path_kernel(
    const float *__restrict__ logits, const int32_t *__restrict__ sizes, int N, int V, int chunks,
    unsigned long long *keys, unsigned int *arrivals, const int32_t *__restrict__ draft_tokens,
    const int32_t *__restrict__ parents, int32_t *__restrict__ accept_len, int32_t *__restrict__ path,
    int32_t *__restrict__ bonus, int32_t *__restrict__ target_argmax, unsigned long long *state) {
  __shared__ unsigned long long red[kThreads / 64];
  __shared__ int s_last;
  const int chunk = static_cast<int>(blockIdx.x % static_cast<unsigned>(chunks));
  const int64_t row = blockIdx.x / static_cast<unsigned>(chunks);
  const int b = static_cast<int>(row / N);
  const int present = present_nodes(sizes, b, N);
  if (row % N >= present) return;  // an absent node: its row is never read and it is not counted
  const int x0 = chunk * kGChunk;
  const unsigned long long best = block_argmax<kVec>(logits + row * V, x0, min(x0 + kGChunk, V), red);
  if (threadIdx.x == 0) {
    atomicExch(keys + row * chunks + chunk, best);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the key is in place before this workgroup is counted
    const unsigned int arrived = atomicAdd(arrivals + b, 1u) + 1u;
    const bool last = arrived == static_cast<unsigned int>(present) * static_cast<unsigned int>(chunks);
    if (last) atomicExch(arrivals + b, 0u);
    s_last = last;
  }
  __syncthreads();
  if (!s_last || threadIdx.x >= 64) return;
  greedy_path_seq<H, true>(b, threadIdx.x, keys, chunks, draft_tokens, parents, sizes, N, V, accept_len, path, bonus,
                           target_argmax, state);
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

// e^x with a finer reduction, for the per-token work: x = (64 n + j) ln2/64
// + r with |r| <= ln2/128, e^x = 2^n * 2^(j/64) * e^r, the 64 values
// 2^(j/64) from a table the workgroup fills once (exp_table_init, exp_fast of
// j ln2/64), e^r from its Taylor series to degree 5 (truncation below 4e-17
// relative). Within a few ulp of e^x (2 ulp worst over 2e7 sampled
// arguments in [-700, 0]). The nearest integer k = 64 n + j comes from
// adding 1.5 * 2^52 (its low bits are then k in two's complement) and 2^n
// from its exponent bits, so the per-token work has no fp64 rounding,
// conversion or ldexp instruction; for x below -708.39 (2^n below the normal
// range) and for x = -inf the result is 0, under 2.3e-308 from e^x.
__device__ inline void exp_table_init(double *tab, int tid) {
  if (tid < 64) tab[tid] = exp_fast(tid * (kLn2Hi / 64.0) + tid * (kLn2Lo / 64.0));
}

__device__ inline double exp_tab(double x, const double *tab) {
  constexpr double kShift = 6755399441055744.0;  // 1.5 * 2^52
  const double ks = fma(x, kLog2eD * 64.0, kShift);
  const double k = ks - kShift;
  const int ki = static_cast<int>(__double_as_longlong(ks));  // k for |k| < 2^31
  double r = fma(-k, kLn2Hi / 64.0, x);  // exact: k has at most 17 bits, the head 32
  r = fma(-k, kLn2Lo / 64.0, r);
  double p = 1.0 / 120.0;
  p = fma(p, r, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  const int e = (ki >> 6) + 1023;  // biased exponent of 2^n
  const double two_n = __longlong_as_double(static_cast<long long>(e) << 52);
  return (e > 0 && x > -745.2) ? tab[ki & 63] * p * two_n : 0.0;
}

// exp_tab for arguments known to lie in [-707, 0]: 2^n is then a normal
// number and so is the result, so the range test is left out and 2^n is
// applied by one ldexp (the same bits as the product with 2^n). NaN in, NaN
// out.
__device__ inline double exp_tab_normal(double x, const double *tab) {
  constexpr double kShift = 6755399441055744.0;  // 1.5 * 2^52
  const double ks = fma(x, kLog2eD * 64.0, kShift);
  const double k = ks - kShift;
  const int ki = static_cast<int>(__double_as_longlong(ks));
  double r = fma(-k, kLn2Hi / 64.0, x);
  r = fma(-k, kLn2Lo / 64.0, r);
  double p = 1.0 / 120.0;
  p = fma(p, r, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  return ldexp(tab[ki & 63] * p, ki >> 6);
}

// x / T in fp64 from a precomputed 1/T and one FMA correction step (exact
// when T = 1)
__device__ inline double div_t(double x, double T, double invT) {
  const double q = x * invT;
  return fma(fma(-q, T, x), invT, q);
}

template <bool kVec>
__global__ void __launch_bounds__(kThreads) softmax_chunk_kernel(const float *__restrict__ target,
                                                                 const float *__restrict__ draft,
                                                                 const int32_t *__restrict__ sizes, int N, int V,
                                                                 int chunks, double T, double invT,
                                                                 double *__restrict__ stats,
                                                                 unsigned long long *__restrict__ counters) {
  __shared__ double red[kThreads / 64];
  const int chunk = static_cast<int>(blockIdx.x % static_cast<unsigned>(chunks));
  const int64_t row = blockIdx.x / static_cast<unsigned>(chunks);  // b * N + j
  const int which = blockIdx.z;                                     // 0 = target, 1 = draft
  const int j = static_cast<int>(row % N);
  if (sizes && j > 0 && j >= sizes[row / N]) return;  // an absent node: its rows are never read
  double *out = stats + ((row * 2 + which) * chunks + chunk) * 2;
  // the path pass's exchange counter of this sequence starts at zero
  if (counters && chunk == 0 && which == 0 && j == 0 && threadIdx.x == 0) counters[(row / N) * 16] = 0ull;
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
  constexpr int kPer = kChunk / kThreads;  // 32 logits per thread, kept in registers as fp32
  float v[kPer];
  if (kVec) {
#pragma unroll
    for (int it = 0; it < kPer / 4; ++it) {
      const int x = x0 + (it * kThreads + threadIdx.x) * 4;
      float4 f = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (x < x1) f = *reinterpret_cast<const float4 *>(p + x);
      v[it * 4 + 0] = f.x;
      v[it * 4 + 1] = f.y;
      v[it * 4 + 2] = f.z;
      v[it * 4 + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
      const int x = x0 + it * kThreads + threadIdx.x;
      v[it] = x < x1 ? p[x] : -INFINITY;
    }
  }
  // x -> x / T is monotonic, so the maximum of the scaled logits is the
  // scaled maximum logit (found in fp32)
  float mf = -INFINITY, mnf = INFINITY;
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    mf = fmaxf(mf, v[it]);
    mnf = fminf(mnf, v[it]);
  }
  for (int m = 32; m >= 1; m >>= 1) mf = fmaxf(mf, __shfl_xor(mf, m));
  __shared__ float redf[kThreads / 64];
  __shared__ double s_tab[64];
  exp_table_init(s_tab, threadIdx.x);
  if ((threadIdx.x & 63) == 0) redf[threadIdx.x >> 6] = mf;
  __syncthreads();
  mf = redf[0];
  for (int i = 1; i < kThreads / 64; ++i) mf = fmaxf(mf, redf[i]);
  const double mx = div_t(mf, T, invT);
  // every argument of this thread at or above -707 (padding, infinities and
  // far-below values fail; NaN, which fminf skips, makes the sum NaN): no
  // range test. Taken per wavefront, and redone with the test by a thread
  // whose sum is not finite, so every term is what exp_tab gives.
  const bool normal = div_t(mnf, T, invT) - mx >= -707.0;
  double zs = 0.0;
  if (__all(normal)) {
    if (T == 1.0) {
#pragma unroll 8
      for (int it = 0; it < kPer; ++it) zs += exp_tab_normal(static_cast<double>(v[it]) - mx, s_tab);
    } else {
#pragma unroll 8
      for (int it = 0; it < kPer; ++it) zs += exp_tab_normal(div_t(v[it], T, invT) - mx, s_tab);
    }
  } else {
    zs = NAN;
  }
  if (!(zs <= 1e300)) {
    zs = 0.0;
    if (T == 1.0) {  // x / 1 = x exactly
#pragma unroll 8
      for (int it = 0; it < kPer; ++it) zs += exp_tab(static_cast<double>(v[it]) - mx, s_tab);
    } else {
#pragma unroll 8
      for (int it = 0; it < kPer; ++it) zs += exp_tab(div_t(v[it], T, invT) - mx, s_tab);  // -inf (padding) gives 0
    }
  }
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

constexpr int kPathThreads = 512;
constexpr int kBlk = 8;           // tokens per register block of a row sweep
constexpr int kWaves = kPathThreads / 64;
constexpr int kRound = 64 * kBlk;  // tokens a wavefront sweeps per round (one block per lane)
constexpr int kRecords = 64;       // per-wavefront mass records of a sweep
constexpr int kLaneRounds = 8;     // rounds whose per-lane block sums a sweep keeps in LDS

// x moved across lanes by the DPP control `ctrl` (rows or banks masked off, and
// lanes with no source when bound_ctrl is set, read 0)
template <int kCtrl, int kRowMask, bool kBound>
__device__ inline double dpp_f64(double x) {
  const long long b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b), kCtrl, kRowMask, 0xf, kBound);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), kCtrl, kRowMask, 0xf, kBound);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}

// inclusive scan over the 64 lanes of a wavefront in a fixed order: within
// each 16-lane row by shifts of 1, 2, 4 and 8, then row 0's total into row
// 1, row 2's into row 3, and the first half's total into the second half
__device__ inline double wave_incl_dpp(double x) {
  x += dpp_f64<0x111, 0xf, true>(x);  // row_shr:1
  x += dpp_f64<0x112, 0xf, true>(x);  // row_shr:2
  x += dpp_f64<0x114, 0xf, true>(x);  // row_shr:4
  x += dpp_f64<0x118, 0xf, true>(x);  // row_shr:8
  x += dpp_f64<0x142, 0xa, false>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_f64<0x143, 0xc, false>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

__device__ inline double lane_f64(double x, int src) {
  const long long b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), src);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), src);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}
constexpr int kMaxGrid = 256;     // workgroups of a path pass that exchange partial sums
constexpr int kMaxExchanges = 128;  // exchanges per sequence: < N stored residuals + 2 draw passes
constexpr int kCounterStride = 16;  // one 128-byte line per sequence counter
constexpr int kSpinLimit = 1 << 22;

// The target distribution pi the walk holds: the current node's target row
// (w == nullptr, invM = 1), or a stored residual w[0..V) of mass 1 / invM.
struct Pi {
  const double *w;
  double invM;
};

// K workgroups per sequence (K = 1 when the batch alone fills the chip),
// each owning a contiguous slice of the vocabulary. Wavefront 0 of every
// workgroup validates the tree and builds the children of every node as a
// bit mask; all threads merge the row statistics and compute for every node
// c its first test's p(t_c) (under its parent's target row) and q_c(t_c);
// all threads of all K workgroups then take the same walk from these copies.
// The current node's children are tested in id order; a rejection followed
// by another sibling stores the residual max(0, pi - q_c) of the vocabulary
// (each workgroup its slice, in one of two per-sequence rows) and the next
// sibling is tested against it. The final draw - from the last rejected
// sibling's residual (built on the fly) or from pi - sweeps the slices once.
// A sweep gives each wavefront a contiguous range of its workgroup's slice,
// taken in rounds in which lane l holds the 8-token block at 8 l, so every
// wavefront load is contiguous (the next round's loads are issued before the
// current round's exponentials). Every sweep ends in an exchange: each workgroup
// publishes its slice's mass, pi's old and new weight at the next sibling's
// token, and its last positive token through device-scope atomics, counts
// itself in, and waits (bounded) until all K have; wavefront 0 then reduces
// the K slices in a fixed order, so every workgroup reaches the same
// decisions. T = 1 has a form of its own (no division of the logits). For the
// draw, the first slice whose running sum passes theta is found, then in it
// the wavefront range, round, lane and token, from the masses the sweep kept;
// only the 8 weights of one block are computed again (and, past the rounds
// whose lane sums the sweep keeps, that round's lane sums).
template <bool kVec, bool kUnitT>
__global__ void __launch_bounds__(kPathThreads) stochastic_path_kernel(
    const float *__restrict__ target, const float *__restrict__ draft, const int32_t *__restrict__ draft_tokens,
    const int32_t *__restrict__ parents, const int32_t *__restrict__ sizes, const float *__restrict__ uniforms,
    int B, int N, int V, int chunks, double T, double invT, const double *__restrict__ stats,
    double *__restrict__ wbuf,
    unsigned long long *__restrict__ sync, int K, int slice, int32_t *__restrict__ accept_len,
    int32_t *__restrict__ path, int32_t *__restrict__ bonus, unsigned long long *state) {
  __shared__ int s_err, s_ok, s_pick, s_lp;
  __shared__ double s_wave[kWaves], s_wpre[kWaves], s_total, s_wt_new, s_wt_old;
  // each wavefront's mass in records of rec_rounds consecutive rounds, and
  // its last token of positive weight (the last sweep's)
  __shared__ double s_wrec[kWaves][kRecords];
  __shared__ double s_lsum[kLaneRounds][kPathThreads];  // each lane's block sum of the first rounds
  __shared__ int s_wlp[kWaves];
  __shared__ double s_pa[128], s_qa[128], s_u[128];
  __shared__ RowStat s_tst[128], s_dst[128];  // merged statistics of every target and draft row
  __shared__ int s_tok[128], s_path[128];
  __shared__ unsigned long long s_child[128][2];  // children of each node: ids 0..63, 64..127
  // the exchange's fixed-order reductions over the K slices: total mass, the
  // new and old weights at the next sibling's token, the last positive token,
  // and each slice's exclusive prefix of the mass
  __shared__ double s_sum, s_sum_new, s_sum_old, s_pre[kMaxGrid], s_inc[kMaxGrid];
  __shared__ int s_glast;
  __shared__ double s_tab[64];
  const int b = blockIdx.x / K, kk = blockIdx.x % K;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t base = static_cast<int64_t>(b) * N;
  // a logit over T (exact when T = 1, the kUnitT form)
  auto scaled = [&](float v) __attribute__((always_inline)) -> double {
    if constexpr (kUnitT)
      return static_cast<double>(v);
    else
      return div_t(v, T, invT);
  };
  const int nb = sizes ? sizes[b] : N;
  const bool bad_size = nb < 1 || nb > N;
  // this workgroup's slice [v0, v1): each wavefront owns a contiguous range
  // of `rounds` rounds; in round r lane l takes the kBlk tokens at
  // wa0 + r kRound + l kBlk, so a wavefront's loads are contiguous and the
  // token order is (wavefront, round, lane, token). A sweep records each
  // wavefront's mass per group of rec_rounds rounds (and, for the first
  // kLaneRounds rounds, every lane's block sum), so that the final draw finds
  // the token where the running sum passes theta by recomputing one block of
  // one wavefront (past those rounds, the lane sums of the rounds of one
  // record).
  const int v0 = min(kk * slice, V), v1 = min(v0 + slice, V);
  const int rounds = (v1 - v0 + kWaves * kRound - 1) / (kWaves * kRound);
  const int rec_rounds = max(1, (rounds + kRecords - 1) / kRecords);
  auto range0 = [&](int w) { return min(v0 + w * rounds * kRound, v1); };
  const int wa0 = range0(wid), wa1 = range0(wid + 1);
  const int x0 = wa0 + lane * kBlk;  // this lane's block in round 0
  const int x1 = wa1;                // every load of the wavefront stops here
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
  exp_table_init(s_tab, tid);
  // thread i < nb (i >= 1) reads node i's parent and token, and, when both are
  // in range, the two logits of its first test (target row of the parent and
  // its own draft row at its token): random reads whose latency then overlaps
  // the statistics merge below
  float l_pa = 0.f, l_qa = 0.f;
  int my_p = -1;
  if (!bad_size && tid >= 1 && tid < nb) {
    my_p = parents[base + tid];
    const int t = draft_tokens[base + tid];
    if (my_p >= 0 && my_p < tid && t >= 0 && t < V) {
      l_pa = target[(base + my_p) * V + t];
      l_qa = draft[(base + tid) * V + t];
    }
  }
  // the chunk statistics of each thread's first row (see the merge below),
  // loaded now so that their latency overlaps the validation
  constexpr int kPreChunks = 4;  // per thread: chunks sub, sub + 4, ...
  const int sub = tid & 3;
  const bool pre_ok = !bad_size && (tid >> 2) < 2 * nb && chunks <= 4 * kPreChunks;
  double pre_m[kPreChunks], pre_s[kPreChunks];
  if (pre_ok) {
    const int r = tid >> 2;
    const double *st = stats + ((base + (r >> 1)) * 2 + (r & 1)) * chunks * 2;
#pragma unroll
    for (int j = 0; j < kPreChunks; ++j) {
      const int c = sub + 4 * j;
      pre_m[j] = c < chunks ? st[2 * c] : -INFINITY;
      pre_s[j] = c < chunks ? st[2 * c + 1] : 0.0;
    }
  }
  if (wid == 0) {
    // validation with the same precedence as a serial check: a node count
    // outside [1, N], a bad parent among the present nodes, then a draft
    // token outside [0, V). Lane i holds nodes i and i + 64.
    bool tree_bad = false, tok_bad = false;
    int p[2], t[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = lane + 64 * h;
      p[h] = -1;
      t[h] = 0;
      if (!bad_size && i < nb) {
        p[h] = parents[base + i];
        tree_bad |= p[h] < -1 || p[h] >= i || (i == 0 && p[h] != -1);
        if (i >= 1) {
          t[h] = draft_tokens[base + i];
          tok_bad |= t[h] < 0 || t[h] >= V;
        }
      }
      if (i < N) s_u[i] = static_cast<double>(uniforms[base + i]);
      if (i >= 1 && i < nb) s_tok[i] = t[h];
    }
    const int err = bad_size                                 ? TV_ERR_INVALID_ARG
                    : __builtin_amdgcn_ballot_w64(tree_bad) ? TV_ERR_INVALID_TREE
                    : __builtin_amdgcn_ballot_w64(tok_bad)  ? TV_ERR_INVALID_ARG
                                                            : 0;
    for (int n = 0; n < (err ? 0 : nb); ++n) {
      const uint64_t k0 = __builtin_amdgcn_ballot_w64(lane >= 1 && lane < nb && p[0] == n);
      const uint64_t k1 = __builtin_amdgcn_ballot_w64(lane + 64 < nb && p[1] == n);
      if (lane == 0) {
        s_child[n][0] = k0;
        s_child[n][1] = k1;
      }
    }
    if (lane == 0) {
      s_err = err;
      s_pick = 0x7FFFFFFF;
      s_lp = -1;
      s_wt_new = 0.0;
      s_wt_old = 0.0;
      s_path[0] = 0;
    }
  }
  __syncthreads();  // s_tab, s_child, s_err
  // first blocks of a target row and a draft row loaded ahead of their sweep,
  // tagged with their node: the root's row and its first child's row after
  // the statistics merge, the next sibling's row during each sweep
  float ppre[kBlk], qpre[kBlk];
  int ppre_node = -1, qpre_node = -1;
  // the lane's round-0 block of the residual the last storing sweep wrote:
  // the next sweep over that residual reads exactly these tokens of it, so
  // it takes them from here instead of from memory
  double wcache[kBlk];
  const double *wcache_row = nullptr;
  // statistics of every present row (target and draft of each node) from
  // its chunks' (max, sum of exp): four threads per row, each taking every
  // fourth chunk, combined in a fixed butterfly so that all four, and every
  // workgroup of the sequence, hold the same values
  if (!bad_size) {
    for (int r = tid >> 2; r < 2 * nb; r += kPathThreads / 4) {
      const int node = r >> 1, which = r & 1;
      const double *st = stats + ((base + node) * 2 + which) * chunks * 2;
      double M = -INFINITY;
      double Z = 0.0;
      if (pre_ok && r == (tid >> 2)) {
#pragma unroll
        for (int j = 0; j < kPreChunks; ++j) M = fmax(M, pre_m[j]);
        M = fmax(M, __shfl_xor(M, 1));
        M = fmax(M, __shfl_xor(M, 2));
#pragma unroll
        for (int j = 0; j < kPreChunks; ++j)
          if (pre_s[j] > 0.0) Z += pre_s[j] * exp_tab(pre_m[j] - M, s_tab);
      } else {
        for (int c = sub; c < chunks; c += 4) M = fmax(M, st[2 * c]);
        M = fmax(M, __shfl_xor(M, 1));
        M = fmax(M, __shfl_xor(M, 2));
        for (int c = sub; c < chunks; c += 4)
          if (st[2 * c + 1] > 0.0) Z += st[2 * c + 1] * exp_tab(st[2 * c] - M, s_tab);
      }
      Z += __shfl_xor(Z, 1);
      Z += __shfl_xor(Z, 2);
      if (sub == 0) {
        if (which == 0)
          s_tst[node] = RowStat{M, Z, 1.0 / Z};
        else
          s_dst[node] = node >= 1 ? RowStat{M, Z, 1.0 / Z} : RowStat{0.0, 1.0, 1.0};
      }
    }
  }
  if (!s_err) {
    load_block(target + base * V, x0, ppre);
    ppre_node = 0;
    if (s_child[0][0] | s_child[0][1]) {
      const int c0 = s_child[0][0] ? __builtin_ctzll(s_child[0][0]) : 64 + __builtin_ctzll(s_child[0][1]);
      load_block(draft + (base + c0) * V, x0, qpre);
      qpre_node = c0;
    }
  }
  __syncthreads();  // s_tst, s_dst, s_err
  // each present node's first test: p(t_c) under its parent's target row
  // and q_c(t_c) (a node without a parent, in a forest, is never tested)
  if (!s_err && tid >= 1 && tid < nb && my_p >= 0) {
    s_pa[tid] = exp_tab(scaled(l_pa) - s_tst[my_p].m, s_tab) * s_tst[my_p].invZ;
    s_qa[tid] = exp_tab(scaled(l_qa) - s_dst[tid].m, s_tab) * s_dst[tid].invZ;
  }
  __syncthreads();
  if (s_err) {
    if (kk == 0) {
      if (tid == 0) {
        raise_error(state, s_err);
        accept_len[b] = -1;
        bonus[b] = -1;
      }
      for (int i = tid; i < N; i += kPathThreads) path[base + i] = -1;
    }
    return;
  }
  double *const buf0 = wbuf + static_cast<int64_t>(b) * 2 * V;
  double *const buf1 = buf0 + V;

  // a token's weight under pi when pi is a target row (padding, -inf, gives
  // 0), and the residual max(0, pi - q) with pi normalised; the sweeps and
  // the final draw's recomputation share these forms
  auto block_w0 = [&](float pl, const RowStat &sp) __attribute__((always_inline)) {
    return exp_tab(scaled(pl) - sp.m, s_tab) * sp.invZ;
  };
  auto block_resid = [&](double w0, const Pi &pi, float ql, const RowStat &sq) __attribute__((always_inline)) {
    return fmax(0.0, w0 * pi.invM - exp_tab(scaled(ql) - sq.m, s_tab) * sq.invZ);
  };
  // one sweep of this wavefront's range; stores every weight into dst if
  // given; the thread holding token tnext records pi's old and new weight
  // there. The form (pi stored or a target row, with or without a sibling's
  // draft row, with or without dst) is chosen once per sweep, so a block of
  // 8 tokens is straight-line code: its 8 (or 16) exponentials overlap, and
  // per-token conditions are selects (tokens past the range weigh 0).
  auto sweep_form = [&](auto has_w, auto has_q, auto has_dst, const float *P, int pnode, const RowStat &sp,
                        const Pi &pi, const float *Q, int qnode, const RowStat &sq, const float *Qnext,
                        int qnext_node, double *dst, int tnext, double &local, int &lastpos)
      __attribute__((always_inline)) {
    constexpr bool kW = decltype(has_w)::value, kQ = decltype(has_q)::value, kDst = decltype(has_dst)::value;
    local = 0.0;
    lastpos = -1;
    const int nr = wa0 < wa1 ? rounds : 0;  // a wavefront with an empty range has no rounds
    double rec = 0.0;
    float pv[kBlk], qv[kBlk], pn[kBlk], qn[kBlk];
    double wv[kBlk], wn[kBlk];
    if constexpr (kW) {
      if (pi.w == wcache_row) {
#pragma unroll
        for (int i = 0; i < kBlk; ++i) wv[i] = wcache[i];
      } else {
        load_wblock(pi.w, x0, wv);
      }
    } else if (pnode == ppre_node) {
#pragma unroll
      for (int i = 0; i < kBlk; ++i) pv[i] = ppre[i];
    } else {
      load_block(P, x0, pv);
    }
    if constexpr (kQ) {
      if (qnode == qpre_node) {
#pragma unroll
        for (int i = 0; i < kBlk; ++i) qv[i] = qpre[i];
      } else {
        load_block(Q, x0, qv);
      }
    }
    // the next sibling's row: its first block loads while this sweep computes
    if (Qnext) {
      load_block(Qnext, x0, qpre);
      qpre_node = qnext_node;
    }
    double w0_at = 0.0, w_at = 0.0;
    bool have_at = false;
    for (int r = 0; r < nr; ++r) {
      const int xb = x0 + r * kRound;
      if (r + 1 < nr) {
        if constexpr (kW)
          load_wblock(pi.w, xb + kRound, wn);
        else
          load_block(P, xb + kRound, pn);
        if constexpr (kQ) load_block(Q, xb + kRound, qn);
      }
      double wb[kBlk];
      double bs = 0.0;
#pragma unroll
      for (int i = 0; i < kBlk; ++i) {
        double w0;
        if constexpr (kW)
          w0 = wv[i];
        else
          w0 = block_w0(pv[i], sp);
        double w = w0;
        if constexpr (kQ) w = block_resid(w0, pi, qv[i], sq);
        wb[i] = w;
        bs += w;
        lastpos = w > 0.0 ? xb + i : lastpos;
        const bool at = xb + i == tnext;
        have_at |= at;
        w0_at = at ? w0 : w0_at;
        w_at = at ? w : w_at;
      }
      // the round's mass over the wavefront (the same fixed-order scan the
      // final draw repeats), added to the current record
      if (r < kLaneRounds) s_lsum[r][tid] = bs;
      rec += lane_f64(wave_incl_dpp(bs), 63);
      if ((r + 1) % rec_rounds == 0 || r + 1 == nr) {
        if (lane == 0) s_wrec[wid][r / rec_rounds] = rec;
        local += rec;
        rec = 0.0;
      }
      if constexpr (kDst) {
        if (r == 0) {
#pragma unroll
          for (int i = 0; i < kBlk; ++i) wcache[i] = wb[i];
        }
        if (xb + kBlk <= x1) {
#pragma unroll
          for (int i = 0; i < kBlk; ++i) dst[xb + i] = wb[i];
        } else {
#pragma unroll
          for (int i = 0; i < kBlk; ++i)
            if (xb + i < x1) dst[xb + i] = wb[i];
        }
      }
#pragma unroll
      for (int i = 0; i < kBlk; ++i) {
        pv[i] = pn[i];
        qv[i] = qn[i];
        wv[i] = wn[i];
      }
    }
    if (have_at) {
      s_wt_old = w0_at;
      s_wt_new = w_at;
    }
    if constexpr (kDst) wcache_row = nr > 0 ? dst : nullptr;
  };
  auto sweep = [&](const float *P, int pnode, const RowStat &sp, const Pi &pi, const float *Q, int qnode,
                   const RowStat &sq, const float *Qnext, int qnext_node, double *dst, int tnext, double &local,
                   int &lastpos) __attribute__((always_inline)) {
    using T0 = std::false_type;
    using T1 = std::true_type;
    if (dst) {  // a rejected sibling with siblings left: always a draft row, pi either form
      if (pi.w)
        sweep_form(T1(), T1(), T1(), P, pnode, sp, pi, Q, qnode, sq, Qnext, qnext_node, dst, tnext, local, lastpos);
      else
        sweep_form(T0(), T1(), T1(), P, pnode, sp, pi, Q, qnode, sq, Qnext, qnext_node, dst, tnext, local, lastpos);
    } else if (Q) {
      if (pi.w)
        sweep_form(T1(), T1(), T0(), P, pnode, sp, pi, Q, qnode, sq, Qnext, qnext_node, dst, tnext, local, lastpos);
      else
        sweep_form(T0(), T1(), T0(), P, pnode, sp, pi, Q, qnode, sq, Qnext, qnext_node, dst, tnext, local, lastpos);
    } else {
      if (pi.w)
        sweep_form(T1(), T0(), T0(), P, pnode, sp, pi, Q, qnode, sq, Qnext, qnext_node, dst, tnext, local, lastpos);
      else
        sweep_form(T0(), T0(), T0(), P, pnode, sp, pi, Q, qnode, sq, Qnext, qnext_node, dst, tnext, local, lastpos);
    }
  };
  // the workgroup's total and each wavefront's exclusive prefix, summed over
  // the wavefront masses in order; the last token of positive weight of
  // each wavefront and of the workgroup
  auto scan = [&](double wave_mass, int lastpos) __attribute__((always_inline)) {
    int lp = lastpos;
    for (int d = 32; d >= 1; d >>= 1) lp = max(lp, __shfl_xor(lp, d));
    if (lane == 0) {
      s_wave[wid] = wave_mass;
      s_wlp[wid] = lp;
      if (lp >= 0) atomicMax(&s_lp, lp);
    }
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
  };
  // the exchange among the K workgroups of this sequence: every slice's mass
  // (as exclusive and inclusive prefixes), weight sums and last positive
  // token into LDS, and the per-sweep records reset; false if a peer never
  // arrived
  int nx = 0;
  auto exchange = [&]() __attribute__((always_inline)) {
    // wavefront 0 publishes this workgroup's values, gathers every slice's
    // (lane i = slice i, K <= 64) and reduces them; the other wavefronts
    // wait at the closing barrier
    if (wid == 0) {
      double m = 0.0, wn = 0.0, wo = 0.0;
      int lp = -1, ok = 1;
      if (K == 1) {
        if (lane == 0) {
          m = s_total;
          wn = s_wt_new;
          wo = s_wt_old;
          lp = s_lp;
        }
      } else {
        unsigned long long *cnt = sync + static_cast<int64_t>(b) * kCounterStride;
        unsigned long long *slots = sync + static_cast<int64_t>(B) * kCounterStride +
                                    (static_cast<int64_t>(nx) * kMaxGrid + static_cast<int64_t>(b) * K) * 4;
        if (lane == 0) {
          unsigned long long *mine = slots + kk * 4;
          atomicExch(mine + 0, static_cast<unsigned long long>(__double_as_longlong(s_total)));
          atomicExch(mine + 1, static_cast<unsigned long long>(__double_as_longlong(s_wt_new)));
          atomicExch(mine + 2, static_cast<unsigned long long>(__double_as_longlong(s_wt_old)));
          atomicExch(mine + 3, static_cast<unsigned long long>(static_cast<long long>(s_lp)));
          // the four values are in place before this workgroup is counted in
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          atomicAdd(cnt, 1ull);
          const unsigned long long want = static_cast<unsigned long long>(K) * (nx + 1);
          ok = 0;
          for (int it = 0; it < kSpinLimit; ++it) {
            if (atomicAdd(cnt, 0ull) >= want) {
              ok = 1;
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
        }
        ok = __shfl(ok, 0);
        if (ok && lane < K) {
          auto *theirs = slots + lane * 4;
          m = __longlong_as_double(static_cast<long long>(atomicAdd(theirs + 0, 0ull)));
          wn = __longlong_as_double(static_cast<long long>(atomicAdd(theirs + 1, 0ull)));
          wo = __longlong_as_double(static_cast<long long>(atomicAdd(theirs + 2, 0ull)));
          lp = static_cast<int>(static_cast<long long>(atomicAdd(theirs + 3, 0ull)));
        }
      }
      if (lane == 0) {  // the per-sweep records start again
        s_wt_new = 0.0;
        s_wt_old = 0.0;
        s_lp = -1;
        s_ok = ok;
      }
      if (ok) {
        // the slices' masses as an inclusive scan (the total is the last
        // lane's), the weight sums and the last positive token, each in a
        // fixed order
        double incl = m;
        for (int d = 1; d < 64; d <<= 1) {
          const double t = __shfl_up(incl, d);
          if (lane >= d) incl += t;
        }
        for (int d = 32; d >= 1; d >>= 1) {
          wn += __shfl_xor(wn, d);
          wo += __shfl_xor(wo, d);
          lp = max(lp, __shfl_xor(lp, d));
        }
        double excl = __shfl_up(incl, 1);
        if (lane == 0) excl = 0.0;
        if (lane < K) {
          s_pre[lane] = excl;
          s_inc[lane] = incl;
        }
        if (lane == K - 1) s_sum = incl;
        if (lane == 0) {
          s_sum_new = wn;
          s_sum_old = wo;
          s_glast = lp;
        }
      }
    }
    ++nx;
    __syncthreads();
    return s_ok != 0;
  };

  // the walk; every thread of every workgroup takes the same decisions
  Pi pi{nullptr, 1.0};
  double wt = 0.0;  // pi's (unnormalised) weight at the next sibling's token, when pi is stored
  int node = 0, k = 0, pend = -1;
  bool ok = true;
  for (;;) {
    const float *P = target + (base + node) * V;
    const RowStat sp = s_tst[node];
    uint64_t kids0 = s_child[node][0], kids1 = s_child[node][1];  // children still to test, in id order
    int acc = -1;
    while (kids0 | kids1) {
      int c;
      if (kids0) {
        c = __builtin_ctzll(kids0);
        kids0 &= kids0 - 1;
      } else {
        c = 64 + __builtin_ctzll(kids1);
        kids1 &= kids1 - 1;
      }
      const double a = pi.w ? (wt * pi.invM) / s_qa[c] : s_pa[c] / s_qa[c];
      if (s_u[c - 1] < a) {
        acc = c;
        break;
      }
      if (!(kids0 | kids1)) {  // the last sibling: its residual is built on the fly by the final draw
        pend = c;
        break;
      }
      double *dst = pi.w == buf0 ? buf1 : buf0;
      const RowStat sq = s_dst[c];
      double local;
      int lastpos;
      const int next = kids0 ? __builtin_ctzll(kids0) : 64 + __builtin_ctzll(kids1);
      // the next sibling's row is swept next (rejected with siblings left, or
      // as the final draw's residual)
      sweep(P, node, sp, pi, draft + (base + c) * V, c, sq, draft + (base + next) * V, next, dst, s_tok[next], local,
            lastpos);
      scan(local, lastpos);
      if (!(ok = exchange())) break;
      const double total = s_sum, wnew = s_sum_new, wold = s_sum_old;
      if (total > 0.0) {
        pi = Pi{dst, 1.0 / total};
        wt = wnew;
      } else if (pi.w) {
        wt = wold;  // a residual of mass 0 leaves pi unchanged
      }
    }
    if (!ok || acc < 0) break;
    node = acc;
    ++k;
    if (tid == 0) s_path[k] = acc;
    pi = Pi{nullptr, 1.0};
  }

  // the final draw
  int writer = 0, pick = -1;
  if (ok) {
    const float *P = target + (base + node) * V;
    const float *Q = pend >= 0 ? draft + (base + pend) * V : nullptr;
    const RowStat sp = s_tst[node];
    const RowStat sq = Q ? s_dst[pend] : RowStat{0.0, 1.0, 1.0};
    const double u = s_u[N - 1];
    for (int pass = 0; pass < 2; ++pass) {
      const float *Qp = pass == 0 ? Q : nullptr;
      double local;
      int lastpos;
      sweep(P, node, sp, pi, Qp, pass == 0 ? pend : -1, sq, nullptr, -1, nullptr, -1, local, lastpos);
      scan(local, lastpos);
      if (!(ok = exchange())) break;
      const double total = s_sum;
      const int glast = s_glast;
      if (Qp && !(total > 0.0)) continue;  // no residual mass: draw from pi instead
      const double theta = u * total;
      // the first slice whose running sum passes theta holds the draw
      const uint64_t crossing = __builtin_amdgcn_ballot_w64(lane < K && s_inc[min(lane, K - 1)] > theta);
      const int cross_wg = crossing ? static_cast<int>(__builtin_ctzll(crossing)) : -1;
      const double wg_prefix = cross_wg >= 0 ? s_pre[cross_wg] : 0.0;
      writer = cross_wg >= 0 ? cross_wg : 0;
      pick = glast;  // rounding left no crossing: the last token of positive weight
      if (cross_wg == kk) {
        // wavefront 0 narrows the crossing down: the first wavefront range,
        // then record, round, lane and token whose running sum passes theta
        // (each level's sums in the order the sweep formed them); where
        // rounding leaves no crossing inside the range found, the range's
        // last token of positive weight
        if (wid == 0) {
          const uint64_t wr_hit = __builtin_amdgcn_ballot_w64(
              lane < kWaves && wg_prefix + s_wpre[min(lane, kWaves - 1)] + s_wave[min(lane, kWaves - 1)] > theta);
          if (wr_hit) {
            const int wc = static_cast<int>(__builtin_ctzll(wr_hit));
            const int ca0 = range0(wc), ca1 = range0(wc + 1);
            double run = wg_prefix + s_wpre[wc];
            int found = -1;
            const int nrec = (rounds + rec_rounds - 1) / rec_rounds;
            for (int q = 0; q < nrec && found < 0; ++q) {
              const double rm = s_wrec[wc][q];
              if (!(run + rm > theta)) {
                run += rm;
                continue;
              }
              for (int r = q * rec_rounds; r < min((q + 1) * rec_rounds, rounds) && found < 0; ++r) {
                const int xr = ca0 + r * kRound;  // the round's first token
                // a token's weight, as the sweep formed it (0 past the range)
                auto token_w = [&](int x) __attribute__((always_inline)) -> double {
                  if (x >= ca1) return 0.0;
                  const double w0 = pi.w ? pi.w[x] : block_w0(P[x], sp);
                  return Qp ? block_resid(w0, pi, Qp[x], sq) : w0;
                };
                // each lane's block sum: kept by the sweep for the first
                // rounds, recomputed in the same order otherwise
                double bs = 0.0;
                if (r < kLaneRounds) {
                  bs = s_lsum[r][wc * 64 + lane];
                } else {
#pragma unroll
                  for (int i = 0; i < kBlk; ++i) bs += token_w(xr + lane * kBlk + i);
                }
                const double incl = wave_incl_dpp(bs);
                const uint64_t lhit = __builtin_amdgcn_ballot_w64(run + incl > theta);
                if (lhit) {
                  // the crossing block: lanes 0..kBlk-1 recompute its tokens,
                  // whose running sum is then taken in token order
                  const int lc = static_cast<int>(__builtin_ctzll(lhit));
                  const int xl = xr + lc * kBlk;
                  const double wi = lane < kBlk ? token_w(xl + lane) : 0.0;
                  double c = run + (lc > 0 ? lane_f64(incl, lc - 1) : 0.0);
                  int f = -1, lpos = -1;
#pragma unroll
                  for (int i = 0; i < kBlk; ++i) {
                    const double w = lane_f64(wi, i);
                    c += w;
                    lpos = w > 0.0 ? xl + i : lpos;
                    if (f < 0 && c > theta) f = xl + i;
                  }
                  found = f >= 0 ? f : (lpos >= 0 ? lpos : s_wlp[wc]);
                }
                run += lane_f64(incl, 63);
              }
              if (found < 0) found = s_wlp[wc];
            }
            if (found < 0) found = s_wlp[wc];
            if (lane == 0 && found >= 0) s_pick = found;
          }
        }
        __syncthreads();
        if (s_pick != 0x7FFFFFFF) pick = s_pick;
      }
      break;
    }
  }
  if (kk != writer) return;
  if (!ok) {  // a peer workgroup never arrived (not co-resident): report and give up
    if (tid == 0) {
      raise_error(state, TV_ERR_HIP);
      accept_len[b] = -1;
      bonus[b] = -1;
    }
    for (int i = tid; i < N; i += kPathThreads) path[base + i] = -1;
    return;
  }
  if (tid == 0) {
    accept_len[b] = k + 1;
    bonus[b] = pick;
    atomicAdd(state + 0, static_cast<unsigned long long>(k + 1));
    atomicAdd(state + 1, 1ull);
  }
  for (int i = tid; i < N; i += kPathThreads) path[base + i] = i <= k ? s_path[i] : -1;
}

}  // namespace

// stochastic: the chunk statistics, then (256-byte aligned) two residual
// rows of V doubles per sequence, then the path pass's exchange area (one
// counter line per sequence, slots for every exchange of up to kMaxGrid
// workgroups)
size_t stats_doubles(int B, int N, int V) {
  const int chunks = (V + kChunk - 1) / kChunk;
  return ((static_cast<size_t>(B) * N * 2 * chunks * 2 + 31) / 32) * 32;
}

size_t accept_ws_bytes(int B, int N, int V, tv_accept_mode mode) {
  if (mode == TV_GREEDY)
    return static_cast<size_t>(B) * N * ((V + kGChunk - 1) / kGChunk) * sizeof(unsigned long long);
  const size_t sync = static_cast<size_t>(B) * kCounterStride + static_cast<size_t>(kMaxExchanges) * kMaxGrid * 4;
  return (stats_doubles(B, N, V) + static_cast<size_t>(B) * 2 * V) * sizeof(double) +
         sync * sizeof(unsigned long long);
}

tv_status launch_accept(tv_ctx *ctx, const float *target_logits, const float *draft_logits,
                        const int32_t *draft_tokens, const int32_t *parents, const int32_t *tree_sizes,
                        const float *uniforms, int B, int N, int V, tv_accept_mode mode, float temperature,
                        int32_t *accept_len, int32_t *path, int32_t *bonus, int32_t *target_argmax,
                        void *workspace) {
  const dim3 blk(kThreads);
  const bool vec = (V % 4) == 0 && (reinterpret_cast<uintptr_t>(target_logits) & 15) == 0 &&
                   (draft_logits == nullptr || (reinterpret_cast<uintptr_t>(draft_logits) & 15) == 0);
  if (mode == TV_GREEDY) {
    const int chunks = (V + kGChunk - 1) / kGChunk;
    auto *keys = static_cast<unsigned long long *>(workspace);
    const dim3 g1(static_cast<unsigned>(static_cast<int64_t>(B) * N * chunks));
    // one launch when the grid is small: the last workgroup of each sequence
    // runs its path logic. Every workgroup then pays two device-scope atomics
    // (about 7.5 ns each, measured across the chip), which outweighs the saved
    // launch beyond a few hundred workgroups.
    if (B <= kMaxFusedSeqs && static_cast<int64_t>(B) * N * chunks <= kMaxFusedGrid) {
      auto *fn = vec ? (N <= 64 ? argmax_path_kernel<true, 1> : argmax_path_kernel<true, 2>)
                     : (N <= 64 ? argmax_path_kernel<false, 1> : argmax_path_kernel<false, 2>);
      hipLaunchKernelGGL(fn, g1, blk, 0, ctx->stream, target_logits, tree_sizes, N, V, chunks, keys,
                         ctx->d_arrivals, draft_tokens, parents, accept_len, path, bonus, target_argmax,
                         ctx->d_state);
      return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
    }
    if (vec)
      hipLaunchKernelGGL(argmax_chunk_kernel<true>, g1, blk, 0, ctx->stream, target_logits, tree_sizes, N, V, chunks,
                         keys);
    else
      hipLaunchKernelGGL(argmax_chunk_kernel<false>, g1, blk, 0, ctx->stream, target_logits, tree_sizes, N, V, chunks,
                         keys);
    if (hipGetLastError() != hipSuccess) return TV_ERR_HIP;
    if (N <= 64)
      hipLaunchKernelGGL(greedy_path_kernel<1>, dim3((B + 3) / 4), dim3(256), 0, ctx->stream, keys, chunks,
                         draft_tokens, parents, tree_sizes, B, N, V, accept_len, path, bonus, target_argmax,
                         ctx->d_state);
    else
      hipLaunchKernelGGL(greedy_path_kernel<2>, dim3((B + 3) / 4), dim3(256), 0, ctx->stream, keys, chunks,
                         draft_tokens, parents, tree_sizes, B, N, V, accept_len, path, bonus, target_argmax,
                         ctx->d_state);
    return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
  }
  const int chunks = (V + kChunk - 1) / kChunk;
  auto *stats = static_cast<double *>(workspace);
  double *wbuf = stats + stats_doubles(B, N, V);
  auto *sync = reinterpret_cast<unsigned long long *>(wbuf + static_cast<size_t>(B) * 2 * V);
  const double T = static_cast<double>(temperature), invT = 1.0 / T;
  // workgroups per sequence for the path pass: enough to fill the chip when
  // the batch is small, each with a slice of at most about 4096 tokens (8 per
  // thread). The K workgroups of a sequence wait for each other, so the grid
  // stays within what the chip holds at once. It is a plain launch: a
  // workgroup held back past the bounded wait (another stream's pass holding
  // part of the chip at the same time) makes the call report TV_ERR_HIP
  // rather than hang.
  const void *forms[4] = {reinterpret_cast<const void *>(stochastic_path_kernel<false, false>),
                          reinterpret_cast<const void *>(stochastic_path_kernel<false, true>),
                          reinterpret_cast<const void *>(stochastic_path_kernel<true, false>),
                          reinterpret_cast<const void *>(stochastic_path_kernel<true, true>)};
  const void *path_fn = forms[(vec ? 2 : 0) + (T == 1.0 ? 1 : 0)];
  int K = 1;
  if (B <= kMaxGrid && V >= 2 * 4096) {
    if (ctx->path_blocks_per_cu == 0) {  // the least over the four forms
      int least = 1 << 30;
      for (const void *fn : forms) {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kPathThreads, 0) != hipSuccess || nb < 1) nb = -1;
        least = min(least, nb);
      }
      ctx->path_blocks_per_cu = least;
    }
    if (ctx->path_blocks_per_cu > 0) {
      // split when every sequence gets at least two workgroups
      const int cap = min(kMaxGrid, ctx->path_blocks_per_cu * ctx->cu_count);
      if (cap / B >= 2) K = max(1, min(min(cap / B, (V + 4095) / 4096), 64));
    }
  }
  const int slice = (((V + K - 1) / K) + 3) / 4 * 4;
  const dim3 g1(static_cast<unsigned>(static_cast<int64_t>(B) * N * chunks), 1, 2);
  unsigned long long *counters = K > 1 ? sync : nullptr;
  if (vec)
    hipLaunchKernelGGL(softmax_chunk_kernel<true>, g1, blk, 0, ctx->stream, target_logits, draft_logits, tree_sizes,
                       N, V, chunks, T, invT, stats, counters);
  else
    hipLaunchKernelGGL(softmax_chunk_kernel<false>, g1, blk, 0, ctx->stream, target_logits, draft_logits, tree_sizes,
                       N, V, chunks, T, invT, stats, counters);
  if (hipGetLastError() != hipSuccess) return TV_ERR_HIP;
  unsigned long long *st = ctx->d_state;
  void *args[] = {const_cast<float **>(&target_logits), const_cast<float **>(&draft_logits),
                  const_cast<int32_t **>(&draft_tokens), const_cast<int32_t **>(&parents),
                  const_cast<int32_t **>(&tree_sizes), const_cast<float **>(&uniforms), &B, &N, &V,
                  const_cast<int *>(&chunks),
                  const_cast<double *>(&T), const_cast<double *>(&invT), &stats, &wbuf, &sync, &K,
                  const_cast<int *>(&slice), &accept_len, &path, &bonus, &st};
  const hipError_t e = hipLaunchKernel(path_fn, dim3(B * K), dim3(kPathThreads), args, 0, ctx->stream);
  return e == hipSuccess && hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

}  // namespace tv
