// attention.hip - tree-masked attention over a paged GQA KV cache.
//
// What is computed (EAGLE-2 deep-dive page, third pillar; production note on
// indexing tree masks over paged memory): every tree node's query rows attend
// to the whole cached prefix of their sequence plus the tree positions whose
// bit is set in the node's ancestor mask. Work unit: one (sequence, KV head,
// block of query rows, key split). All query heads of a GQA group share the
// KV head, so a workgroup stages each 64-key K/V tile once in LDS and reuses
// it for every (node, head-in-group) row it owns. Only the tiles that overlap
// the tree positions [L, L + N) evaluate the mask; prefix tiles never do.
// Softmax is the online (running max / running sum) form in base 2; long key
// ranges are split across workgroups and merged by a combine kernel.
#include <math.h>

#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kRows = 64;       // query rows per workgroup
constexpr int kKeys = 64;       // keys per tile
constexpr int kWaveRows = 16;   // rows per wavefront (4 wavefronts)
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
  const uint16_t *q, *k, *v;
  const int32_t *page_table, *prefix_lens;
  const uint64_t *mask;
  int64_t num_pages;
  int maxp, max_prefix_len;
  int B, N, Hq, Hkv, G, rows, rows_pad;
  float scale_log2;
  void *out;
  int out_bf16;
  float *ws_o, *ws_ml;
  int S, chunk_tiles;
  unsigned long long *state;
};

template <int D>
__global__ void __launch_bounds__(256) attn_fma_kernel(AttnArgs a) {
  constexpr int DC = D / 64;  // output columns per lane
  __shared__ float Qs[kRows][D];
  __shared__ float Ks[kKeys][D + 1];
  __shared__ float Vs[kKeys][D];
  __shared__ float Ps[4][kWaveRows][kKeys];
  __shared__ int bad_page;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.y / a.Hkv, g = blockIdx.y % a.Hkv, s = blockIdx.z, rb = blockIdx.x;
  const int L = a.prefix_lens[b];
  const bool bad_len = L < 0 || L > a.max_prefix_len;
  const int T = bad_len ? 0 : L + a.N;
  const int tiles_b = (T + kKeys - 1) / kKeys;
  const int t_begin = s * a.chunk_tiles;
  const int t_end = min(t_begin + a.chunk_tiles, tiles_b);
  if (tid == 0) bad_page = 0;

  for (int e = tid; e < kRows * D; e += 256) {
    const int r = e / D, d = e % D, row = rb * kRows + r;
    float val = 0.f;
    if (row < a.rows) {
      const int i = row / a.G, h = g * a.G + row % a.G;
      val = bf16_bits_to_float(a.q[((static_cast<int64_t>(b) * a.N + i) * a.Hq + h) * D + d]);
    }
    Qs[r][d] = val;
  }
  uint64_t mrow[kWaveRows];
#pragma unroll
  for (int r = 0; r < kWaveRows; ++r) {
    const int row = rb * kRows + w * kWaveRows + r;
    const int i = row < a.rows ? row / a.G : 0;
    mrow[r] = a.mask ? a.mask[static_cast<int64_t>(b) * a.N + i] : ~0ull;
  }
  float m[kWaveRows], l[kWaveRows], o[kWaveRows][DC];
#pragma unroll
  for (int r = 0; r < kWaveRows; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int c = 0; c < DC; ++c) o[r][c] = 0.f;
  }

  for (int tile = t_begin; tile < t_end; ++tile) {
    const int t0 = tile * kKeys;
    __syncthreads();
    // gather the 64-token K/V tile: 4 pages of 16 tokens, 16-byte loads
    for (int e = tid * 8; e < kKeys * D; e += 256 * 8) {
      const int tok = e / D, d = e % D, t = t0 + tok;
      uint4 kk = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (t < T) {
        const int pid = a.page_table[static_cast<int64_t>(b) * a.maxp + t / kPage];
        if (pid >= 0 && pid < a.num_pages) {
          const int64_t off = ((static_cast<int64_t>(pid) * a.Hkv + g) * kPage + t % kPage) * D + d;
          kk = *reinterpret_cast<const uint4 *>(a.k + off);
          vv = *reinterpret_cast<const uint4 *>(a.v + off);
        } else {
          bad_page = 1;
        }
      }
      const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w}, vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Ks[tok][d + 2 * j] = __uint_as_float(kw[j] << 16);
        Ks[tok][d + 2 * j + 1] = __uint_as_float(kw[j] & 0xFFFF0000u);
        Vs[tok][d + 2 * j] = __uint_as_float(vw[j] << 16);
        Vs[tok][d + 2 * j + 1] = __uint_as_float(vw[j] & 0xFFFF0000u);
      }
    }
    __syncthreads();

    // scores: lane = key
    float sacc[kWaveRows];
#pragma unroll
    for (int r = 0; r < kWaveRows; ++r) sacc[r] = 0.f;
    for (int d = 0; d < D; ++d) {
      const float kd = Ks[lane][d];
#pragma unroll
      for (int r = 0; r < kWaveRows; ++r) sacc[r] = fmaf(Qs[w * kWaveRows + r][d], kd, sacc[r]);
    }
    const int t = t0 + lane;
    const bool key_ok = t < T;
    const bool is_tree = t >= L;
    const int j = t - L;
#pragma unroll
    for (int r = 0; r < kWaveRows; ++r) {
      const bool vis = key_ok && (!is_tree || ((mrow[r] >> (j & 63)) & 1ull));
      const float sv = vis ? sacc[r] * a.scale_log2 : -INFINITY;
      const float mnew = fmaxf(m[r], wave_max(sv));
      const float mref = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = exp2f(m[r] - mref);
      const float p = exp2f(sv - mref);
      l[r] = l[r] * alpha + wave_sum(p);
      m[r] = mnew;
      Ps[w][r][lane] = p;
#pragma unroll
      for (int c = 0; c < DC; ++c) o[r][c] *= alpha;
    }
    __syncthreads();
    for (int k = 0; k < kKeys; ++k) {
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const float vk = Vs[k][c * 64 + lane];
#pragma unroll
        for (int r = 0; r < kWaveRows; ++r) o[r][c] = fmaf(Ps[w][r][k], vk, o[r][c]);
      }
    }
  }
  __syncthreads();
  const bool bad = bad_len || bad_page;
  if (bad && tid == 0) raise_error(a.state, TV_ERR_INVALID_ARG);

#pragma unroll
  for (int r = 0; r < kWaveRows; ++r) {
    const int row = rb * kRows + w * kWaveRows + r;
    if (row >= a.rows) continue;
    if (a.S == 1) {
      const int i = row / a.G, h = g * a.G + row % a.G;
      const int64_t base = ((static_cast<int64_t>(b) * a.N + i) * a.Hq + h) * D;
      const float inv = 1.f / l[r];
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const float val = bad ? NAN : o[r][c] * inv;
        if (a.out_bf16)
          static_cast<uint16_t *>(a.out)[base + c * 64 + lane] = float_to_bf16_bits(val);
        else
          static_cast<float *>(a.out)[base + c * 64 + lane] = val;
      }
    } else {
      const int64_t slot = (static_cast<int64_t>(b * a.Hkv + g) * a.S + s) * a.rows_pad + row;
#pragma unroll
      for (int c = 0; c < DC; ++c) a.ws_o[slot * D + c * 64 + lane] = o[r][c];
      if (lane == 0) {
        a.ws_ml[slot * 2] = bad ? NAN : m[r];
        a.ws_ml[slot * 2 + 1] = l[r];
      }
    }
  }
}

// Merges the S partial (m, l, o) triples of each row in a fixed split order.
template <int D>
__global__ void __launch_bounds__(D) attn_combine_kernel(AttnArgs a) {
  const int bh = blockIdx.x / a.rows, row = blockIdx.x % a.rows, d = threadIdx.x;
  const int b = bh / a.Hkv, g = bh % a.Hkv;
  float M = -INFINITY;
  bool bad = false;
  for (int s = 0; s < a.S; ++s) {
    const float ms = a.ws_ml[((static_cast<int64_t>(bh) * a.S + s) * a.rows_pad + row) * 2];
    bad |= isnan(ms);
    M = fmaxf(M, ms);
  }
  float lsum = 0.f, acc = 0.f;
  for (int s = 0; s < a.S; ++s) {
    const int64_t slot = (static_cast<int64_t>(bh) * a.S + s) * a.rows_pad + row;
    const float wgt = exp2f(a.ws_ml[slot * 2] - M);
    lsum = fmaf(wgt, a.ws_ml[slot * 2 + 1], lsum);
    acc = fmaf(wgt, a.ws_o[slot * D + d], acc);
  }
  const float val = bad ? NAN : acc / lsum;
  const int i = row / a.G, h = g * a.G + row % a.G;
  const int64_t idx = ((static_cast<int64_t>(b) * a.N + i) * a.Hq + h) * D + d;
  if (a.out_bf16)
    static_cast<uint16_t *>(a.out)[idx] = float_to_bf16_bits(val);
  else
    static_cast<float *>(a.out)[idx] = val;
}

}  // namespace

AttnPlan plan_attention(int cu_count, int B, int N, int Hq, int Hkv, int D, int max_prefix_len) {
  AttnPlan p{};
  const int G = Hq / Hkv;
  const int rows = G * N;
  p.row_block = kRows;
  p.row_blocks = (rows + kRows - 1) / kRows;
  const int tiles = (max_prefix_len + N + kKeys - 1) / kKeys;
  const int64_t base = static_cast<int64_t>(B) * Hkv * p.row_blocks;
  const int64_t target = 2ll * cu_count;
  int S = static_cast<int>((target + base - 1) / (base > 0 ? base : 1));
  S = S < 1 ? 1 : (S > tiles ? tiles : S);
  if (S < 1) S = 1;
  p.chunk_tiles = (tiles + S - 1) / S;
  if (p.chunk_tiles < 1) p.chunk_tiles = 1;
  p.S = (tiles + p.chunk_tiles - 1) / p.chunk_tiles;
  if (p.S < 1) p.S = 1;
  p.ws_bytes = p.S > 1 ? static_cast<size_t>(B) * Hkv * p.S * p.row_blocks * kRows * (D + 2) * sizeof(float) : 0;
  return p;
}

tv_status launch_attention(tv_ctx *ctx, const AttnPlan &plan, const void *q, const void *k_pages,
                           const void *v_pages, int64_t num_pages, const int32_t *page_table, int maxp,
                           const int32_t *prefix_lens, int max_prefix_len, const uint64_t *tree_mask, int B, int N,
                           int Hq, int Hkv, int D, float sm_scale, void *out, tv_dtype out_dtype, void *workspace) {
  AttnArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k_pages);
  a.v = static_cast<const uint16_t *>(v_pages);
  a.page_table = page_table;
  a.prefix_lens = prefix_lens;
  a.mask = tree_mask;
  a.num_pages = num_pages;
  a.maxp = maxp;
  a.max_prefix_len = max_prefix_len;
  a.B = B;
  a.N = N;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.rows = a.G * N;
  a.rows_pad = plan.row_blocks * kRows;
  a.scale_log2 = sm_scale * kLog2e;
  a.out = out;
  a.out_bf16 = out_dtype == TV_BF16;
  a.S = plan.S;
  a.chunk_tiles = plan.chunk_tiles;
  a.state = ctx->d_state;
  if (plan.S > 1) {
    a.ws_o = static_cast<float *>(workspace);
    a.ws_ml = a.ws_o + static_cast<int64_t>(B) * Hkv * plan.S * a.rows_pad * D;
  }
  const dim3 grid(plan.row_blocks, B * Hkv, plan.S);
  if (D == 128)
    hipLaunchKernelGGL(attn_fma_kernel<128>, grid, dim3(256), 0, ctx->stream, a);
  else
    hipLaunchKernelGGL(attn_fma_kernel<64>, grid, dim3(256), 0, ctx->stream, a);
  if (hipGetLastError() != hipSuccess) return TV_ERR_HIP;
  if (plan.S > 1) {
    const dim3 cgrid(B * Hkv * a.rows);
    if (D == 128)
      hipLaunchKernelGGL(attn_combine_kernel<128>, cgrid, dim3(128), 0, ctx->stream, a);
    else
      hipLaunchKernelGGL(attn_combine_kernel<64>, cgrid, dim3(64), 0, ctx->stream, a);
    if (hipGetLastError() != hipSuccess) return TV_ERR_HIP;
  }
  return TV_OK;
}

}  // namespace tv
