// mask.hip - ancestor-or-self bitmask builder.
//
// Follows the tree-mask assembly in the EAGLE-2 deep-dive page's reference
// code: row i marks node i and every node on its parent chain. Instead of a
// per-node walk, one wavefront holds one sequence and uses pointer doubling:
// after round r a node knows its ancestors at distance < 2^r and its 2^r-th
// ancestor, so log2(N) rounds cover any depth. Up to 64 nodes, lane i is node
// i and the ancestor set is one 64-bit word; up to 128, lane i holds nodes i
// and i + 64, each with a two-word set. Nodes past the sequence's node count
// are absent: their parents are not read and their rows are written empty.
#include "tv_internal.h"

namespace tv {

namespace {

__device__ inline int size_of(const int32_t *sizes, int b, int N) { return sizes ? sizes[b] : N; }

__global__ void __launch_bounds__(256) build_mask_kernel(const int32_t *__restrict__ parents,
                                                         const int32_t *__restrict__ sizes, int B, int N,
                                                         uint64_t *__restrict__ mask, int32_t *__restrict__ depth,
                                                         unsigned long long *state) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= B) return;
  const int nb = size_of(sizes, b, N);
  const bool bad_size = nb < 1 || nb > N;
  const bool live = !bad_size && lane < nb;
  const int p = live ? parents[static_cast<int64_t>(b) * N + lane] : -1;
  const bool bad = bad_size || __ballot(live && (p < -1 || p >= lane)) != 0;

  unsigned long long anc = live ? (1ull << lane) : 0ull;
  int jump = (live && !bad) ? p : -1;
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
  if (bad && lane == 0) raise_error(state, bad_size ? TV_ERR_INVALID_ARG : TV_ERR_INVALID_TREE);
  if (lane < N) {
    const int64_t idx = static_cast<int64_t>(b) * N + lane;
    mask[idx] = (bad || !live) ? 0ull : anc;
    if (depth) depth[idx] = (bad || !live) ? -1 : (__popcll(anc) - 1);
  }
}

// 64 < N <= 128: lane i holds nodes i (half 0) and i + 64 (half 1)
__global__ void __launch_bounds__(256) build_mask128_kernel(const int32_t *__restrict__ parents,
                                                            const int32_t *__restrict__ sizes, int B, int N,
                                                            uint64_t *__restrict__ mask, int32_t *__restrict__ depth,
                                                            unsigned long long *state) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= B) return;
  const int nb = size_of(sizes, b, N);
  const bool bad_size = nb < 1 || nb > N;
  bool live[2], bad_any = bad_size;
  int jump[2];
  unsigned long long lo[2], hi[2];  // ancestor set: nodes 0..63 in lo, 64..127 in hi
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = lane + 64 * k;
    live[k] = !bad_size && i < nb;
    const int p = live[k] ? parents[static_cast<int64_t>(b) * N + i] : -1;
    bad_any |= live[k] && (p < -1 || p >= i);
    jump[k] = live[k] ? p : -1;
    lo[k] = live[k] && k == 0 ? (1ull << lane) : 0ull;
    hi[k] = live[k] && k == 1 ? (1ull << lane) : 0ull;
  }
  const bool bad = __ballot(bad_any) != 0;
  if (bad) jump[0] = jump[1] = -1;
#pragma unroll
  for (int r = 0; r < 7; ++r) {
    unsigned long long nlo[2], nhi[2];
    int nj[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      // the values of node jump[k], which lane jump % 64 holds in half jump / 64
      const int j = jump[k] >= 0 ? jump[k] : lane + 64 * k;
      const int src = j & 63;
      const unsigned long long lo0 = shfl_u64(lo[0], src), lo1 = shfl_u64(lo[1], src);
      const unsigned long long hi0 = shfl_u64(hi[0], src), hi1 = shfl_u64(hi[1], src);
      const int j0 = __shfl(jump[0], src), j1 = __shfl(jump[1], src);
      const bool upper = j >= 64;
      nlo[k] = lo[k];
      nhi[k] = hi[k];
      nj[k] = jump[k];
      if (jump[k] >= 0) {
        nlo[k] |= upper ? lo1 : lo0;
        nhi[k] |= upper ? hi1 : hi0;
        nj[k] = upper ? j1 : j0;
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      lo[k] = nlo[k];
      hi[k] = nhi[k];
      jump[k] = nj[k];
    }
  }
  if (bad && lane == 0) raise_error(state, bad_size ? TV_ERR_INVALID_ARG : TV_ERR_INVALID_TREE);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = lane + 64 * k;
    if (i < N) {
      const int64_t idx = static_cast<int64_t>(b) * N + i;
      const bool ok = !bad && live[k];
      mask[2 * idx] = ok ? lo[k] : 0ull;
      mask[2 * idx + 1] = ok ? hi[k] : 0ull;
      if (depth) depth[idx] = ok ? (__popcll(lo[k]) + __popcll(hi[k]) - 1) : -1;
    }
  }
}

}  // namespace

tv_status launch_build_mask(tv_ctx *ctx, const int32_t *parents, const int32_t *tree_sizes, int B, int N,
                            uint64_t *mask, int32_t *depth) {
  const int blocks = (B + 3) / 4;
  if (N <= 64)
    hipLaunchKernelGGL(build_mask_kernel, dim3(blocks), dim3(256), 0, ctx->stream, parents, tree_sizes, B, N, mask,
                       depth, ctx->d_state);
  else
    hipLaunchKernelGGL(build_mask128_kernel, dim3(blocks), dim3(256), 0, ctx->stream, parents, tree_sizes, B, N,
                       mask, depth, ctx->d_state);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

}  // namespace tv
