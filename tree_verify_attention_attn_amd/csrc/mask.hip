// mask.hip - ancestor-or-self bitmask builder.
//
// Follows the tree-mask assembly in the EAGLE-2 deep-dive page's reference
// code: row i marks node i and every node on its parent chain. Instead of a
// per-node walk, one wavefront holds one sequence (lane i = node i, N <= 64)
// and uses pointer doubling: after round r a lane knows its ancestors at
// distance < 2^r and its 2^r-th ancestor, so six rounds cover depth 63.
#include "tv_internal.h"

namespace tv {

__global__ void __launch_bounds__(256) build_mask_kernel(const int32_t *__restrict__ parents, int B, int N,
                                                         uint64_t *__restrict__ mask, int32_t *__restrict__ depth,
                                                         unsigned long long *state) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= B) return;
  const bool live = lane < N;
  const int p = live ? parents[static_cast<int64_t>(b) * N + lane] : -1;
  const bool bad = live && (p < -1 || p >= lane);
  const bool any_bad = __ballot(bad) != 0;

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
  if (any_bad && lane == 0) raise_error(state, TV_ERR_INVALID_TREE);
  if (live) {
    const int64_t idx = static_cast<int64_t>(b) * N + lane;
    mask[idx] = any_bad ? 0ull : anc;
    if (depth) depth[idx] = any_bad ? -1 : (__popcll(anc) - 1);
  }
}

tv_status launch_build_mask(tv_ctx *ctx, const int32_t *parents, int B, int N, uint64_t *mask, int32_t *depth) {
  const int blocks = (B + 3) / 4;
  hipLaunchKernelGGL(build_mask_kernel, dim3(blocks), dim3(256), 0, ctx->stream, parents, B, N, mask, depth,
                     ctx->d_state);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

}  // namespace tv
