// tree.hip - dynamic draft-tree construction on the device.
//
// EAGLE-2 deep-dive page, dynamic-tree algorithm and its reference code's
// builder: a node's cumulative score is the product of the draft
// probabilities on its root path; the queue starts with the root's top-k
// proposals; the highest-scoring candidate becomes the next node (equal
// scores: the one queued first); a node shallower than the depth limit
// queues its top-k children whose cumulative score is above the threshold
// (the reference code's strict test); construction stops at the node budget,
// root included, or when the queue is empty. The tree is emitted with its
// ancestor masks, ready for the attention call.
//
// One wavefront per sequence. The sequence's proposal table (row i: what the
// draft head proposes for the node created i-th, at most 128 x 32 entries) is
// copied into LDS first, so every pop is LDS and register work: a
// lane-strided scan of the candidate pool (four loads in flight per lane) for
// each lane's best (score, queue position), a wavefront maximum of those pairs moved with DPP row shifts and
// broadcasts, and the new node's fields kept by lane node % 64, half
// node / 64 (parent, token, depth, score, two-word ancestor set). Accepted
// children are appended in slot order through a ballot prefix, which keeps
// the queue order of the definition.
#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kMaxK = 32;
constexpr int kMaxN = 128;
constexpr int kMaxPool = kMaxK + (kMaxN - 1) * kMaxK;  // root proposals + k per other node

// (score, position) of the better candidate: higher score, then the one
// queued first
__device__ inline bool better(double os, int oj, double s, int j) { return os > s || (os == s && oj < j); }

// one step of the wavefront maximum over (score, position), moving values
// with DPP; lanes without a source in this pattern keep their own pair
template <int kCtrl, int kRowMask>
__device__ inline void best_step(double &s, int &j) {
  const int hi = __builtin_amdgcn_update_dpp(__double2hiint(s), __double2hiint(s), kCtrl, kRowMask, 0xF, false);
  const int lo = __builtin_amdgcn_update_dpp(__double2loint(s), __double2loint(s), kCtrl, kRowMask, 0xF, false);
  const int oj = __builtin_amdgcn_update_dpp(j, j, kCtrl, kRowMask, 0xF, false);
  const double os = __hiloint2double(hi, lo);
  if (better(os, oj, s, j)) {
    s = os;
    j = oj;
  }
}

__device__ inline uint64_t read_lane_u64(uint64_t v, int l) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v & 0xFFFFFFFFull), l));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), l));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// the best (score, position) of the wavefront, returned to every lane:
// prefix maxima within each row of 16 lanes (row_shr 1, 2, 4, 8), then
// across rows (row_bcast 15 and 31) into lane 63, then read back
__device__ inline void wave_best(double &s, int &j) {
  best_step<0x111, 0xF>(s, j);
  best_step<0x112, 0xF>(s, j);
  best_step<0x114, 0xF>(s, j);
  best_step<0x118, 0xF>(s, j);
  best_step<0x142, 0xA>(s, j);
  best_step<0x143, 0xC>(s, j);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(s), 63);
  const int lo = __builtin_amdgcn_readlane(__double2loint(s), 63);
  j = __builtin_amdgcn_readlane(j, 63);
  s = __hiloint2double(hi, lo);
}

__global__ void __launch_bounds__(64) build_tree_kernel(const int32_t *__restrict__ root_tokens,
                                                        const int32_t *__restrict__ cand_tokens,
                                                        const float *__restrict__ cand_probs, int N, int k, int k_root,
                                                        double threshold, int max_depth, int32_t *__restrict__ parents,
                                                        int32_t *__restrict__ tokens, int32_t *__restrict__ depth,
                                                        uint64_t *__restrict__ mask, double *__restrict__ scores,
                                                        int32_t *__restrict__ n_nodes,
                                                        unsigned long long *state) {
  __shared__ float s_prob[kMaxN * kMaxK];
  __shared__ int32_t s_tok[kMaxN * kMaxK];
  __shared__ double s_score[kMaxPool];  // queued candidates; -1 once made a node
  __shared__ int16_t s_src[kMaxPool];   // proposer row * 32 + slot
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t rows = static_cast<int64_t>(N) * k;
  const int32_t *ct = cand_tokens + b * rows;
  const float *cp = cand_probs + b * rows;
  bool bad = false;
  for (int j = lane; j < rows; j += 64) {
    const float p = cp[j];
    bad |= !(p >= 0.0f);  // NaN or negative
    s_prob[(j / k) * kMaxK + j % k] = p;
    s_tok[(j / k) * kMaxK + j % k] = ct[j];
  }
  bad = __builtin_amdgcn_ballot_w64(bad) != 0;
  const int root_tok = root_tokens[b];
  __syncthreads();

  // lane i holds nodes i (half 0) and i + 64 (half 1): parent, token,
  // depth, cumulative score, ancestor set (nodes 0..63 in word 0, 64..127 in
  // word 1)
  int my_parent[2] = {-1, -1}, my_token[2] = {root_tok, root_tok}, my_depth[2] = {0, 0};
  double my_score[2] = {lane == 0 ? 1.0 : 0.0, 0.0};
  uint64_t my_m0[2] = {1ull << lane, 0ull}, my_m1[2] = {0ull, 1ull << lane};
  int n = 0;
  if (!bad) {
    n = 1;
    int q = 0;  // pool size
    for (int s = lane; s < k_root; s += 64) {  // the root's proposals are queued unconditionally
      s_score[s] = static_cast<double>(s_prob[s]);
      s_src[s] = static_cast<int16_t>(s);
    }
    q = k_root;
    __syncthreads();
    while (n < N) {
      // best alive candidate: highest score, earliest queued on ties
      double bs = -1.0;
      int bj = 0x7FFFFFFF;
      for (int j0 = lane; j0 < q; j0 += 64 * 4) {
        double sc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) sc[u] = j0 + 64 * u < q ? s_score[j0 + 64 * u] : -2.0;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (sc[u] > bs) {  // positions increase, so '>' keeps the earliest
            bs = sc[u];
            bj = j0 + 64 * u;
          }
      }
      wave_best(bs, bj);
      if (bs < 0.0) break;  // queue empty
      const int src = s_src[bj];
      const int row = src >> 5, slot = src & 31;
      const int id = n++;
      // the parent's fields, from the lane and half that hold it (the same
      // for every lane)
      const int ph = row >> 6, pl = row & 63;
      const int pdepth = __builtin_amdgcn_readlane(ph ? my_depth[1] : my_depth[0], pl);
      const uint64_t pm0 = read_lane_u64(ph ? my_m0[1] : my_m0[0], pl);
      const uint64_t pm1 = read_lane_u64(ph ? my_m1[1] : my_m1[0], pl);
      __syncthreads();  // every lane has read s_score[bj] before it is retired
      if (lane == 0) s_score[bj] = -1.0;
      if (lane == (id & 63)) {
        const int hh = id >> 6;
        my_parent[hh] = row;
        my_token[hh] = s_tok[row * kMaxK + slot];
        my_depth[hh] = pdepth + 1;
        my_score[hh] = bs;
        my_m0[hh] = pm0 | (hh == 0 ? (1ull << lane) : 0ull);
        my_m1[hh] = pm1 | (hh == 1 ? (1ull << lane) : 0ull);
      }
      if (pdepth + 1 < max_depth) {
        // the new node's proposals above the threshold, in slot order
        double c = 0.0;
        bool take = false;
        if (lane < k) {
          c = bs * static_cast<double>(s_prob[id * kMaxK + lane]);
          take = c > threshold;
        }
        const uint64_t tk = __builtin_amdgcn_ballot_w64(take);
        if (take) {
          const int at = q + __popcll(tk & ((1ull << lane) - 1ull));
          s_score[at] = c;
          s_src[at] = static_cast<int16_t>(id * 32 + lane);
        }
        q += __popcll(tk);
      }
      __syncthreads();
    }
  }
  const int W = (N + 63) / 64;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int i = lane + 64 * hh;
    if (i < N) {
      const int64_t o = static_cast<int64_t>(b) * N + i;
      const bool live = i < n;
      parents[o] = live ? my_parent[hh] : -1;
      tokens[o] = live ? my_token[hh] : root_tok;
      if (depth) depth[o] = live ? my_depth[hh] : 0;
      if (mask) {
        mask[o * W] = live ? my_m0[hh] : (hh == 0 ? (1ull << lane) : 0ull);
        if (W > 1) mask[o * W + 1] = live ? my_m1[hh] : (hh == 1 ? (1ull << lane) : 0ull);
      }
      if (scores) scores[o] = live ? my_score[hh] : 0.0;
    }
  }
  if (lane == 0) {
    if (n_nodes) n_nodes[b] = n;
    if (bad) raise_error(state, TV_ERR_INVALID_ARG);
  }
}

}  // namespace

tv_status launch_build_tree(tv_ctx *ctx, const int32_t *root_tokens, const int32_t *cand_tokens,
                            const float *cand_probs, int B, int N, int k, int k_root, float threshold, int max_depth,
                            int32_t *parents, int32_t *tokens, int32_t *depth, uint64_t *mask, double *scores,
                            int32_t *n_nodes) {
  hipLaunchKernelGGL(build_tree_kernel, dim3(B), dim3(64), 0, ctx->stream, root_tokens, cand_tokens, cand_probs, N, k,
                     k_root, static_cast<double>(threshold), max_depth, parents, tokens, depth, mask, scores, n_nodes,
                     ctx->d_state);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

}  // namespace tv
