// tv_internal.h - shared internals of libtreeverify (device code for gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/treeverify.h"

struct tv_ctx {
  int device;
  hipStream_t stream;
  int cu_count;
  // d_state[0] = tau sum, d_state[1] = tau cycles, d_state[2] low 32 bits = sticky error code
  unsigned long long *d_state;
  // resident workgroups per CU of the stochastic path pass (0 = not yet
  // queried, -1 = query failed)
  int path_blocks_per_cu;
  // per-sequence arrival counters of the one-launch greedy acceptance
  // (tv::kMaxFusedSeqs words, zero between calls)
  unsigned int *d_arrivals;
  // recorded on the old stream when the context is rebound, so that calls on
  // the new stream start after the work already queued
  hipEvent_t rebind_event;
  // device address of tv_attention_noalloc's scratch on this context's device
  void *scratch;
};

namespace tv {

constexpr int kPage = 16;
constexpr int kMaxPrefix = 1 << 30;  // largest max_prefix_len: token positions and key counts stay in int32
constexpr int kMaxFusedSeqs = 65536;  // sequences with an arrival counter for one-launch greedy acceptance

// Records the first device-detected error of a context (later ones are dropped).
__device__ inline void raise_error(unsigned long long *state, int code) {
  atomicCAS(reinterpret_cast<int *>(state + 2), 0, code);
}

__device__ inline float bf16_bits_to_float(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

__device__ inline uint16_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return static_cast<uint16_t>((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ inline unsigned long long shfl_u64(unsigned long long v, int src) {
  int lo = __shfl(static_cast<int>(v & 0xFFFFFFFFull), src);
  int hi = __shfl(static_cast<int>(v >> 32), src);
  return (static_cast<unsigned long long>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

__device__ inline unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  int lo = __shfl_xor(static_cast<int>(v & 0xFFFFFFFFull), m);
  int hi = __shfl_xor(static_cast<int>(v >> 32), m);
  return (static_cast<unsigned long long>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

__device__ inline float wave_max(float v) {
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

__device__ inline float wave_sum(float v) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// Host-side launchers (defined in the kernels' translation units).
tv_status launch_build_mask(tv_ctx *ctx, const int32_t *parents, const int32_t *tree_sizes, int B, int N,
                            uint64_t *mask, int32_t *depth);

struct AttnPlan {
  int S;            // key splits per (sequence, KV head, row block)
  int chunk_tiles;  // 64-key tiles per split
  int qb;           // wavefronts per workgroup (32 query rows each): 2, 4 or 8
  int ksplit;       // 1: two wavefronts share one 32-row block and split its tiles
  int row_block;    // query rows (node, head-in-group) per workgroup
  int row_blocks;   // ceil(G*N / row_block)
  int order;        // 1: workgroups take (sequence, KV head) units longest first (order in the workspace)
  int nt;           // 1: K/V loads non-temporal (the K/V stream exceeds the Infinity Cache)
  size_t ws_bytes;  // fp32 partials + (m, l), or the unit order
};
AttnPlan plan_attention(int cu_count, int B, int N, int Hq, int Hkv, int D, int max_prefix_len);
tv_status launch_attention(tv_ctx *ctx, const AttnPlan &plan, const void *q, const void *k_pages,
                           const void *v_pages, int64_t num_pages, const int32_t *page_table, int maxp,
                           const int32_t *prefix_lens, int max_prefix_len, const uint64_t *tree_mask,
                           const int32_t *tree_sizes, int B, int N, int Hq, int Hkv, int D, float sm_scale, void *out,
                           tv_dtype out_dtype, void *workspace);

size_t accept_ws_bytes(int B, int N, int V, tv_accept_mode mode);
tv_status launch_accept(tv_ctx *ctx, const float *target_logits, const float *draft_logits,
                        const int32_t *draft_tokens, const int32_t *parents, const int32_t *tree_sizes,
                        const float *uniforms, int B, int N, int V, tv_accept_mode mode, float temperature,
                        int32_t *accept_len, int32_t *path, int32_t *bonus, int32_t *target_argmax,
                        void *workspace);

tv_status launch_commit(tv_ctx *ctx, void *k_pages, void *v_pages, int64_t num_pages, const int32_t *page_table,
                        int maxp, const int32_t *prefix_lens, int max_prefix_len, const int32_t *draft_tokens,
                        const int32_t *path, const int32_t *accept_len, const int32_t *bonus, int B, int N, int Hkv,
                        int D, int32_t *new_prefix_lens, int32_t *emitted, int32_t *next_root);

tv_status launch_build_tree(tv_ctx *ctx, const int32_t *root_tokens, const int32_t *cand_tokens,
                            const float *cand_probs, int B, int N, int k, int k_root, float threshold, int max_depth,
                            int32_t *parents, int32_t *tokens, int32_t *depth, uint64_t *mask, double *scores,
                            int32_t *n_nodes);

tv_status launch_clear_state(tv_ctx *ctx, int first_word, int n_words);

}  // namespace tv
