// api.hip - the C ABI of libtreeverify: argument checks, planning, launches.
// Host-detected errors return before anything is launched.
#include <math.h>
#include <stdlib.h>

#include <mutex>

#include "tv_internal.h"

namespace tv {

namespace {

__global__ void clear_words_kernel(unsigned long long *p, int n) {
  if (static_cast<int>(threadIdx.x) < n) p[threadIdx.x] = 0ull;
}

__global__ void clear_u32_kernel(unsigned int *p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

}  // namespace

// Scratch of tv_attention_noalloc: split partials or the unit order of the
// attention plan, for callers that cannot allocate. The array is a device
// global of the code object, so each GPU holds its own copy at its own
// address from the module's load until the process ends; host code uses the
// per-device address that hipGetSymbolAddress returns, never the array's
// name. Every tv_attention_noalloc call on a device shares it.
static __device__ __align__(256) unsigned char scratch[TV_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` on each device, or null
}  // namespace

// The device address of `scratch` on `device` (which must be current),
// looked up once per device; null if the lookup fails.
void *scratch_address(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[device]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[device] = p;
  }
  return g_scratch[device];
}

tv_status launch_clear_state(tv_ctx *ctx, int first_word, int n_words) {
  hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(64), 0, ctx->stream, ctx->d_state + first_word, n_words);
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

}  // namespace tv

using namespace tv;

extern "C" {

tv_status tv_create(tv_ctx **out, int device, void *hip_stream) {
  if (!out) return TV_ERR_INVALID_ARG;
  *out = nullptr;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) return TV_ERR_INVALID_ARG;
  if (hipSetDevice(device) != hipSuccess) return TV_ERR_HIP;
  tv_ctx *ctx = static_cast<tv_ctx *>(calloc(1, sizeof(tv_ctx)));
  if (!ctx) return TV_ERR_HIP;
  ctx->device = device;
  ctx->stream = static_cast<hipStream_t>(hip_stream);
  auto fail = [&]() {
    if (ctx->d_state) (void)hipFree(ctx->d_state);
    if (ctx->d_arrivals) (void)hipFree(ctx->d_arrivals);
    if (ctx->rebind_event) (void)hipEventDestroy(ctx->rebind_event);
    free(ctx);
    return TV_ERR_HIP;
  };
  if (hipDeviceGetAttribute(&ctx->cu_count, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      hipMalloc(reinterpret_cast<void **>(&ctx->d_state), 64) != hipSuccess ||
      hipMalloc(reinterpret_cast<void **>(&ctx->d_arrivals), kMaxFusedSeqs * sizeof(unsigned int)) != hipSuccess ||
      hipEventCreateWithFlags(&ctx->rebind_event, hipEventDisableTiming) != hipSuccess)
    return fail();
  // the no-allocation entry point's scratch on this device (its address is
  // looked up here, at set-up, with the device current)
  ctx->scratch = scratch_address(device);
  if (!ctx->scratch) return fail();
  hipLaunchKernelGGL(clear_u32_kernel, dim3(64), dim3(256), 0, ctx->stream, ctx->d_arrivals, kMaxFusedSeqs);
  if (hipGetLastError() != hipSuccess || launch_clear_state(ctx, 0, 8) != TV_OK ||
      hipStreamSynchronize(ctx->stream) != hipSuccess)
    return fail();
  *out = ctx;
  return TV_OK;
}

tv_status tv_destroy(tv_ctx *ctx) {
  if (!ctx) return TV_ERR_INVALID_ARG;
  (void)hipSetDevice(ctx->device);
  (void)hipStreamSynchronize(ctx->stream);
  (void)hipFree(ctx->d_state);
  (void)hipFree(ctx->d_arrivals);
  (void)hipEventDestroy(ctx->rebind_event);
  free(ctx);
  return TV_OK;
}

tv_status tv_set_stream(tv_ctx *ctx, void *hip_stream) {
  if (!ctx) return TV_ERR_INVALID_ARG;
  const hipStream_t next = static_cast<hipStream_t>(hip_stream);
  if (next != ctx->stream) {
    // the context's device counters are shared by its calls: calls on the
    // new stream wait for what is already queued on the old one
    if (hipEventRecord(ctx->rebind_event, ctx->stream) != hipSuccess ||
        hipStreamWaitEvent(next, ctx->rebind_event, 0) != hipSuccess)
      return TV_ERR_HIP;
    ctx->stream = next;
  }
  return TV_OK;
}

tv_status tv_build_mask(tv_ctx *ctx, const int32_t *parents, const int32_t *tree_sizes, int32_t B, int32_t N,
                        uint64_t *mask, int32_t *depth) {
  if (!ctx || B < 0 || N < 0) return TV_ERR_INVALID_ARG;
  if (N > 128) return TV_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(B) * N == 0) return TV_OK;
  if (!parents || !mask) return TV_ERR_INVALID_ARG;
  return launch_build_mask(ctx, parents, tree_sizes, B, N, mask, depth);
}

size_t tv_attention_workspace_bytes(tv_ctx *ctx, int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t max_prefix_len) {
  if (!ctx || B <= 0 || N <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_prefix_len < 0) return 0;
  if (N > 128 || max_prefix_len > kMaxPrefix) return 0;
  return plan_attention(ctx->cu_count, B, N, Hq, Hkv, D, max_prefix_len).ws_bytes;
}

tv_status tv_attention(tv_ctx *ctx, const void *q, const void *k_pages, const void *v_pages, int64_t num_pages,
                       const int32_t *page_table, int32_t maxp, const int32_t *prefix_lens, int32_t max_prefix_len,
                       const uint64_t *tree_mask, const int32_t *tree_sizes, int32_t B, int32_t N, int32_t Hq,
                       int32_t Hkv, int32_t D, float sm_scale, void *out, tv_dtype out_dtype, void *workspace,
                       size_t workspace_bytes) {
  if (!ctx || B < 0 || N < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || num_pages < 0 || maxp < 0 || max_prefix_len < 0)
    return TV_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return TV_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return TV_ERR_UNSUPPORTED;
  if (N > 128 || max_prefix_len > kMaxPrefix) return TV_ERR_UNSUPPORTED;
  if (!isfinite(sm_scale)) return TV_ERR_INVALID_ARG;
  if (out_dtype != TV_F32 && out_dtype != TV_BF16) return TV_ERR_INVALID_ARG;
  if (static_cast<int64_t>(B) * N == 0) return TV_OK;
  if (static_cast<int64_t>(maxp) * kPage < static_cast<int64_t>(max_prefix_len) + N) return TV_ERR_INVALID_ARG;
  if (!q || !k_pages || !v_pages || !page_table || !prefix_lens || !out) return TV_ERR_INVALID_ARG;
  const AttnPlan plan = plan_attention(ctx->cu_count, B, N, Hq, Hkv, D, max_prefix_len);
  // one workgroup per (b, g, row group, split) on a 1-D grid of int32 block ids
  if (static_cast<int64_t>(B) * Hkv * plan.row_blocks * plan.S > 0x7FFFFFFF) return TV_ERR_UNSUPPORTED;
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes)) return TV_ERR_WORKSPACE;
  return launch_attention(ctx, plan, q, k_pages, v_pages, num_pages, page_table, maxp, prefix_lens, max_prefix_len,
                          tree_mask, tree_sizes, B, N, Hq, Hkv, D, sm_scale, out, out_dtype, workspace);
}

tv_status tv_attention_noalloc(tv_ctx *ctx, const void *q, const void *k_pages, const void *v_pages,
                               int64_t num_pages, const int32_t *page_table, int32_t maxp,
                               const int32_t *prefix_lens, int32_t max_prefix_len, const uint64_t *tree_mask,
                               const int32_t *tree_sizes, int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                               float sm_scale, void *out, tv_dtype out_dtype) {
  if (!ctx || !ctx->scratch) return TV_ERR_INVALID_ARG;
  if (B < 0 || N < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_prefix_len < 0) return TV_ERR_INVALID_ARG;
  if (N <= 128 && max_prefix_len <= kMaxPrefix && static_cast<int64_t>(B) * N > 0) {
    const AttnPlan plan = plan_attention(ctx->cu_count, B, N, Hq, Hkv, D, max_prefix_len);
    if (plan.ws_bytes > TV_NOALLOC_SCRATCH_BYTES) return TV_ERR_WORKSPACE;
  }
  // the same checks, plan and kernels as tv_attention, with the device's
  // scratch as the workspace
  return tv_attention(ctx, q, k_pages, v_pages, num_pages, page_table, maxp, prefix_lens, max_prefix_len, tree_mask,
                      tree_sizes, B, N, Hq, Hkv, D, sm_scale, out, out_dtype, ctx->scratch,
                      TV_NOALLOC_SCRATCH_BYTES);
}

size_t tv_accept_workspace_bytes(int32_t B, int32_t N, int32_t V, tv_accept_mode mode) {
  if (B <= 0 || N <= 0 || V <= 0 || (mode != TV_GREEDY && mode != TV_STOCHASTIC)) return 0;
  return accept_ws_bytes(B, N, V, mode);
}

tv_status tv_accept(tv_ctx *ctx, const float *target_logits, const float *draft_logits, const int32_t *draft_tokens,
                    const int32_t *parents, const int32_t *tree_sizes, const float *uniforms, int32_t B, int32_t N,
                    int32_t V,
                    tv_accept_mode mode, float temperature, int32_t *accept_len, int32_t *path, int32_t *bonus_token,
                    int32_t *target_argmax, void *workspace, size_t workspace_bytes) {
  if (!ctx || B < 0 || V <= 0) return TV_ERR_INVALID_ARG;
  if (mode != TV_GREEDY && mode != TV_STOCHASTIC) return TV_ERR_INVALID_ARG;
  if (mode == TV_STOCHASTIC && (!(temperature > 0.0f) || !isfinite(temperature))) return TV_ERR_INVALID_ARG;
  if (B == 0) return TV_OK;
  if (N < 1) return TV_ERR_INVALID_ARG;
  if (N > 128) return TV_ERR_UNSUPPORTED;
  if (!target_logits || !draft_tokens || !parents || !accept_len || !path || !bonus_token) return TV_ERR_INVALID_ARG;
  if (mode == TV_STOCHASTIC && (!draft_logits || !uniforms)) return TV_ERR_INVALID_ARG;
  // one workgroup of 256 threads per (row, chunk) on a 1-D grid; a chunk is
  // 16384 tokens for the greedy argmax, 8192 for the stochastic statistics
  const int64_t chunk = mode == TV_GREEDY ? 16384 : 8192;
  if (static_cast<int64_t>(B) * N * ((static_cast<int64_t>(V) + chunk - 1) / chunk) * 256 > 0xFFFFFFFFLL)
    return TV_ERR_UNSUPPORTED;
  // the stochastic path pass: at least one 512-thread workgroup per sequence
  if (mode == TV_STOCHASTIC && static_cast<int64_t>(B) * 512 > 0xFFFFFFFFLL) return TV_ERR_UNSUPPORTED;
  const size_t need = accept_ws_bytes(B, N, V, mode);
  if (!workspace || workspace_bytes < need) return TV_ERR_WORKSPACE;
  return launch_accept(ctx, target_logits, draft_logits, draft_tokens, parents, tree_sizes, uniforms, B, N, V, mode,
                       temperature, accept_len, path, bonus_token, mode == TV_GREEDY ? target_argmax : nullptr,
                       workspace);
}

tv_status tv_commit(tv_ctx *ctx, void *k_pages, void *v_pages, int64_t num_pages, const int32_t *page_table,
                    int32_t maxp, const int32_t *prefix_lens, int32_t max_prefix_len, const int32_t *draft_tokens,
                    const int32_t *path, const int32_t *accept_len, const int32_t *bonus_token, int32_t B, int32_t N,
                    int32_t Hkv, int32_t D, int32_t *new_prefix_lens, int32_t *emitted, int32_t *next_root) {
  if (!ctx || B < 0 || Hkv <= 0 || num_pages < 0 || maxp < 0 || max_prefix_len < 0) return TV_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return TV_ERR_UNSUPPORTED;
  if (B == 0) return TV_OK;
  if (N < 1) return TV_ERR_INVALID_ARG;
  if (N > 128 || max_prefix_len > kMaxPrefix) return TV_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(B) * Hkv > 0x7FFFFFFF) return TV_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(maxp) * kPage < static_cast<int64_t>(max_prefix_len) + N) return TV_ERR_INVALID_ARG;
  if (!k_pages || !v_pages || !page_table || !prefix_lens || !draft_tokens || !path || !accept_len || !bonus_token ||
      !new_prefix_lens || !next_root)
    return TV_ERR_INVALID_ARG;
  return launch_commit(ctx, k_pages, v_pages, num_pages, page_table, maxp, prefix_lens, max_prefix_len, draft_tokens,
                       path, accept_len, bonus_token, B, N, Hkv, D, new_prefix_lens, emitted, next_root);
}

tv_status tv_build_tree(tv_ctx *ctx, const int32_t *root_tokens, const int32_t *cand_tokens, const float *cand_probs,
                        int32_t B, int32_t N, int32_t k, int32_t k_root, float threshold, int32_t max_depth,
                        int32_t *parents, int32_t *tokens, int32_t *depth, uint64_t *mask, double *scores,
                        int32_t *n_nodes) {
  if (!ctx || B < 0 || k < 1 || k_root < 1 || k_root > k || max_depth < 1 || isnan(threshold))
    return TV_ERR_INVALID_ARG;
  if (k > 32) return TV_ERR_UNSUPPORTED;
  if (B == 0) return TV_OK;
  if (N < 1) return TV_ERR_INVALID_ARG;
  if (N > 128) return TV_ERR_UNSUPPORTED;
  if (!root_tokens || !cand_tokens || !cand_probs || !parents || !tokens) return TV_ERR_INVALID_ARG;
  return launch_build_tree(ctx, root_tokens, cand_tokens, cand_probs, B, N, k, k_root, threshold, max_depth, parents,
                           tokens, depth, mask, scores, n_nodes);
}

tv_status tv_tau(tv_ctx *ctx, double *tau, uint64_t *cycles) {
  if (!ctx || !tau) return TV_ERR_INVALID_ARG;
  unsigned long long h[2] = {0, 0};
  if (hipMemcpyAsync(h, ctx->d_state, sizeof(h), hipMemcpyDeviceToHost, ctx->stream) != hipSuccess ||
      hipStreamSynchronize(ctx->stream) != hipSuccess)
    return TV_ERR_HIP;
  *tau = h[1] ? static_cast<double>(h[0]) / static_cast<double>(h[1]) : 0.0;
  if (cycles) *cycles = h[1];
  return TV_OK;
}

tv_status tv_tau_reset(tv_ctx *ctx) {
  if (!ctx) return TV_ERR_INVALID_ARG;
  return launch_clear_state(ctx, 0, 2);
}

tv_status tv_device_error(tv_ctx *ctx, int32_t *code) {
  if (!ctx || !code) return TV_ERR_INVALID_ARG;
  unsigned long long h = 0;
  if (hipMemcpyAsync(&h, ctx->d_state + 2, sizeof(h), hipMemcpyDeviceToHost, ctx->stream) != hipSuccess ||
      hipStreamSynchronize(ctx->stream) != hipSuccess)
    return TV_ERR_HIP;
  *code = static_cast<int32_t>(h & 0xFFFFFFFFull);
  if (launch_clear_state(ctx, 2, 1) != TV_OK || hipStreamSynchronize(ctx->stream) != hipSuccess) return TV_ERR_HIP;
  return TV_OK;
}

int32_t tv_tree_budget(int32_t concurrency, int32_t max_nodes) {
  if (concurrency < 0 || max_nodes < 1 || max_nodes > 128) return -1;
  int32_t n = max_nodes;
  if (concurrency > 64)
    n = 1;
  else if (concurrency > 48)
    n = max_nodes / 4;
  else if (concurrency > 32)
    n = max_nodes / 2;
  return n < 1 ? 1 : n;
}

const char *tv_status_string(tv_status s) {
  switch (s) {
    case TV_OK: return "ok";
    case TV_ERR_INVALID_ARG: return "invalid argument";
    case TV_ERR_INVALID_TREE: return "invalid tree (parent not earlier than its child, or rooted root)";
    case TV_ERR_UNSUPPORTED: return "unsupported shape or mode";
    case TV_ERR_WORKSPACE: return "workspace missing or too small";
    case TV_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

}  // extern "C"
