/* c_caller.c - one verification cycle driven from plain C through the
 * library's C ABI, with no Python in the process: tv_build_mask, tv_attention,
 * tv_accept (greedy, or sampled when a temperature is given) and tv_commit on
 * device 0, then tv_tau and tv_device_error.
 *
 * Usage: c_caller DIR
 *   DIR/shape.txt  "B N Hq Hkv D num_pages maxp max_prefix_len V sm_scale [temperature]"
 *   DIR/q.bin      bf16 bits [B][N][Hq][D]        DIR/k.bin, v.bin  bf16 bits [num_pages][Hkv][16][D]
 *   DIR/table.bin  int32 [B][maxp]                DIR/plens.bin     int32 [B]
 *   DIR/parents.bin, tokens.bin  int32 [B][N]     DIR/logits.bin    fp32 [B][N][V]
 *   with a temperature also DIR/draft.bin fp32 [B][N][V] and DIR/uniforms.bin fp32 [B][N]
 * Writes DIR/mask.bin (uint64 [B][N][W]), depth.bin, out.bin (fp32
 * [B][N][Hq][D]), accept_len.bin, path.bin, bonus.bin, argmax.bin (greedy
 * only), then, after the commit, k_new.bin, v_new.bin (the pools),
 * new_lens.bin, emitted.bin and next_root.bin, and prints "tau T cycles C
 * device_error E". Exits non-zero on any failed call. Test infrastructure:
 * the GPU tests run it and compare its files with the oracle. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "treeverify.h"

static const char *g_dir;

static void fail(const char *what, const char *why) {
  fprintf(stderr, "c_caller: %s: %s\n", what, why);
  exit(1);
}

#define HIP_CHECK(x)                                          \
  do {                                                        \
    hipError_t e_ = (x);                                      \
    if (e_ != hipSuccess) fail(#x, hipGetErrorString(e_));    \
  } while (0)
#define TV_CHECK(x)                                           \
  do {                                                        \
    tv_status s_ = (x);                                       \
    if (s_ != TV_OK) fail(#x, tv_status_string(s_));          \
  } while (0)

/* Reads DIR/name, which must hold exactly `bytes` bytes, into device memory. */
static void *upload(const char *name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) fail(path, "cannot open");
  void *h = malloc(bytes ? bytes : 1);
  if (!h) fail(path, "out of host memory");
  if (fread(h, 1, bytes, f) != bytes || fgetc(f) != EOF) fail(path, "size differs from the shape");
  fclose(f);
  void *d = NULL;
  HIP_CHECK(hipMalloc(&d, bytes ? bytes : 1));
  HIP_CHECK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  free(h);
  return d;
}

static void *device_buffer(size_t bytes) {
  void *d = NULL;
  HIP_CHECK(hipMalloc(&d, bytes ? bytes : 1));
  return d;
}

static void download(const char *name, const void *d, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  void *h = malloc(bytes ? bytes : 1);
  if (!h) fail(path, "out of host memory");
  HIP_CHECK(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
  FILE *f = fopen(path, "wb");
  if (!f || fwrite(h, 1, bytes, f) != bytes || fclose(f) != 0) fail(path, "cannot write");
  free(h);
}

int main(int argc, char **argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: c_caller DIR\n");
    return 2;
  }
  g_dir = argv[1];
  char path[4096];
  snprintf(path, sizeof path, "%s/shape.txt", g_dir);
  FILE *f = fopen(path, "r");
  if (!f) fail(path, "cannot open");
  int B, N, Hq, Hkv, D, maxp, max_prefix_len, V;
  long long num_pages;
  float sm_scale;
  if (fscanf(f, "%d %d %d %d %d %lld %d %d %d %f", &B, &N, &Hq, &Hkv, &D, &num_pages, &maxp, &max_prefix_len, &V,
             &sm_scale) != 10)
    fail(path, "expected B N Hq Hkv D num_pages maxp max_prefix_len V sm_scale [temperature]");
  float temperature = 1.0f;
  const int sampled = fscanf(f, "%f", &temperature) == 1;
  fclose(f);
  if (B < 1 || N < 1 || N > 128 || Hq < 1 || Hkv < 1 || D < 1 || num_pages < 1 || maxp < 1 || V < 1)
    fail(path, "sizes out of range");
  const size_t W = (size_t)(N + 63) / 64, rows = (size_t)B * N;
  const size_t kv_bytes = (size_t)num_pages * Hkv * 16 * D * 2;

  tv_ctx *ctx = NULL;
  TV_CHECK(tv_create(&ctx, 0, NULL));  /* the null stream of device 0 */

  void *q = upload("q.bin", rows * Hq * D * 2);
  void *k = upload("k.bin", kv_bytes);
  void *v = upload("v.bin", kv_bytes);
  int32_t *table = (int32_t *)upload("table.bin", (size_t)B * maxp * 4);
  int32_t *plens = (int32_t *)upload("plens.bin", (size_t)B * 4);
  int32_t *parents = (int32_t *)upload("parents.bin", rows * 4);
  int32_t *tokens = (int32_t *)upload("tokens.bin", rows * 4);
  float *logits = (float *)upload("logits.bin", rows * V * 4);
  float *draft = sampled ? (float *)upload("draft.bin", rows * V * 4) : NULL;
  float *uniforms = sampled ? (float *)upload("uniforms.bin", rows * 4) : NULL;

  uint64_t *mask = (uint64_t *)device_buffer(rows * W * 8);
  int32_t *depth = (int32_t *)device_buffer(rows * 4);
  float *out = (float *)device_buffer(rows * Hq * D * 4);
  int32_t *accept_len = (int32_t *)device_buffer((size_t)B * 4);
  int32_t *path_d = (int32_t *)device_buffer(rows * 4);
  int32_t *bonus = (int32_t *)device_buffer((size_t)B * 4);
  int32_t *argmax = (int32_t *)device_buffer(rows * 4);
  int32_t *new_lens = (int32_t *)device_buffer((size_t)B * 4);
  int32_t *emitted = (int32_t *)device_buffer(rows * 4);
  int32_t *next_root = (int32_t *)device_buffer((size_t)B * 4);

  TV_CHECK(tv_build_mask(ctx, parents, NULL, B, N, mask, depth));

  const size_t aws = tv_attention_workspace_bytes(ctx, B, N, Hq, Hkv, D, max_prefix_len);
  void *attn_ws = aws ? device_buffer(aws) : NULL;
  TV_CHECK(tv_attention(ctx, q, k, v, (int64_t)num_pages, table, maxp, plens, max_prefix_len, mask, NULL, B, N, Hq,
                        Hkv, D, sm_scale, out, TV_F32, attn_ws, aws));

  const tv_accept_mode mode = sampled ? TV_STOCHASTIC : TV_GREEDY;
  const size_t cws = tv_accept_workspace_bytes(B, N, V, mode);
  void *acc_ws = device_buffer(cws);
  TV_CHECK(tv_accept(ctx, logits, draft, tokens, parents, NULL, uniforms, B, N, V, mode, temperature, accept_len,
                     path_d, bonus, sampled ? NULL : argmax, acc_ws, cws));

  /* the accepted rows into the prefix, the grown lengths, the emitted tokens
   * and the next root, all from the acceptance outputs on the device */
  TV_CHECK(tv_commit(ctx, k, v, (int64_t)num_pages, table, maxp, plens, max_prefix_len, tokens, path_d, accept_len,
                     bonus, B, N, Hkv, D, new_lens, emitted, next_root));

  double tau = 0.0;
  uint64_t cycles = 0;
  int32_t code = 0;
  TV_CHECK(tv_tau(ctx, &tau, &cycles));
  TV_CHECK(tv_device_error(ctx, &code));

  download("mask.bin", mask, rows * W * 8);
  download("depth.bin", depth, rows * 4);
  download("out.bin", out, rows * Hq * D * 4);
  download("accept_len.bin", accept_len, (size_t)B * 4);
  download("path.bin", path_d, rows * 4);
  download("bonus.bin", bonus, (size_t)B * 4);
  if (!sampled) download("argmax.bin", argmax, rows * 4);
  download("k_new.bin", k, kv_bytes);
  download("v_new.bin", v, kv_bytes);
  download("new_lens.bin", new_lens, (size_t)B * 4);
  download("emitted.bin", emitted, rows * 4);
  download("next_root.bin", next_root, (size_t)B * 4);
  printf("tau %.17g cycles %llu device_error %d\n", tau, (unsigned long long)cycles, (int)code);

  void *bufs[] = {q, k, v, table, plens, parents, tokens, logits, draft, uniforms, mask, depth, out, accept_len,
                  path_d, bonus, argmax, new_lens, emitted, next_root, attn_ws, acc_ws};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i)
    if (bufs[i]) HIP_CHECK(hipFree(bufs[i]));
  TV_CHECK(tv_destroy(ctx));
  return 0;
}
