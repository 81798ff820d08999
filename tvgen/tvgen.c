/*
 * tvgen.c - seeded, counter-based synthetic input generator.
 *
 * Serves both the oracle tests and the GPU path. It holds none of the
 * verification arithmetic (no attention, no masks, no acceptance): only
 * random streams, the Box-Muller transform, bf16 rounding and Gumbel-max
 * draws used to pick draft tokens.
 *
 * Random stream definition (splitmix64 finaliser used as a counter-based
 * generator, after Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014):
 *   mix(z)        = z ^= z>>30; z *= 0xBF58476D1CE4E5B9;
 *                   z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31
 *   key(seed,tid) = mix(seed * GAMMA ^ mix(tid + GAMMA))
 *   x(seed,tid,i) = mix(key + (i + 1) * GAMMA),   GAMMA = 0x9E3779B97F4A7C15
 * Derived values:
 *   uniform24(x)  = (x >> 40) * 2^-24            in [0, 1), exact in fp32
 *   uniform53(x)  = ((x >> 11) + 1) * 2^-53      in (0, 1]
 *   normal(e)     = Box-Muller on the pair p = e/2:
 *                   r = sqrt(-2 ln uniform53(x(2p))), a = 2 pi uniform53(x(2p+1))
 *                   even e -> r cos a, odd e -> r sin a; times sigma, in fp64
 *   bf16(v)       = fp64 -> fp32 (round to nearest even) -> bf16 (round to
 *                   nearest even on the upper 16 bits)
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBULL;
  z ^= z >> 31;
  return z;
}

uint64_t tvg_key(uint64_t seed, uint64_t tid) { return mix64(seed * GAMMA ^ mix64(tid + GAMMA)); }

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

static inline double u53(uint64_t x) { return (double)((x >> 11) + 1) * 0x1.0p-53; }

static inline double normal_at(uint64_t key, uint64_t e) {
  uint64_t p = e >> 1;
  double r = sqrt(-2.0 * log(u53(draw(key, 2 * p))));
  double a = 6.283185307179586476925286766559 * u53(draw(key, 2 * p + 1));
  return (e & 1) ? r * sin(a) : r * cos(a);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

void tvg_u64(uint64_t seed, uint64_t tid, uint64_t offset, int64_t n, uint64_t *out) {
  uint64_t key = tvg_key(seed, tid);
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t e = 0; e < n; ++e) out[e] = draw(key, offset + (uint64_t)e);
}

void tvg_uniform_f32(uint64_t seed, uint64_t tid, uint64_t offset, int64_t n, float *out) {
  uint64_t key = tvg_key(seed, tid);
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t e = 0; e < n; ++e) out[e] = (float)(draw(key, offset + (uint64_t)e) >> 40) * 0x1.0p-24f;
}

void tvg_normal_f64(uint64_t seed, uint64_t tid, uint64_t offset, int64_t n, double sigma, double *out) {
  uint64_t key = tvg_key(seed, tid);
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t e = 0; e < n; ++e) out[e] = sigma * normal_at(key, offset + (uint64_t)e);
}

void tvg_normal_f32(uint64_t seed, uint64_t tid, uint64_t offset, int64_t n, double sigma, float *out) {
  uint64_t key = tvg_key(seed, tid);
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t e = 0; e < n; ++e) out[e] = (float)(sigma * normal_at(key, offset + (uint64_t)e));
}

void tvg_normal_bf16(uint64_t seed, uint64_t tid, uint64_t offset, int64_t n, double sigma, uint16_t *out) {
  uint64_t key = tvg_key(seed, tid);
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t e = 0; e < n; ++e) out[e] = f32_to_bf16_rne((float)(sigma * normal_at(key, offset + (uint64_t)e)));
}

/* Gumbel-max draw of one token per row from softmax(logits[row] / T):
 * token = argmax_x (logits[row][x] / T + g_x), g_x = -ln(-ln uniform53),
 * with the uniforms taken from stream (seed, tid) at offset row * V + x.
 * Used only to choose draft tokens the way a sampling draft would. */
void tvg_gumbel_argmax(uint64_t seed, uint64_t tid, const float *logits, int64_t rows, int64_t V, double T,
                       int32_t *out) {
  uint64_t key = tvg_key(seed, tid);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double best = -INFINITY;
    int32_t arg = 0;
    for (int64_t x = 0; x < V; ++x) {
      double u = u53(draw(key, (uint64_t)(r * V + x)));
      if (u >= 1.0) u = 1.0 - 0x1.0p-53;
      double g = -log(-log(u));
      double v = (double)logits[r * V + x] / T + g;
      if (v > best) {
        best = v;
        arg = (int32_t)x;
      }
    }
    out[r] = arg;
  }
}
