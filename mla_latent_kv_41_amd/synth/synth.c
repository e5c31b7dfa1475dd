/*
 * Seeded synthetic inputs for absorbed-MLA decode.
 *
 * This module draws random numbers and nothing else: it holds none of the
 * attention arithmetic. Both the fp64 oracle and the HIP path are fed from
 * it, so they see bit-identical inputs.
 *
 * Generator: a counter-based stream. Element i of the stream keyed by
 * (seed, tag) is splitmix64(key + (i + 1) * 0x9E3779B97F4A7C15) (the finaliser
 * of Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
 * OOPSLA 2014). Its top 53 bits give a uniform in [0, 1). Normals come from
 * the Box-Muller transform on consecutive uniform pairs. Because every element
 * is a pure function of its index, any slice can be drawn on its own and the
 * threads never need to agree on an order.
 *
 * Rounding to bf16 is round-to-nearest, ties-to-even, taken directly from the
 * fp64 value (no intermediate fp32 rounding).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_finalise(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* FNV-1a over the tag, then mixed with the seed: one key per named tensor. */
uint64_t synth_key(uint64_t seed, const char* tag) {
  uint64_t h = 0xCBF29CE484222325ULL;
  for (const unsigned char* p = (const unsigned char*)tag; *p; ++p) {
    h ^= *p;
    h *= 0x100000001B3ULL;
  }
  return sm64_finalise(seed * SYNTH_GAMMA ^ h);
}

static inline uint64_t draw_u64(uint64_t key, uint64_t i) {
  return sm64_finalise(key + (i + 1) * SYNTH_GAMMA);
}

static inline double draw_uniform(uint64_t key, uint64_t i) {
  return (double)(draw_u64(key, i) >> 11) * 0x1.0p-53;
}

/* Normal number i of the stream: pair p = i / 2 uses uniforms 2p and 2p+1. */
static inline double draw_normal(uint64_t key, uint64_t i) {
  const uint64_t p = i >> 1;
  const double u1 = draw_uniform(key, 2 * p);
  const double u2 = draw_uniform(key, 2 * p + 1);
  const double r = sqrt(-2.0 * log(1.0 - u1)); /* 1 - u1 is in (0, 1] */
  const double a = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

/* fp64 -> bf16 bits, round to nearest even. */
uint16_t synth_f64_to_bf16(double x) {
  if (isnan(x)) return 0x7FC0;
  if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
  if (isinf(x)) return signbit(x) ? 0xFF80 : 0x7F80;
  int e;
  (void)frexp(x, &e); /* |x| = f * 2^e, f in [0.5, 1) */
  /* bf16 keeps 8 significant bits; below 2^-126 the spacing is fixed at 2^-133. */
  int q = e - 8;
  if (q < -133) q = -133;
  const double quantum = ldexp(1.0, q);
  const double r = rint(x / quantum) * quantum; /* exact scaling, ties to even */
  if (fabs(r) > 0x1.FEp127) return signbit(x) ? 0xFF80 : 0x7F80;
  const float f = (float)r; /* r is a bf16 value, so this is exact */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

void synth_normal_f64(uint64_t key, uint64_t start, uint64_t n, double std, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < (int64_t)n; ++k) out[k] = std * draw_normal(key, start + (uint64_t)k);
}

void synth_normal_f32(uint64_t key, uint64_t start, uint64_t n, double std, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < (int64_t)n; ++k) out[k] = (float)(std * draw_normal(key, start + (uint64_t)k));
}

void synth_normal_bf16(uint64_t key, uint64_t start, uint64_t n, double std, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < (int64_t)n; ++k)
    out[k] = synth_f64_to_bf16(std * draw_normal(key, start + (uint64_t)k));
}

/*
 * Rows of `width` normals, each divided by its root-mean-square
 * (x / sqrt(mean(x^2) + eps), no gain), then written as bf16 or fp32.
 * Row r uses stream elements [r * width, (r + 1) * width).
 */
void synth_rmsnorm_rows(uint64_t key, uint64_t row0, uint64_t rows, int width, double eps,
                        int as_bf16, void* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < (int64_t)rows; ++r) {
    double buf[4096];
    const int w = width < 4096 ? width : 4096;
    const uint64_t base = (row0 + (uint64_t)r) * (uint64_t)width;
    double ss = 0.0;
    for (int c = 0; c < w; ++c) {
      buf[c] = draw_normal(key, base + (uint64_t)c);
      ss += buf[c] * buf[c];
    }
    const double inv = 1.0 / sqrt(ss / w + eps);
    if (as_bf16) {
      uint16_t* o = (uint16_t*)out + (uint64_t)r * (uint64_t)width;
      for (int c = 0; c < w; ++c) o[c] = synth_f64_to_bf16(buf[c] * inv);
    } else {
      float* o = (float*)out + (uint64_t)r * (uint64_t)width;
      for (int c = 0; c < w; ++c) o[c] = (float)(buf[c] * inv);
    }
  }
}

/* Integers uniform on [lo, hi], inclusive at both ends (rejection-free: 53-bit
 * uniform times the range, floored; the bias is below 2^-39 for ranges < 2^14). */
void synth_uniform_int(uint64_t key, uint64_t n, int32_t lo, int32_t hi, int32_t* out) {
  const double span = (double)hi - (double)lo + 1.0;
  for (uint64_t k = 0; k < n; ++k) {
    int64_t v = (int64_t)lo + (int64_t)floor(draw_uniform(key, k) * span);
    if (v > hi) v = hi;
    out[k] = (int32_t)v;
  }
}

/* Fisher-Yates shuffle of 0..n-1: step k swaps slot n-1-k with a uniform slot
 * in [0, n-1-k]. */
void synth_permutation(uint64_t key, int32_t n, int32_t* out) {
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t k = 0; k + 1 < n; ++k) {
    const int32_t top = n - 1 - k;
    int32_t j = (int32_t)floor(draw_uniform(key, (uint64_t)k) * (double)(top + 1));
    if (j > top) j = top;
    const int32_t t = out[top];
    out[top] = out[j];
    out[j] = t;
  }
}
