/*
 * ORACLE — test infrastructure, not the product.
 *
 * A plain fp64 CPU definition of Multi-head Latent Attention decode over a
 * latent KV cache. Only the tests, the smoke check and the benchmark's CPU
 * baseline call it; the GPU library neither links nor calls it, and it shares
 * no code with the GPU library.
 *
 * What it computes, per sequence b, query j and head i (pages: "MLA多头潜在注意力
 * 机制" §2.2 and §3.2 training forward; the interview guide §6.2 `MLA` module;
 * the linear-algebra page, "潜在向量的压缩与上投影" and "解耦 RoPE"):
 *
 *   K[t]   = c_t · W_UK[:, i*d_n : (i+1)*d_n]         explicit up-projection
 *   V[t]   = c_t · W_UV[:, i*d_v : (i+1)*d_v]
 *   kR[t]  = RoPE(k_R,t, t)    one decoupled key, shared by all heads; optionally
 *                              rounded to bf16, the way the cache stores it
 *   q      = [ q_nope ‖ RoPE(q_R, p_j) ],  p_j = kv_len - n_q + j
 *   s_t    = scale · ( q_nope·K[t] + RoPE(q_R)·kR[t] )    for t <= p_j (causal)
 *   p_t    = exp(s_t - max s) / Σ exp(s_t - max s)    (max subtracted: interview
 *                                                       guide §7.3)
 *   out    = Σ_t p_t V[t],  heads concatenated as out[i*d_v + d]
 *   gated:   out[c] *= 1 / (1 + exp(-(x · W_G)[c]))      (Gated-MLA page §2.6)
 *
 * The absorbed twin (tutorial §3.1, both identities) computes the same result
 * without explicit K or V:
 *   q_abs = q_nope · W_UK_iᵀ (length d_c);  s_t = scale·(q_abs·c_t + RoPE(q_R)·kR[t])
 *   o_lat = Σ_t p_t c_t;  out = o_lat · W_UV_i
 * It exists to pin the identity; the explicit form is the reference answer.
 *
 * RoPE: pairs (x[2k], x[2k+1]) rotated by the angle pos * base^(-2k/d_r),
 * k = 0 .. d_r/2 - 1 (the pages only say "rotation on the complex plane"; this
 * is the RoFormer convention, taken as the plainest reading).
 *
 * Parity status of each function is stated at its definition.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F64 = 0, ORACLE_F32 = 1, ORACLE_BF16 = 2 };

typedef struct {
  int32_t h, d_c, d_r, d_n, d_v;
  double scale;     /* score scale; the workloads use 1 / sqrt(d_n + d_r) */
  double rope_base; /* 10000 in every workload */
  int32_t store_bf16; /* 1: rotated k_R is rounded to bf16 before use */
} oracle_dims;

/* Exact widening load of element i of a tensor stored as f64, f32 or bf16 bits. */
static double ld(const void* p, int type, size_t i) {
  if (type == ORACLE_F64) return ((const double*)p)[i];
  if (type == ORACLE_F32) return (double)((const float*)p)[i];
  uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/*
 * Nearest bf16 value to x, ties to the one with an even last significand bit.
 * bf16 has 8 significant bits; below 2^-126 its spacing is fixed at 2^-133.
 * Pinned by the tests against torch's float64 -> bfloat16 conversion.
 */
double oracle_round_bf16(double x) {
  if (x == 0.0 || isnan(x) || isinf(x)) return x;
  int e;
  frexp(x, &e); /* |x| in [2^(e-1), 2^e) */
  int q = e - 8;
  if (q < -133) q = -133;
  const double step = ldexp(1.0, q);
  const double lo = floor(x / step); /* x / step is exact: power-of-two scaling */
  const double frac = x / step - lo;
  double k;
  if (frac > 0.5)
    k = lo + 1.0;
  else if (frac < 0.5)
    k = lo;
  else
    k = (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0;
  const double r = k * step;
  if (fabs(r) > 0x1.FEp127) return copysign(INFINITY, x);
  return r;
}

/* RoPE of one d_r-vector at position pos. Pinned by the tests: norm kept,
 * identity at 0, relative-position property, equality with complex products. */
void oracle_rope(const double* x, int32_t d_r, int64_t pos, double base, double* out) {
  for (int32_t k = 0; k < d_r / 2; ++k) {
    const double theta = (double)pos * pow(base, -2.0 * (double)k / (double)d_r);
    const double c = cos(theta), s = sin(theta);
    const double a = x[2 * k], b = x[2 * k + 1];
    out[2 * k] = a * c - b * s;
    out[2 * k + 1] = a * s + b * c;
  }
}

typedef struct {
  const oracle_dims* d;
  int32_t B, n_q, T_stride, in_type;
  const void *c_kv, *k_r, *q_nope, *q_r, *w_uk, *w_uv, *x, *w_g;
  const int32_t* kv_len;
  int32_t d_model;
} problem;

/* Rotated (and optionally bf16-rounded) decoupled keys of sequence b, tokens 0..T-1. */
static void rotated_keys(const problem* P, int32_t b, int32_t T, double* kr) {
  const oracle_dims* d = P->d;
  double raw[1024];
  for (int32_t t = 0; t < T; ++t) {
    const size_t base = ((size_t)b * P->T_stride + t) * (size_t)d->d_r;
    for (int32_t r = 0; r < d->d_r; ++r) raw[r] = ld(P->k_r, P->in_type, base + r);
    oracle_rope(raw, d->d_r, t, d->rope_base, kr + (size_t)t * d->d_r);
    if (d->store_bf16)
      for (int32_t r = 0; r < d->d_r; ++r)
        kr[(size_t)t * d->d_r + r] = oracle_round_bf16(kr[(size_t)t * d->d_r + r]);
  }
}

/* Softmax over s[0..n-1] with the maximum subtracted; writes p, returns lse. */
static double softmax(const double* s, int32_t n, double* p) {
  double m = -INFINITY;
  for (int32_t t = 0; t < n; ++t) m = s[t] > m ? s[t] : m;
  double z = 0.0;
  for (int32_t t = 0; t < n; ++t) {
    p[t] = exp(s[t] - m);
    z += p[t];
  }
  for (int32_t t = 0; t < n; ++t) p[t] /= z;
  return m + log(z);
}

static void apply_gate(const problem* P, int32_t b, int32_t j, int32_t i, double* o) {
  const oracle_dims* d = P->d;
  const int32_t width = d->h * d->d_v;
  for (int32_t e = 0; e < d->d_v; ++e) {
    const int32_t col = i * d->d_v + e;
    double g = 0.0;
    for (int32_t k = 0; k < P->d_model; ++k)
      g += ld(P->x, P->in_type, ((size_t)b * P->n_q + j) * P->d_model + k) *
           ld(P->w_g, P->in_type, (size_t)k * width + col);
    o[e] *= 1.0 / (1.0 + exp(-g));
  }
}

/* One (sequence, head): explicit K and V, then standard causal softmax attention. */
static void head_unabsorbed(const problem* P, int32_t b, int32_t i, double* out, double* lse,
                            double* probs, int64_t probs_stride) {
  const oracle_dims* d = P->d;
  const int32_t T = P->kv_len[b], N = T - P->n_q, dq = d->d_n + d->d_r;
  double* K = (double*)calloc((size_t)T * d->d_n, sizeof(double));
  double* V = (double*)calloc((size_t)T * d->d_v, sizeof(double));
  double* kr = (double*)malloc(((size_t)T * d->d_r + 1) * sizeof(double));
  double* s = (double*)malloc((size_t)T * sizeof(double));
  double* p = (double*)malloc((size_t)T * sizeof(double));
  double* q = (double*)malloc((size_t)dq * sizeof(double));
  double* o = (double*)malloc((size_t)d->d_v * sizeof(double));
  double raw[1024];

  /* K[t] = c_t · W_UK_i and V[t] = c_t · W_UV_i */
  for (int32_t t = 0; t < T; ++t) {
    const size_t cb = ((size_t)b * P->T_stride + t) * (size_t)d->d_c;
    for (int32_t c = 0; c < d->d_c; ++c) {
      const double x = ld(P->c_kv, P->in_type, cb + c);
      const size_t ku = (size_t)c * d->h * d->d_n + (size_t)i * d->d_n;
      const size_t vu = (size_t)c * d->h * d->d_v + (size_t)i * d->d_v;
      for (int32_t e = 0; e < d->d_n; ++e) K[(size_t)t * d->d_n + e] += x * ld(P->w_uk, P->in_type, ku + e);
      for (int32_t e = 0; e < d->d_v; ++e) V[(size_t)t * d->d_v + e] += x * ld(P->w_uv, P->in_type, vu + e);
    }
  }
  if (d->d_r) rotated_keys(P, b, T, kr);

  for (int32_t j = 0; j < P->n_q; ++j) {
    const int32_t pos = N + j, n_vis = pos + 1;
    const size_t qb = (((size_t)b * P->n_q + j) * d->h + i);
    for (int32_t e = 0; e < d->d_n; ++e) q[e] = ld(P->q_nope, P->in_type, qb * d->d_n + e);
    if (d->d_r) {
      for (int32_t r = 0; r < d->d_r; ++r) raw[r] = ld(P->q_r, P->in_type, qb * d->d_r + r);
      oracle_rope(raw, d->d_r, pos, d->rope_base, q + d->d_n);
    }
    for (int32_t t = 0; t < n_vis; ++t) {
      double acc = 0.0;
      for (int32_t e = 0; e < d->d_n; ++e) acc += q[e] * K[(size_t)t * d->d_n + e];
      for (int32_t r = 0; r < d->d_r; ++r) acc += q[d->d_n + r] * kr[(size_t)t * d->d_r + r];
      s[t] = d->scale * acc;
    }
    const double l = softmax(s, n_vis, p);
    for (int32_t e = 0; e < d->d_v; ++e) {
      double acc = 0.0;
      for (int32_t t = 0; t < n_vis; ++t) acc += p[t] * V[(size_t)t * d->d_v + e];
      o[e] = acc;
    }
    if (P->x) apply_gate(P, b, j, i, o);
    const size_t ob = ((size_t)b * P->n_q + j) * (size_t)d->h * d->d_v + (size_t)i * d->d_v;
    for (int32_t e = 0; e < d->d_v; ++e) out[ob + e] = o[e];
    if (lse) lse[qb] = l;
    if (probs) {
      double* pr = probs + (int64_t)qb * probs_stride;
      for (int32_t t = 0; t < n_vis && t < probs_stride; ++t) pr[t] = p[t];
    }
  }
  free(K); free(V); free(kr); free(s); free(p); free(q); free(o);
}

/* One (sequence, head) the absorbed way: scores and the weighted sum in latent space. */
static void head_absorbed(const problem* P, int32_t b, int32_t i, double* out, double* lse,
                          double* probs, int64_t probs_stride) {
  const oracle_dims* d = P->d;
  const int32_t T = P->kv_len[b], N = T - P->n_q;
  double* kr = (double*)malloc(((size_t)T * d->d_r + 1) * sizeof(double));
  double* s = (double*)malloc((size_t)T * sizeof(double));
  double* p = (double*)malloc((size_t)T * sizeof(double));
  double* qa = (double*)malloc((size_t)d->d_c * sizeof(double));
  double* ol = (double*)malloc((size_t)d->d_c * sizeof(double));
  double* o = (double*)malloc((size_t)d->d_v * sizeof(double));
  double qr[1024], raw[1024];
  if (d->d_r) rotated_keys(P, b, T, kr);

  for (int32_t j = 0; j < P->n_q; ++j) {
    const int32_t pos = N + j, n_vis = pos + 1;
    const size_t qb = (((size_t)b * P->n_q + j) * d->h + i);
    /* q_abs[c] = Σ_e q_nope[e] W_UK[c, i*d_n + e] */
    for (int32_t c = 0; c < d->d_c; ++c) {
      double acc = 0.0;
      for (int32_t e = 0; e < d->d_n; ++e)
        acc += ld(P->q_nope, P->in_type, qb * d->d_n + e) *
               ld(P->w_uk, P->in_type, (size_t)c * d->h * d->d_n + (size_t)i * d->d_n + e);
      qa[c] = acc;
    }
    if (d->d_r) {
      for (int32_t r = 0; r < d->d_r; ++r) raw[r] = ld(P->q_r, P->in_type, qb * d->d_r + r);
      oracle_rope(raw, d->d_r, pos, d->rope_base, qr);
    }
    for (int32_t t = 0; t < n_vis; ++t) {
      const size_t cb = ((size_t)b * P->T_stride + t) * (size_t)d->d_c;
      double acc = 0.0;
      for (int32_t c = 0; c < d->d_c; ++c) acc += qa[c] * ld(P->c_kv, P->in_type, cb + c);
      for (int32_t r = 0; r < d->d_r; ++r) acc += qr[r] * kr[(size_t)t * d->d_r + r];
      s[t] = d->scale * acc;
    }
    const double l = softmax(s, n_vis, p);
    for (int32_t c = 0; c < d->d_c; ++c) ol[c] = 0.0;
    for (int32_t t = 0; t < n_vis; ++t) {
      const size_t cb = ((size_t)b * P->T_stride + t) * (size_t)d->d_c;
      for (int32_t c = 0; c < d->d_c; ++c) ol[c] += p[t] * ld(P->c_kv, P->in_type, cb + c);
    }
    for (int32_t e = 0; e < d->d_v; ++e) {
      double acc = 0.0;
      for (int32_t c = 0; c < d->d_c; ++c)
        acc += ol[c] * ld(P->w_uv, P->in_type, (size_t)c * d->h * d->d_v + (size_t)i * d->d_v + e);
      o[e] = acc;
    }
    if (P->x) apply_gate(P, b, j, i, o);
    const size_t ob = ((size_t)b * P->n_q + j) * (size_t)d->h * d->d_v + (size_t)i * d->d_v;
    for (int32_t e = 0; e < d->d_v; ++e) out[ob + e] = o[e];
    if (lse) lse[qb] = l;
    if (probs) {
      double* pr = probs + (int64_t)qb * probs_stride;
      for (int32_t t = 0; t < n_vis && t < probs_stride; ++t) pr[t] = p[t];
    }
  }
  free(kr); free(s); free(p); free(qa); free(ol); free(o);
}

/*
 * Decode for the selected (sequence, head) pairs, or all of them when n_sel < 0.
 *
 * c_kv [B][T_stride][d_c], k_r [B][T_stride][d_r] (raw), q_nope [B][n_q][h][d_n],
 * q_r [B][n_q][h][d_r] (raw), w_uk [d_c][h*d_n], w_uv [d_c][h*d_v],
 * x [B][n_q][d_model] and w_g [d_model][h*d_v] (both NULL when ungated), all of
 * in_type. kv_len[b] includes the n_q new tokens. Outputs: out [B][n_q][h*d_v],
 * lse [B][n_q][h] (optional), probs [B][n_q][h][probs_stride] (optional).
 * Entries of unselected pairs are left untouched. Returns 0, or -1 on a shape
 * the definition does not cover (kv_len < n_q, kv_len > T_stride, odd d_r).
 */
int32_t oracle_mla_decode(const oracle_dims* d, int32_t B, int32_t n_q, int32_t T_stride,
                          int32_t in_type, const void* c_kv, const void* k_r,
                          const int32_t* kv_len, const void* q_nope, const void* q_r,
                          const void* w_uk, const void* w_uv, const void* x, const void* w_g,
                          int32_t d_model, int32_t n_sel, const int32_t* sel_b,
                          const int32_t* sel_h, int32_t absorbed, double* out, double* lse,
                          double* probs, int64_t probs_stride) {
  if (d->d_r % 2 || d->d_r > 1024 || n_q < 1) return -1;
  for (int32_t b = 0; b < B; ++b)
    if (kv_len[b] < n_q || kv_len[b] > T_stride) return -1;
  problem P = {d, B, n_q, T_stride, in_type, c_kv, k_r, q_nope, q_r, w_uk, w_uv, x, w_g, kv_len, d_model};
  const int64_t n = n_sel < 0 ? (int64_t)B * d->h : n_sel;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t k = 0; k < n; ++k) {
    const int32_t b = n_sel < 0 ? (int32_t)(k / d->h) : sel_b[k];
    const int32_t i = n_sel < 0 ? (int32_t)(k % d->h) : sel_h[k];
    if (absorbed)
      head_absorbed(&P, b, i, out, lse, probs, probs_stride);
    else
      head_unabsorbed(&P, b, i, out, lse, probs, probs_stride);
  }
  return 0;
}

/* Rotated, storage-rounded decoupled keys as the cache holds them: kr [B][T][d_r]. */
void oracle_cache_keys(const oracle_dims* d, int32_t B, int32_t T_stride, int32_t in_type,
                       const void* k_r, const int32_t* kv_len, double* kr) {
  problem P = {d, B, 1, T_stride, in_type, NULL, k_r, NULL, NULL, NULL, NULL, NULL, NULL, kv_len, 0};
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t b = 0; b < B; ++b) rotated_keys(&P, b, kv_len[b], kr + (size_t)b * T_stride * d->d_r);
}

/*
 * Latent cache row of one token from its hidden state, for the fused append.
 * Parity pinned by the tests: 50-digit decimal brute force, torch's rms_norm with
 * a complex-number RoPE in fp64, the identity-weight closed form, and the gain and
 * scale invariants.
 *
 * Pages: tutorial §2.2 (c_KV = h · W_DKV, W_DKV of d_model × d_c) and §6.3 (an
 * RMSNorm over the d_c latent right after the down-projection); the interview
 * guide §6.2 `MLA` module (k_R from its own d_model → d_rope projection of the
 * same input); linear-algebra page "解耦 RoPE" (k_R is cached rotated).
 *
 *   c      = h · W_DKV                                     [d_c]
 *   c_norm = gain ⊙ c / sqrt(mean_n c[n]² + eps)           (gain NULL: ones)
 *   k      = RoPE(h · W_KR, pos)                           [d_r]
 *   out    = [ c_norm ‖ k ] in fp64; the caller rounds to the cache type.
 *
 * hidden [M][d_model], w_dkv [d_model][d_c], w_kr [d_model][d_r] of in_type;
 * gain [d_c] fp64 or NULL; pos [M]; out [M][d_c + d_r]. Returns -1 on a bad shape.
 */
int32_t oracle_project_latent(int32_t M, int32_t d_model, int32_t d_c, int32_t d_r,
                              int32_t in_type, const void* hidden, const void* w_dkv,
                              const void* w_kr, const double* gain, double eps,
                              const int64_t* pos, double base, double* out) {
  if (M < 0 || d_model <= 0 || d_c <= 0 || d_r < 0 || d_r % 2 || d_r > 1024 || !(eps >= 0.0))
    return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t m = 0; m < M; ++m) {
    double* row = out + (size_t)m * (d_c + d_r);
    double kraw[1024];
    for (int32_t n = 0; n < d_c; ++n) row[n] = 0.0;
    for (int32_t n = 0; n < d_r; ++n) kraw[n] = 0.0;
    /* both products, k ascending for every output element */
    for (int32_t k = 0; k < d_model; ++k) {
      const double hk = ld(hidden, in_type, (size_t)m * d_model + k);
      for (int32_t n = 0; n < d_c; ++n) row[n] += hk * ld(w_dkv, in_type, (size_t)k * d_c + n);
      for (int32_t n = 0; n < d_r; ++n) kraw[n] += hk * ld(w_kr, in_type, (size_t)k * d_r + n);
    }
    double ss = 0.0;
    for (int32_t n = 0; n < d_c; ++n) ss += row[n] * row[n];
    const double rms = sqrt(ss / (double)d_c + eps);
    for (int32_t n = 0; n < d_c; ++n) row[n] = (gain ? gain[n] : 1.0) * (row[n] / rms);
    if (d_r) oracle_rope(kraw, d_r, pos[m], base, row + d_c);
  }
  return 0;
}

/* Storage rounding of n values to bf16 (oracle_round_bf16 elementwise). */
void oracle_round_bf16_array(int64_t n, const double* x, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_round_bf16(x[i]);
}

int32_t oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
