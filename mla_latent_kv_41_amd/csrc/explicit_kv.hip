// The non-absorbed form of MLA decode on the GPU, for comparison with the absorbed
// path (MLA tutorial page §3.2: the training-time forward up-projects the cached
// latent into per-head keys and values, k = c_KV · W_UK and v = c_KV · W_UV, then
// runs standard attention; §3.3 compares the two at decode).
//
//   expand_kernel:   K[b][t][i][:] = c_t · W_UK_i and V[b][t][i][:] = c_t · W_UV_i for
//                    every cached token, fp32 (bf16 MFMA products, fp32 accumulation)
//   explicit_decode_kernel: per (sequence, head, token range), the scores
//                    scale · (q_nope · K_t + RoPE(q_R) · k_R,t) against the explicit
//                    keys (k_R, shared by all heads, from the latent cache), online
//                    max-subtracted softmax (interview guide §7.3), O = Σ_t p_t V_t;
//                    fp32 arithmetic throughout
//   explicit_combine_kernel: merges the token ranges (log-sum-exp weights), applies
//                    the sigmoid gate (Gated-MLA page §2.6), writes out and lse
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr int kHeadDim = 128;      // d_qk_nope = d_v
constexpr int kTokPerWave = 32;    // expand: tokens per wave (one MFMA row block)
constexpr int kTokPerWg = 128;     // expand: tokens per workgroup
constexpr int kGroup = 8;          // decode: lanes per token (16 of the 128 dims each)
}  // namespace

// W [d_c][h*128] (formula layout) -> MFMA B-operand fragments of the products
// D[t][e] = Σ_c C[t][c] W_i[c][e]: fragment (i, nb < 4, ks < d_c/16), lane l holds
// W[16ks + 8(l/32) + e][i*128 + 32nb + l%32], e = 0..7 (one contiguous 1 KiB per
// fragment). `which` = 0 packs W_UK, 1 packs W_UV, into consecutive regions.
__global__ void pack_c_kernel(const uint16_t* __restrict__ w_uk, const uint16_t* __restrict__ w_uv,
                              uint16_t* __restrict__ packed, int h, int d_c) {
  const int KS = d_c / 16;
  const int64_t per = static_cast<int64_t>(h) * 4 * KS * 64;  // lanes per region
  const int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= 2 * per) return;
  const uint16_t* w = g < per ? w_uk : w_uv;
  const int64_t gg = g < per ? g : g - per;
  const int l = static_cast<int>(gg % 64);
  const int64_t f = gg / 64;
  const int ks = static_cast<int>(f % KS), nb = static_cast<int>((f / KS) % 4), i = static_cast<int>(f / (4 * KS));
  const int64_t width = static_cast<int64_t>(h) * kHeadDim;
  const int64_t col = static_cast<int64_t>(i) * kHeadDim + 32 * nb + l % 32;
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t r = 16 * ks + 8 * (l / 32) + 2 * e;
    o[e] = static_cast<uint32_t>(w[r * width + col]) | (static_cast<uint32_t>(w[(r + 1) * width + col]) << 16);
  }
  *reinterpret_cast<u32x4*>(packed + g * 8) = o;
}

// Cache row of token t of sequence b (bf16), or nullptr outside the cache.
__device__ __forceinline__ const uint16_t* latent_row(const CacheRef& c, int b, int t, int row) {
  const uint16_t* base = static_cast<const uint16_t*>(c.data);
  if (c.block_table == nullptr) return base + (static_cast<int64_t>(b) * c.t_max + t) * row;
  const int blk = t / c.block_size;
  if (blk >= c.max_blocks) return nullptr;
  const int32_t id = c.block_table[static_cast<int64_t>(b) * c.max_blocks + blk];
  if (id < 0 || id >= c.n_blocks) return nullptr;
  return base + (static_cast<int64_t>(id) * c.block_size + t % c.block_size) * row;
}

// grid (batch * ceil(max_kv_len / 128), h, 2), 256 threads. Workgroup (blk, i, kv)
// takes 128 tokens of one sequence, head i, and K (kv = 0) or V (kv = 1); wave w
// takes 32 of the tokens: D[t][e] = Σ_c C[t][c] W_i[c][e] on v_mfma_f32_32x32x16_bf16,
// the A operand straight from the cache rows (lane l: token l%32, latent columns
// 16ks + 8(l/32) .. + 7, one 16-byte load), the B operand from the packed weights.
// Lane l of the result holds column 32nb + l%32 of rows 8(v/4) + 4(l/32) + v%4, so
// each store writes 128 contiguous bytes of a row per half wave.
__global__ __launch_bounds__(256) void expand_kernel(ExpandArgs a) {
  const int TB = (a.max_kv_len + kTokPerWg - 1) / kTokPerWg;
  const int b = blockIdx.x / TB, tb = blockIdx.x - (blockIdx.x / TB) * TB;
  const int i = blockIdx.y, which = blockIdx.z;
  const int l = threadIdx.x % 64, w = threadIdx.x / 64;
  const int kv = min(a.kv_lens[b], a.max_kv_len);
  const int t0 = kTokPerWg * tb + kTokPerWave * w;
  if (t0 >= kv) return;
  const int KS = a.d_c / 16, row = a.d_c + a.d_r;
  const int t = t0 + (l & 31);
  const uint16_t* src = t < kv ? latent_row(a.cache, b, t, row) : nullptr;
  const u32x4* wp = reinterpret_cast<const u32x4*>(a.packed) +
                    (static_cast<int64_t>(which) * a.h + i) * 4 * KS * 64 + l;
  f32x16 acc[4] = {};
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4 af = src ? *reinterpret_cast<const u32x4*>(src + 16 * ks + 8 * (l >> 5)) : u32x4{0u, 0u, 0u, 0u};
    u32x4 bf[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) bf[nb] = wp[(nb * KS + ks) * 64];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af), as_bf16x8(bf[nb]), acc[nb], 0, 0, 0);
  }
  float* dst = which == 0 ? a.k_out : a.v_out;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int tt = t0 + 8 * (v / 4) + 4 * (l >> 5) + (v & 3);
    if (tt >= kv) continue;
    float* p = dst + ((static_cast<int64_t>(b) * a.max_kv_len + tt) * a.h + i) * kHeadDim;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) p[32 * nb + (l & 31)] = acc[nb][v];
  }
}

hipError_t launch_expand(const ExpandArgs& a, hipStream_t s) {
  if (a.d_c % 16 != 0 || a.h <= 0) return hipErrorInvalidValue;
  const int64_t n = static_cast<int64_t>(a.h) * 4 * (a.d_c / 16) * 64 * 2;
  pack_c_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), 256, 0, s>>>(
      a.w_uk, a.w_uv, const_cast<uint16_t*>(a.packed), a.h, a.d_c);
  const int TB = (a.max_kv_len + kTokPerWg - 1) / kTokPerWg;
  expand_kernel<<<dim3(static_cast<unsigned>(a.batch * TB), a.h, 2), 256, 0, s>>>(a);
  return hipGetLastError();
}

// grid (batch * n_splits * h), 256 threads; workgroup ((b, s), i) takes head i over
// tokens [s * chunk, min((s + 1) * chunk, kv)). Within a wave, lane group g = l/8
// takes one token of each 8-token chunk and lane k = l%8 dims 16k .. 16k + 15 of the
// key and value (and rotated-key dims 8k .. 8k + 7); wave w takes chunks w, w + 4, ...
// Each lane group keeps its own running max, sum and output per query; the groups,
// then the waves (through LDS), are merged at the end, and the range's (O, m, l) per
// (query, head) is written in base-2 units.
template <int NQ>
__global__ __launch_bounds__(256) void explicit_decode_kernel(ExplicitArgs a) {
  __shared__ float s_o[4][NQ][kHeadDim];
  __shared__ float s_ml[4][NQ][2];
  const int tid = threadIdx.x, l = tid % 64, w = tid / 64;
  const int g = l >> 3, k = l & 7;
  const int i = blockIdx.x % a.h;
  const int bs = blockIdx.x / a.h;
  const int b = bs / a.n_splits, s = bs - b * a.n_splits;
  const int kv = min(a.kv_lens[b], a.max_kv_len);
  const int t_begin = s * a.chunk, t_end = min(t_begin + a.chunk, kv);
  const int row = 512 + a.d_r;

  // this lane's query slices, pre-scaled by scale * log2(e)
  float qn[NQ][16], qr[NQ][8];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int jj = min(j, a.n_q - 1);
    const int64_t qb = (static_cast<int64_t>(b) * a.n_q + jj) * a.h + i;
#pragma unroll
    for (int e = 0; e < 16; ++e) qn[j][e] = bf16_bits_to_f32(a.q_nope[qb * kHeadDim + 16 * k + e]) * a.qscale;
#pragma unroll
    for (int e = 0; e < 8; ++e) qr[j][e] = 0.f;
    if (a.d_r > 0) {
      const double pos = static_cast<double>(kv - a.n_q + jj);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int pr = 4 * k + p;  // rotation pair pr: columns 2pr, 2pr + 1
        const double theta = pos * a.inv_freq[pr];
        const double red = theta - 6.283185307179586 * rint(theta * 0.15915494309189535);
        float sn, cs;
        sincosf(static_cast<float>(red), &sn, &cs);
        const float x0 = bf16_bits_to_f32(a.q_rope[qb * a.d_r + 2 * pr]);
        const float x1 = bf16_bits_to_f32(a.q_rope[qb * a.d_r + 2 * pr + 1]);
        qr[j][2 * p] = (x0 * cs - x1 * sn) * a.qscale;
        qr[j][2 * p + 1] = (x0 * sn + x1 * cs) * a.qscale;
      }
    }
  }
  float m[NQ], lsum[NQ], o[NQ][16];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    m[j] = -INFINITY;
    lsum[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) o[j][e] = 0.f;
  }

  for (int c0 = t_begin + kGroup * w; c0 < t_end; c0 += 4 * kGroup) {  // uniform per wave
    const int t = c0 + g;
    const bool valid = t < t_end;
    f32x4 kk[4], vv[4];
    u32x4 kr = {0u, 0u, 0u, 0u};
    if (valid) {
      const int64_t base = ((static_cast<int64_t>(b) * a.max_kv_len + t) * a.h + i) * kHeadDim + 16 * k;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        kk[q] = *reinterpret_cast<const f32x4*>(a.k + base + 4 * q);
        vv[q] = *reinterpret_cast<const f32x4*>(a.v + base + 4 * q);
      }
      if (a.d_r > 0) {
        const uint16_t* rw = latent_row(a.cache, b, t, row);
        if (rw) kr = *reinterpret_cast<const u32x4*>(rw + 512 + 8 * k);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) kk[q] = vv[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float krf[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      krf[2 * e] = __uint_as_float(kr[e] << 16);
      krf[2 * e + 1] = __uint_as_float(kr[e] & 0xFFFF0000u);
    }
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      if (j >= a.n_q) break;
      float sc = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) sc = fmaf(qn[j][4 * q + e], kk[q][e], sc);
#pragma unroll
      for (int e = 0; e < 8; ++e) sc = fmaf(qr[j][e], krf[e], sc);
      sc += __shfl_xor(sc, 1);
      sc += __shfl_xor(sc, 2);
      sc += __shfl_xor(sc, 4);
      const bool vis = valid && t <= kv - a.n_q + j;
      if (vis) {  // online softmax of this lane group's tokens
        const float mn = fmaxf(m[j], sc);
        const float alpha = fast_exp2(m[j] - mn), p = fast_exp2(sc - mn);
        lsum[j] = lsum[j] * alpha + p;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) o[j][4 * q + e] = fmaf(p, vv[q][e], o[j][4 * q + e] * alpha);
        m[j] = mn;
      }
    }
  }
  // merge the 8 lane groups of the wave (lanes l, l ^ 8, l ^ 16, l ^ 32 hold the same dims)
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    float mx = m[j];
    mx = fmaxf(mx, __shfl_xor(mx, 8));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float f = m[j] == -INFINITY ? 0.f : fast_exp2(m[j] - mx);
    float ls = lsum[j] * f;
    ls += __shfl_xor(ls, 8);
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float x = o[j][e] * f;
      x += __shfl_xor(x, 8);
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      o[j][e] = x;
    }
    if (g == 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s_o[w][j][16 * k + e] = o[j][e];
      if (k == 0) {
        s_ml[w][j][0] = mx;
        s_ml[w][j][1] = ls;
      }
    }
  }
  __syncthreads();
  // merge the 4 waves; thread (j, d) writes the range's partial
  for (int x = tid; x < NQ * kHeadDim; x += 256) {
    const int j = x / kHeadDim, d = x - j * kHeadDim;
    if (j >= a.n_q) continue;
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) mx = fmaxf(mx, s_ml[q][j][0]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float f = s_ml[q][j][0] == -INFINITY ? 0.f : fast_exp2(s_ml[q][j][0] - mx);
      L += f * s_ml[q][j][1];
      O += f * s_o[q][j][d];
    }
    float* part = a.part + ((static_cast<int64_t>(bs) * a.n_q + j) * a.h + i) * (kHeadDim + 2);
    part[d] = O;
    if (d == 0) {
      part[kHeadDim] = mx;
      part[kHeadDim + 1] = L;
    }
  }
}

// grid (ceil(B * n_q * h / 4)), 256 threads: wave w takes one (b, j, i) row, lane l
// its dims 2l, 2l + 1. Merges the ranges holding tokens of the row and writes
// out[b][j][i * 128 + d] (times the gate's sigmoid) and lse.
__global__ __launch_bounds__(256) void explicit_combine_kernel(ExplicitArgs a) {
  const int l = threadIdx.x % 64;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
  const int64_t rows = static_cast<int64_t>(a.batch) * a.n_q * a.h;
  if (r >= rows) return;
  const int i = static_cast<int>(r % a.h);
  const int64_t m = r / a.h;  // b * n_q + j
  const int b = static_cast<int>(m / a.n_q), j = static_cast<int>(m % a.n_q);
  const int kv = min(a.kv_lens[b], a.max_kv_len);
  const int ns = kv >= a.n_q ? min(a.n_splits, (kv + a.chunk - 1) / a.chunk) : 0;
  auto part = [&](int s) -> const float* {
    return a.part + (((static_cast<int64_t>(b) * a.n_splits + s) * a.n_q + j) * a.h + i) * (kHeadDim + 2);
  };
  float mx = -INFINITY;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, part(s)[kHeadDim]);
  const float mref = mx == -INFINITY ? 0.f : mx;
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float* p = part(s);
    const float f = p[kHeadDim] == -INFINITY ? 0.f : fast_exp2(p[kHeadDim] - mref);
    L += f * p[kHeadDim + 1];
    o0 += f * p[2 * l];
    o1 += f * p[2 * l + 1];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  o0 *= inv;
  o1 *= inv;
  const int width = a.h * kHeadDim;
  const int col = i * kHeadDim + 2 * l;
  if (a.gate) {
    float g0 = 0.f, g1 = 0.f;
    for (int ks = 0; ks < kGateSplit; ++ks) {
      const float* gp = a.gate + (static_cast<int64_t>(ks) * (a.batch * a.n_q) + m) * width + col;
      g0 += gp[0];
      g1 += gp[1];
    }
    o0 *= 1.f / (1.f + __expf(-g0));
    o1 *= 1.f / (1.f + __expf(-g1));
  }
  *reinterpret_cast<f32x2*>(a.out + m * width + col) = f32x2{o0, o1};
  if (a.lse && l == 0) a.lse[r] = L > 0.f ? (mx + __log2f(L)) * kLn2 : -INFINITY;
}

hipError_t launch_explicit_decode(const ExplicitArgs& a, hipEvent_t ev0, hipEvent_t ev1, hipStream_t s) {
  if (a.n_q < 1 || a.n_q > 4 || (a.d_r != 0 && a.d_r != 64)) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.batch) * a.n_splits * a.h));
  if (ev0) hipEventRecord(ev0, s);
  if (a.n_q == 1) explicit_decode_kernel<1><<<grid, 256, 0, s>>>(a);
  else if (a.n_q == 2) explicit_decode_kernel<2><<<grid, 256, 0, s>>>(a);
  else explicit_decode_kernel<4><<<grid, 256, 0, s>>>(a);
  if (ev1) hipEventRecord(ev1, s);
  const int64_t rows = static_cast<int64_t>(a.batch) * a.n_q * a.h;
  explicit_combine_kernel<<<dim3(static_cast<unsigned>((rows + 3) / 4)), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
