// Split combine + W_UV up-projection (+ sigmoid output gate) for the bf16 path.
//
// Combine: the ranges s of one (query, head) row carry (O_s, m_s, l_s) in fp32,
// O_s and l_s relative to their own reference m_s (base-2 units). The merge is the
// max-subtracted softmax of the interview guide §7.3 applied across ranges:
//   M = max_s m_s,  L = Σ_s 2^(m_s - M) l_s,  o_lat = Σ_s 2^(m_s - M) O_s / L,
//   lse = (M + log2 L) ln 2 (natural-log units).
// Up-projection (MLA tutorial page §3.1 and the `bhsc,hdc->bhsd` einsum of §5.1):
// out[m, i*128 + d] = o_lat[m, i, :] · W_UV_i[:, d], on v_mfma_f32_32x32x16_bf16
// with o_lat entering as a hi + lo pair of bf16 rows (about 16 significant bits).
// Gate (Gated-MLA page §2.6): out *= sigmoid(g), g = x · W_G per channel of the
// concatenated heads.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr int kGateSplit = 16;             // K-splits of the gate GEMM
constexpr int kHalf = 256;                 // latent columns per workgroup (half of d_c)
constexpr int kAStride = kHalf * 2 + 16;   // bytes per o_lat half row in LDS (padded)
constexpr int kBatch = 8;                  // partial half rows per row in flight at once
constexpr int kWaves = 8;                  // waves per workgroup
constexpr int kRowsPerWave = 4;            // query rows per wave (32 per workgroup)
}  // namespace

// grid (h, 2, ceil(M / R)), 512 threads, R <= 32 query rows per workgroup. Workgroup
// (i, kh, mb) takes head i, latent columns [256 kh, 256 kh + 256) and query rows
// m0 .. m0 + R - 1, and adds its share of the up-projection,
//   out[m][i*128 + d] += Σ_{c in half kh} o_lat[m][i][c] · W_UV_i[c][d],
// into the output with fp32 atomics (the output was zeroed by the query preparation
// of the same call). Each output element gets exactly two addends onto zero, so the
// sum does not depend on their order. Splitting the latent dimension, not the rows,
// reads each partial row and each W_UV_i once.
//
// Sequence b's ranges hold partial indices seq_off[b] .. seq_off[b + 1] - 1 (the
// plan's compact layout). Wave w takes rows w, w + 8, w + 16, w + 24, lane l columns
// 4l .. 4l + 3 of the half row. Everything a wave needs goes out at once: the (m, l)
// of each row's first 64 ranges (lane s: range s) and the half rows of its first 8
// ranges, so a wave waits for memory about once. Lane s then forms range s's weight
// 2^(m_s - M) / L, which the merge reads back with readlane; further ranges come 8
// at a time. Ranges merge in a fixed order, so the result is deterministic. Waves
// 0-3 also load the W_UV_i fragments first and run the up-projection.
__global__ __launch_bounds__(kWaves * 64) void combine_kernel(CombineArgs a) {
  __shared__ __attribute__((aligned(16))) char s_hi[32 * kAStride];
  __shared__ __attribute__((aligned(16))) char s_lo[32 * kAStride];
  const int i = blockIdx.x, kh = blockIdx.y, mb = blockIdx.z;
  const int tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int M = a.batch * a.n_q;
  const int m0 = mb * a.rows_per_wg;
  const int rows = min(a.rows_per_wg, M - m0);
  const int64_t rstride = static_cast<int64_t>(a.n_q) * a.h;  // partial rows per range

  // W_UV_i fragments of wave w's 32 output columns, 16 k-steps of half kh
  u32x4 bfr[16];
  if (w < 4 && !a.o_lat) {
    const u32x4* wv = reinterpret_cast<const u32x4*>(a.w_uv_pk) + ((static_cast<int64_t>(i) * 4 + w) * 32 + 16 * kh) * 64 + l;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) bfr[ks] = wv[ks * 64];
  }

  // this wave's rows: (first partial row, number of ranges)
  int64_t row0[kRowsPerWave];
  int ns[kRowsPerWave];
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) {
    const int r = w + kWaves * k;
    ns[k] = 0;
    row0[k] = 0;
    if (r < rows) {  // uniform
      const int m = m0 + r, b = m / a.n_q, j = m - b * a.n_q;
      const int p0 = a.seq_off[b];
      ns[k] = a.seq_off[b + 1] - p0;
      row0[k] = (static_cast<int64_t>(p0) * a.n_q + j) * a.h + i;
    }
  }
  // (m, l) of ranges l (< 64) and the first kBatch half rows of every row
  f32x2 ml[kRowsPerWave];
  f32x4 v[kRowsPerWave][kBatch];
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) {
    ml[k] = l < ns[k] ? *reinterpret_cast<const f32x2*>(a.ml_part + (row0[k] + l * rstride) * 2)
                      : f32x2{-INFINITY, 0.f};
    const float* src = a.o_part + row0[k] * 512 + kHalf * kh + 4 * l;
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      v[k][u] = u < ns[k] ? *reinterpret_cast<const f32x4*>(src + u * rstride * 512) : f32x4{0.f, 0.f, 0.f, 0.f};
  }

#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) {
    const int r = w + kWaves * k;
    if (r >= 32) break;
    u32x2 hv = {0u, 0u}, lv = {0u, 0u};
    if (r < rows) {  // uniform
      // ---- statistics over the ranges (ranges past 64 in a loop)
      float mx = ml[k][0];
      for (int s = l + 64; s < ns[k]; s += 64) mx = fmaxf(mx, a.ml_part[(row0[k] + s * rstride) * 2]);
      mx = wave_max(mx);
      const float mref = mx == -INFINITY ? 0.f : mx;
      float L = l < ns[k] ? fast_exp2(ml[k][0] - mref) * ml[k][1] : 0.f;
      for (int s = l + 64; s < ns[k]; s += 64) {
        const f32x2 q = *reinterpret_cast<const f32x2*>(a.ml_part + (row0[k] + s * rstride) * 2);
        L += fast_exp2(q[0] - mref) * q[1];
      }
      L = wave_sum(L);
      const float inv_l = L > 0.f ? 1.f / L : 0.f;
      if (kh == 0 && a.lse && l == 0) a.lse[static_cast<int64_t>(m0 + r) * a.h + i] = L > 0.f ? (mx + __log2f(L)) * kLn2 : -INFINITY;
      // ---- merge: o = Σ_s 2^(m_s - M) / L · O_s over this lane's 4 columns
      const float wl = l < ns[k] ? fast_exp2(ml[k][0] - mref) * inv_l : 0.f;  // weight of range l
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < kBatch; ++u) o += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u)) * v[k][u];
      const float* src = a.o_part + row0[k] * 512 + kHalf * kh + 4 * l;
      for (int s0 = kBatch; s0 < ns[k]; s0 += kBatch) {  // uniform: rows with more than 8 ranges
        f32x4 q[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
          q[u] = s0 + u < ns[k] ? *reinterpret_cast<const f32x4*>(src + (s0 + u) * rstride * 512) : f32x4{0.f, 0.f, 0.f, 0.f};
        float wb = 0.f;  // lane u < kBatch: weight of range s0 + u past the first 64
        if (s0 >= 64 && l < kBatch && s0 + l < ns[k])
          wb = fast_exp2(a.ml_part[(row0[k] + (s0 + l) * rstride) * 2] - mref) * inv_l;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const float wu = s0 < 64 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s0 + u))
                                   : __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wb), u));
          o += wu * q[u];
        }
      }
      if (a.o_lat) {  // latent mode: the merged latent half row is the output
        *reinterpret_cast<f32x4*>(a.o_lat + (static_cast<int64_t>(m0 + r) * a.h + i) * 512 + kHalf * kh + 4 * l) = o;
        continue;
      }
      // o_lat as a hi + lo pair of bf16 (hi = bf16(o), lo = bf16(o - hi))
      hv = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      lv = u32x2{pack_bf16x2(o[0] - __uint_as_float(hv[0] << 16), o[1] - __uint_as_float(hv[0] & 0xFFFF0000u)),
                 pack_bf16x2(o[2] - __uint_as_float(hv[1] << 16), o[3] - __uint_as_float(hv[1] & 0xFFFF0000u))};
    }
    // rows past `rows` stay zero: the MFMA below reads 32 rows
    *(lds_u32x2*)(lds_ptr(s_hi) + r * kAStride + l * 8) = hv;
    *(lds_u32x2*)(lds_ptr(s_lo) + r * kAStride + l * 8) = lv;
  }
  if (a.o_lat) return;  // uniform: no up-projection in latent mode
  __syncthreads();
  if (w >= 4) return;

  // ---- out[m][i*128 + 32w + ..] += (o_hi + o_lo)[m][half kh] · W_UV_i[half kh][32w + ..]
  f32x16 acc = {};
  const int arow = (l & 31) * kAStride + (l >> 5) * 16;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const u32x4 ah = *(lds_u32x4*)(lds_ptr(s_hi) + arow + ks * 32);
    const u32x4 al = *(lds_u32x4*)(lds_ptr(s_lo) + arow + ks * 32);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ah), as_bf16x8(bfr[ks]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(al), as_bf16x8(bfr[ks]), acc, 0, 0, 0);
  }
  const int width = a.h * 128;
  const int col = i * 128 + 32 * w + (l & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = 8 * (v / 4) + 4 * (l >> 5) + (v & 3);
    if (r >= rows) continue;
    const int m = m0 + r;
    float ov = acc[v];
    if (a.gate) {  // out = sigmoid(g) (o_0 + o_1): each half carries its factor
      float g = 0.f;
      for (int ks = 0; ks < kGateSplit; ++ks) g += a.gate[(static_cast<int64_t>(ks) * M + m) * width + col];
      ov *= 1.f / (1.f + __expf(-g));
    }
    atomicAdd(a.out + static_cast<int64_t>(m) * width + col, ov);
  }
}

hipError_t launch_combine_bf16(const CombineArgs& a, hipStream_t s) {
  const int M = a.batch * a.n_q;
  if (a.rows_per_wg < 1 || a.rows_per_wg > kWaves * kRowsPerWave || M <= 0) return hipErrorInvalidValue;
  const dim3 grid(a.h, 2, (M + a.rows_per_wg - 1) / a.rows_per_wg);
  combine_kernel<<<grid, kWaves * 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
