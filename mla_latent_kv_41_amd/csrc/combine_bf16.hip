// Split combine + W_UV up-projection (+ sigmoid output gate) for the bf16 path.
//
// Combine: the ranges s of one (query, head) row carry (O_s, m_s, l_s) in fp32,
// O_s and l_s relative to their own reference m_s (base-2 units). The merge is the
// max-subtracted softmax of the interview guide §7.3 applied across ranges:
//   M = max_s m_s,  L = Σ_s 2^(m_s - M) l_s,  o_lat = Σ_s 2^(m_s - M) O_s / L,
//   lse = (M + log2 L) ln 2 (natural-log units).
// Up-projection (MLA tutorial page §3.1 and the `bhsc,hdc->bhsd` einsum of §5.1):
// out[m, i*128 + d] = o_lat[m, i, :] · W_UV_i[:, d], on v_mfma_f32_16x16x32_bf16
// (16 query rows per block, the most a workgroup merges) with o_lat entering as a
// hi + lo pair of bf16 rows (about 16 significant bits), stored once per output
// element.
// Gate (Gated-MLA page §2.6): out *= sigmoid(g), g = x · W_G per channel of the
// concatenated heads.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr int kWaves = 8;                 // waves per workgroup
constexpr int kAStride = 512 * 2 + 16;    // bytes per merged row in LDS (512 bf16, padded)

template <int N>
struct VecT {
  typedef float T __attribute__((ext_vector_type(N)));
};
template <>
struct VecT<1> {
  typedef float T;
};

// the N bf16 halves of N floats, packed into N / 2 words (N = 1: the low half of one)
template <int N>
__device__ __forceinline__ void to_bf16_pair(const float (&x)[N], uint32_t (&hi)[(N + 1) / 2], uint32_t (&lo)[(N + 1) / 2]) {
#pragma unroll
  for (int k = 0; k < (N + 1) / 2; ++k) {
    const float x0 = x[2 * k], x1 = 2 * k + 1 < N ? x[2 * k + 1] : 0.f;
    hi[k] = pack_bf16x2(x0, x1);
    lo[k] = pack_bf16x2(x0 - __uint_as_float(hi[k] << 16), x1 - __uint_as_float(hi[k] & 0xFFFF0000u));
  }
}
}  // namespace

// grid (h, ceil(M / R)), 512 threads; R = rows_per_wg in {32, 16, 8, 4, 2, 1} query rows.
// Workgroup (i, mb) merges query rows m0 .. m0 + R - 1 of head i over all 512 latent
// columns and writes their up-projection
//   out[m][i*128 + d] = Σ_c o_lat[m][i][c] · W_UV_i[c][d]
// with plain stores: every output element has one writer, so the output needs no
// clearing and the result does not depend on timing.
//
// Merge. The statistics of a row are formed by whole waves: WPR = 8 / R waves share
// a row when R < 8, each taking 512 / WPR columns (VW = 8 / WPR per lane); with R = 8,
// 16 or 32 each wave takes one, two or four rows (columns 8l .. 8l + 7 per lane). Sequence b's
// ranges hold partial indices seq_off[b] .. seq_off[b + 1] - 1. Lane s reads range
// s's (m, l) (ranges past 64 in a loop), wave reductions give M and L, lane s forms
// the weight 2^(m_s - M) / L, and the merge reads the weights back with readlane.
// The first NB partial rows of every row go out at once, further ones NB at a time;
// ranges merge in a fixed order.
//
// Up-projection, on v_mfma_f32_16x16x32_bf16: the merged rows enter as hi + lo pairs
// of bf16 rows from LDS (rows past the workgroup's read as zeros), 16 rows per MFMA
// block. Wave w computes the 16 output columns of block w over all 512 latent columns
// (its 16 W_UV_i fragments are loaded first), applies the gate and stores. Every
// workgroup reads all of W_UV_i (128 KiB), so more rows per workgroup read it fewer
// times: a batch of many query rows takes 32.
template <int WPR, int RPW>
__global__ __launch_bounds__(kWaves * 64) void combine_kernel(CombineArgs a) {
  constexpr int VW = 8 / WPR;              // floats per lane of a row
  static_assert(RPW == 1 || WPR == 1, "several rows per wave only with whole rows");
  constexpr int NB = WPR == 1 ? 4 : 8;     // partial rows per row in flight
  constexpr int kRows = WPR == 1 ? kWaves * RPW : kWaves / WPR;  // query rows per workgroup
  constexpr int NRB = (kRows + 15) / 16;                          // 16-row MFMA blocks
  using V = typename VecT<VW>::T;
  __shared__ __attribute__((aligned(16))) char s_hi[kRows * kAStride];
  __shared__ __attribute__((aligned(16))) char s_lo[kRows * kAStride];
  const int i = blockIdx.x, mb = blockIdx.y;
  const int tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int M = a.batch * a.n_q;
  const int R = a.rows_per_wg;
  const int m0 = mb * R;
  const int rows = min(R, M - m0);
  const int64_t rstride = static_cast<int64_t>(a.n_q) * a.h;  // partial rows per range
  const bool latent = a.o_lat != nullptr;

  // W_UV_i fragments of output column block w, the 16 k-steps of 32 latent columns
  u32x4 bfr[16];
  if (!latent) {
    const u32x4* wv = reinterpret_cast<const u32x4*>(a.w_uv_pk) + ((static_cast<int64_t>(i) * kWaves + w) * 16) * 64 + l;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) bfr[ks] = wv[ks * 64];
  }

  // this wave's rows and columns
  const int sub = WPR == 1 ? 0 : w % WPR;
  const int col0 = sub * (512 / WPR) + VW * l;
  int rr[RPW], ns[RPW];
  int64_t row0[RPW];
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    rr[k] = WPR == 1 ? w + kWaves * k : w / WPR;
    ns[k] = 0;
    row0[k] = 0;
    if (rr[k] < rows) {  // uniform
      const int m = m0 + rr[k], b = m / a.n_q, j = m - b * a.n_q;
      const int p0 = a.seq_off[b];
      ns[k] = a.seq_off[b + 1] - p0;
      row0[k] = (static_cast<int64_t>(p0) * a.n_q + j) * a.h + i;
    }
  }
  // (m, l) of ranges l (< 64) and the first NB partial rows of every row
  f32x2 ml[RPW];
  V v[RPW][NB];
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    ml[k] = l < ns[k] ? *reinterpret_cast<const f32x2*>(a.ml_part + (row0[k] + l * rstride) * 2) : f32x2{-INFINITY, 0.f};
    const float* src = a.o_part + row0[k] * 512 + col0;
#pragma unroll
    for (int u = 0; u < NB; ++u) v[k][u] = u < ns[k] ? *reinterpret_cast<const V*>(src + u * rstride * 512) : V{};
  }

#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int r = rr[k];
    if (r >= rows) continue;  // uniform
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
    if (a.lse && sub == 0 && l == 0) a.lse[static_cast<int64_t>(m0 + r) * a.h + i] = L > 0.f ? (mx + __log2f(L)) * kLn2 : -INFINITY;
    // ---- merge: o = Σ_s 2^(m_s - M) / L · O_s over this lane's VW columns
    const float wl = l < ns[k] ? fast_exp2(ml[k][0] - mref) * inv_l : 0.f;  // weight of range l
    V o = V{};
#pragma unroll
    for (int u = 0; u < NB; ++u) o += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u)) * v[k][u];
    const float* src = a.o_part + row0[k] * 512 + col0;
    for (int s0 = NB; s0 < ns[k]; s0 += NB) {  // uniform: rows with more than NB ranges
      V q[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) q[u] = s0 + u < ns[k] ? *reinterpret_cast<const V*>(src + (s0 + u) * rstride * 512) : V{};
      float wb = 0.f;  // lane u < NB: weight of range s0 + u past the first 64
      if (s0 >= 64 && l < NB && s0 + l < ns[k]) wb = fast_exp2(a.ml_part[(row0[k] + (s0 + l) * rstride) * 2] - mref) * inv_l;
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const float wu = s0 < 64 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s0 + u))
                                 : __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wb), u));
        o += wu * q[u];
      }
    }
    if (latent) {  // the merged latent row is the output
      *reinterpret_cast<V*>(a.o_lat + (static_cast<int64_t>(m0 + r) * a.h + i) * 512 + col0) = o;
      continue;
    }
    // o as a hi + lo pair of bf16 (hi = bf16(o), lo = bf16(o - hi)) into the MFMA rows
    float x[VW];
    __builtin_memcpy(x, &o, sizeof(x));
    uint32_t hi[(VW + 1) / 2], lo[(VW + 1) / 2];
    to_bf16_pair<VW>(x, hi, lo);
    const int boff = r * kAStride + col0 * 2;
    if constexpr (VW == 8) {
      *(lds_u32x4*)(lds_ptr(s_hi) + boff) = u32x4{hi[0], hi[1], hi[2], hi[3]};
      *(lds_u32x4*)(lds_ptr(s_lo) + boff) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    } else if constexpr (VW == 4) {
      *(lds_u32x2*)(lds_ptr(s_hi) + boff) = u32x2{hi[0], hi[1]};
      *(lds_u32x2*)(lds_ptr(s_lo) + boff) = u32x2{lo[0], lo[1]};
    } else if constexpr (VW == 2) {
      *(__attribute__((address_space(3))) uint32_t*)(lds_ptr(s_hi) + boff) = hi[0];
      *(__attribute__((address_space(3))) uint32_t*)(lds_ptr(s_lo) + boff) = lo[0];
    } else {
      *(__attribute__((address_space(3))) uint16_t*)(lds_ptr(s_hi) + boff) = static_cast<uint16_t>(hi[0]);
      *(__attribute__((address_space(3))) uint16_t*)(lds_ptr(s_lo) + boff) = static_cast<uint16_t>(lo[0]);
    }
  }
  if (latent) return;  // uniform: no up-projection in latent mode
  __syncthreads();

  // ---- (o_hi + o_lo)[rows][:] · W_UV_i[:][16 w + ..]; A row l%16 (zero past the
  //      workgroup's rows), row 16 rb + l%16 of block rb, k = 32 ks + 8 (l/16) + e;
  //      the hi and lo products run as two accumulation chains, added at the end
  f32x4 acc_h[NRB], acc_l[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) acc_h[rb] = acc_l[rb] = f32x4{};
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int ar = 16 * rb + (l & 15);
      const int aoff = ar * kAStride + (l >> 4) * 16 + ks * 64;
      u32x4 ah = {0u, 0u, 0u, 0u}, al = {0u, 0u, 0u, 0u};
      if (ar < rows) {
        ah = *(lds_u32x4*)(lds_ptr(s_hi) + aoff);
        al = *(lds_u32x4*)(lds_ptr(s_lo) + aoff);
      }
      acc_h[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah), as_bf16x8(bfr[ks]), acc_h[rb], 0, 0, 0);
      acc_l[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(al), as_bf16x8(bfr[ks]), acc_l[rb], 0, 0, 0);
    }
  }
  // D lane l: output column 16 w + l % 16, rows 16 rb + 4 (l / 16) + v
  const int width = a.h * 128;
  const int col = i * 128 + 16 * w + (l & 15);
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = 16 * rb + 4 * (l >> 4) + v;
    if (r >= rows) continue;
    const int m = m0 + r;
    float ov = acc_h[rb][v] + acc_l[rb][v];
    if (a.gate) {  // out = sigmoid(g) o
      float g = 0.f;
      for (int ks = 0; ks < kGateSplit; ++ks) g += a.gate[(static_cast<int64_t>(ks) * M + m) * width + col];
      ov *= 1.f / (1.f + __expf(-g));
    }
    a.out[static_cast<int64_t>(m) * width + col] = ov;
  }
}

hipError_t launch_combine_bf16(const CombineArgs& a, hipStream_t s) {
  const int M = a.batch * a.n_q;
  const int R = a.rows_per_wg;
  if (!(R == 32 || R == 16 || R == 8 || R == 4 || R == 2 || R == 1) || M <= 0) return hipErrorInvalidValue;
  const dim3 grid(a.h, (M + R - 1) / R);
  if (R == 32) combine_kernel<1, 4><<<grid, kWaves * 64, 0, s>>>(a);
  else if (R == 16) combine_kernel<1, 2><<<grid, kWaves * 64, 0, s>>>(a);
  else if (R == 8) combine_kernel<1, 1><<<grid, kWaves * 64, 0, s>>>(a);
  else if (R == 4) combine_kernel<2, 1><<<grid, kWaves * 64, 0, s>>>(a);
  else if (R == 2) combine_kernel<4, 1><<<grid, kWaves * 64, 0, s>>>(a);
  else combine_kernel<8, 1><<<grid, kWaves * 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
