// Weight absorption packing and query preparation for the bf16 matrix-core path.
//
// Absorption (MLA tutorial page §3.1, §3.2 and the `bhsd,hcd->bhsc` einsum of
// §5.1): W_UK is folded into the query, q_abs[m, i, :] = q_nope[m, i, :] · W_UK_iᵀ,
// a [1 x 128] · [128 x 512] product per head, batched over all M = B * n_q query
// rows so each W_UK_i is read once per step. The decoupled query key is rotated
// (interview guide §6.2; linear-algebra page "解耦 RoPE"). Both parts are scaled
// by scale * log2(e), so the attention kernel works in base-2 exponent units.
//
// Packing (done once at load, tutorial §3.2): W_UK and W_UV are re-laid out per
// head in the exact per-lane fragment order of v_mfma_f32_32x32x16_bf16, so every
// weight load in the hot kernels is one contiguous 1 KiB wave transaction.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

// Fragment order (64 lanes x 8 bf16 = 1 KiB per fragment):
//   W_UK (B operand of D[m][c] = q_nope[m][:] · W_UK_i[c][:]):
//     frag (i, nb < 16, ks < 8), lane l: W_UK[32nb + l%32][i*128 + 16ks + 8(l/32) + e]
//   W_UV (B operand of D[m][d] = o_lat[m][:] · W_UV_i[:][d]):
//     frag (i, nb < 4, ks < 32), lane l: W_UV[16ks + 8(l/32) + e][i*128 + 32nb + l%32]
__global__ void pack_kernel(const uint16_t* __restrict__ w_uk, const uint16_t* __restrict__ w_uv,
                            uint16_t* __restrict__ packed, int h) {
  const int64_t per = static_cast<int64_t>(h) * 8192;  // lanes per region
  const int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= 2 * per) return;
  const int64_t width = static_cast<int64_t>(h) * 128;
  uint16_t v[8];
  if (g < per) {
    const int l = g % 64;
    const int64_t f = g / 64;
    const int ks = f % 8, nb = (f / 8) % 16, i = static_cast<int>(f / 128);
    const int64_t r = 32 * nb + l % 32;
    const int64_t c0 = static_cast<int64_t>(i) * 128 + 16 * ks + 8 * (l / 32);
    for (int e = 0; e < 8; ++e) v[e] = w_uk[r * width + c0 + e];
  } else {
    const int64_t gg = g - per;
    const int l = gg % 64;
    const int64_t f = gg / 64;
    const int ks = f % 32, nb = (f / 32) % 4, i = static_cast<int>(f / 128);
    const int64_t col = static_cast<int64_t>(i) * 128 + 32 * nb + l % 32;
    for (int e = 0; e < 8; ++e) v[e] = w_uv[(16 * ks + 8 * (l / 32) + e) * width + col];
  }
  u32x4 o;
  for (int e = 0; e < 4; ++e) o[e] = static_cast<uint32_t>(v[2 * e]) | (static_cast<uint32_t>(v[2 * e + 1]) << 16);
  *reinterpret_cast<u32x4*>(packed + g * 8) = o;
}

hipError_t launch_pack_bf16(const uint16_t* w_uk, const uint16_t* w_uv, uint16_t* packed, int h,
                            hipStream_t s) {
  const int64_t n = static_cast<int64_t>(h) * 8192 * 2;
  pack_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), 256, 0, s>>>(w_uk, w_uv, packed, h);
  return hipGetLastError();
}

// Q_cat is written in the attention kernel's B-fragment order, so each of its
// fragment loads is one contiguous 1 KiB wave read: element (row m, head i,
// column c) sits in workgroup (b, hg) = (m / n_q, i / HG) with HG = R / n_q heads
// per workgroup of R rows, at row r = (m % n_q) HG + i % HG, wave r / 32, k-step
// c / 16, lane (r % 32) + 32 ((c / 8) % 2), element c % 8.
__device__ __forceinline__ int64_t qfrag_off(const QPrepArgs& a, int m, int i, int c) {
  const int KS = (512 + a.d_r) / 16;
  const int HG = a.rows_per_wg / a.n_q;
  const int hgroups = a.h / HG;
  const int nw = a.rows_per_wg / 32;
  const int b = m / a.n_q, j = m % a.n_q;
  const int hg = i / HG, r = j * HG + i % HG;
  const int lane = (r & 31) + 32 * ((c >> 3) & 1);
  return ((((static_cast<int64_t>(b) * hgroups + hg) * nw + (r >> 5)) * KS + (c >> 4)) * 64 + lane) * 8 + (c & 7);
}

// grid (h, 4): head i, quarter cq of the 512 latent columns; 4 waves, wave w owns
// the 32 columns of block nb = 4cq + w and loops over 32-row blocks of M. The
// 32 x 128 bf16 result block is staged in LDS and written out as 16-byte chunks in
// the fragment order above.
__global__ __launch_bounds__(256) void qprep_kernel(QPrepArgs a) {
  constexpr int kStride = 128 * 2 + 16;  // bytes per staged row (padded)
  __shared__ __attribute__((aligned(16))) char s_q[32 * kStride];
  const int i = blockIdx.x, cq = blockIdx.y;
  const int tid = threadIdx.x, l = tid % 64;
  // zero this head's quarter of the output columns (the combine adds into them)
  for (int idx = tid; idx < a.M * 32; idx += blockDim.x)
    a.out[static_cast<int64_t>(idx / 32) * a.h * 128 + i * 128 + 32 * cq + idx % 32] = 0.f;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int nb = 4 * cq + w;
  const u32x4* wk = reinterpret_cast<const u32x4*>(a.w_uk_pk) + ((static_cast<int64_t>(i) * 16 + nb) * 8) * 64 + l;
  u32x4 bfr[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) bfr[ks] = wk[ks * 64];
  for (int mb = 0; mb * 32 < a.M; ++mb) {
    const int m_a = 32 * mb + l % 32;
    f32x16 acc = {};
    const u32x4* qn = reinterpret_cast<const u32x4*>(a.q_nope + (static_cast<int64_t>(m_a) * a.h + i) * 128) + (l / 32);
    u32x4 af[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) af[ks] = m_a < a.M ? qn[2 * ks] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[ks]), as_bf16x8(bfr[ks]), acc, 0, 0, 0);
    // stage: row 8(v/4) + 4(l/32) + v%4, column 32w + l%32 of the block
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 8 * (v / 4) + 4 * (l / 32) + v % 4;
      *(__attribute__((address_space(3))) uint16_t*)(lds_ptr(s_q) + r * kStride + (32 * w + (l & 31)) * 2) =
          f32_to_bf16_bits(acc[v] * a.qscale);
    }
    __syncthreads();
    // 32 rows x 16 chunks of 16 B: two chunks per thread
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int q = tid + 256 * k, r = q / 16, ch = q % 16;
      const int m = 32 * mb + r;
      if (m < a.M) {
        const u32x4 v = *(lds_u32x4*)(lds_ptr(s_q) + r * kStride + ch * 16);
        *reinterpret_cast<u32x4*>(a.q_cat + qfrag_off(a, m, i, 128 * cq + ch * 8)) = v;
      }
    }
  }
  if (a.d_r == 0) return;
  // RoPE of q_R for rows m = cq (mod 4): angle pos * inv_freq[k], formed and reduced
  // modulo 2π in fp64; sine and cosine of the reduced angle in fp32.
  const int half = a.d_r / 2;
  const int rows = (a.M - cq + 3) / 4;
  for (int idx = tid; idx < rows * half; idx += blockDim.x) {
    const int m = 4 * (idx / half) + cq, k = idx % half;
    const int b = m / a.n_q, j = m % a.n_q;
    const int kv = min(a.kv_lens[b], a.max_kv_len);
    const double theta = static_cast<double>(kv - a.n_q + j) * a.inv_freq[k];
    const double red = theta - 6.283185307179586 * rint(theta * 0.15915494309189535);
    float sn, cs;
    sincosf(static_cast<float>(red), &sn, &cs);
    const uint16_t* qr = a.q_rope + (static_cast<int64_t>(m) * a.h + i) * a.d_r;
    const float x0 = bf16_bits_to_f32(qr[2 * k]), x1 = bf16_bits_to_f32(qr[2 * k + 1]);
    uint16_t* dst = a.q_cat + qfrag_off(a, m, i, 512 + 2 * k);  // columns 512+2k, 513+2k share a chunk
    dst[0] = f32_to_bf16_bits((x0 * cs - x1 * sn) * a.qscale);
    dst[1] = f32_to_bf16_bits((x0 * sn + x1 * cs) * a.qscale);
  }
}

hipError_t launch_qprep_bf16(const QPrepArgs& a, hipStream_t s) {
  qprep_kernel<<<dim3(a.h, 4), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
