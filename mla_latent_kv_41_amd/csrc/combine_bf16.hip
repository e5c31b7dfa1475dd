// Split combine + W_UV up-projection (+ sigmoid output gate) for the bf16 path.
//
// Combine: the splits of one (query, head) row carry (O_s, m_s, l_s) with O_s and
// l_s relative to their own running max m_s (base-2 units). The merge is the
// max-subtracted softmax of the interview guide §7.3 applied across splits:
//   M = max_s m_s,  L = Σ_s 2^(m_s - M) l_s,  o_lat = Σ_s 2^(m_s - M) O_s / L,
//   lse = (M + log2 L) ln 2 (natural-log units).
// Up-projection (MLA tutorial page §3.1 and the `bhsc,hdc->bhsd` einsum of §5.1):
// out[m, i*128 + d] = o_lat[m, i, :] · W_UV_i[:, d], on v_mfma_f32_32x32x16_bf16.
// Gate (Gated-MLA page §2.6): out *= sigmoid(g), g = x · W_G per channel of the
// concatenated heads.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr int kRows = 32;               // query rows per workgroup
constexpr int kOStride = 512 * 2 + 16;  // bytes per o_lat row in LDS (padded)
constexpr int kGateSplit = 16;          // K-splits of the gate GEMM
}  // namespace

// grid (h, ceil(M / 32)), 256 threads.
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  __shared__ __attribute__((aligned(16))) char s_o[kRows * kOStride];
  const int i = blockIdx.x, mb = blockIdx.y;
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
  const int M = a.batch * a.n_q;

  // ---- phase 1: merge splits, one wave per row (rows w, w+4, ...)
  for (int r = w; r < kRows; r += 4) {
    const int m = kRows * mb + r;
    uint32_t packed[4] = {0u, 0u, 0u, 0u};
    if (m < M) {
      const int b = m / a.n_q, j = m % a.n_q;
      const int kv = min(a.kv_lens[b], a.max_kv_len);
      const int ns = kv >= a.n_q ? min((kv + a.chunk - 1) / a.chunk, a.n_splits) : 0;
      const int64_t row_stride = static_cast<int64_t>(a.n_q) * a.h;  // rows between splits
      const int64_t row0 = (static_cast<int64_t>(b) * a.n_splits * a.n_q + j) * a.h + i;
      float M_ = -INFINITY;
      for (int s = 0; s < ns; ++s) M_ = fmaxf(M_, a.ml_part[(row0 + s * row_stride) * 2]);
      const float mref = M_ == -INFINITY ? 0.f : M_;
      float L = 0.f;
      float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < ns; ++s) {
        const int64_t rr = row0 + s * row_stride;
        const float ws = fast_exp2(a.ml_part[rr * 2] - mref);
        L += ws * a.ml_part[rr * 2 + 1];
        const f32x4* op = reinterpret_cast<const f32x4*>(a.o_part + rr * 512) + 2 * l;
        const f32x4 v0 = op[0], v1 = op[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] += ws * v0[e];
          o[4 + e] += ws * v1[e];
        }
      }
      const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) packed[e] = pack_bf16x2(o[2 * e] * inv, o[2 * e + 1] * inv);
      if (a.lse && l == 0) a.lse[static_cast<int64_t>(m) * a.h + i] = L > 0.f ? (M_ + __log2f(L)) * kLn2 : -INFINITY;
    }
    u32x4 pv = {packed[0], packed[1], packed[2], packed[3]};
    *reinterpret_cast<u32x4*>(s_o + r * kOStride + l * 16) = pv;
  }
  __syncthreads();

  // ---- phase 2: out[m][32w + ..] = o_lat[m][:] · W_UV_i[:, 32w + ..]
  const u32x4* wv = reinterpret_cast<const u32x4*>(a.w_uv_pk) + ((static_cast<int64_t>(i) * 4 + w) * 32) * 64 + l;
  const char* arow = s_o + (l & 31) * kOStride + (l >> 5) * 16;
  f32x16 acc = {};
#pragma unroll 8
  for (int ks = 0; ks < 32; ++ks) {
    const u32x4 af = *reinterpret_cast<const u32x4*>(arow + ks * 32);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af), as_bf16x8(wv[ks * 64]), acc, 0, 0, 0);
  }
  const int width = a.h * 128;
  const int col = i * 128 + 32 * w + (l & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int m = kRows * mb + 8 * (v / 4) + 4 * (l >> 5) + (v & 3);
    if (m >= M) continue;
    float o = acc[v];
    if (a.gate) {
      float g = 0.f;
      for (int ks = 0; ks < kGateSplit; ++ks) g += a.gate[(static_cast<int64_t>(ks) * M + m) * width + col];
      o *= 1.f / (1.f + __expf(-g));
    }
    a.out[static_cast<int64_t>(m) * width + col] = o;
  }
}

hipError_t launch_combine_bf16(const CombineArgs& a, hipStream_t s) {
  const int M = a.batch * a.n_q;
  combine_kernel<<<dim3(a.h, (M + kRows - 1) / kRows), 256, 0, s>>>(a);
  return hipGetLastError();
}

// Gate logits, split over K: g[ks][m][n] = Σ_{k in split ks} x[m][k] W_G[k][n].
// grid (N / 512, 16), 256 threads, two columns per thread, M <= 32 rows.
__global__ __launch_bounds__(256) void gate_kernel(GateArgs a) {
  __shared__ float s_x[32 * 256];
  const int n = (blockIdx.x * 256 + threadIdx.x) * 2;
  const int kper = a.d_model / kGateSplit;
  const int k0 = blockIdx.y * kper;
  for (int mm0 = 0; mm0 < a.M; mm0 += 32) {
    const int rows = min(32, a.M - mm0);
    for (int kb = 0; kb < kper; kb += 256) {
      const int kn = min(256, kper - kb);
      __syncthreads();
      for (int e = threadIdx.x; e < rows * 256; e += 256) {
        const int mm = e / 256, kk = e % 256;
        s_x[e] = kk < kn ? bf16_bits_to_f32(a.x[static_cast<int64_t>(mm0 + mm) * a.d_model + k0 + kb + kk]) : 0.f;
      }
      __syncthreads();
      float acc0[32], acc1[32];
#pragma unroll
      for (int mm = 0; mm < 32; ++mm) acc0[mm] = acc1[mm] = 0.f;
      if (n < a.N) {
        const uint32_t* wp = reinterpret_cast<const uint32_t*>(a.w_g + static_cast<int64_t>(k0 + kb) * a.N + n);
        for (int kk = 0; kk < kn; ++kk) {
          const uint32_t wbits = wp[static_cast<int64_t>(kk) * (a.N / 2)];
          const float w0 = __uint_as_float(wbits << 16), w1 = __uint_as_float(wbits & 0xFFFF0000u);
#pragma unroll
          for (int mm = 0; mm < 32; ++mm) {
            const float xv = s_x[mm * 256 + kk];
            acc0[mm] = fmaf(xv, w0, acc0[mm]);
            acc1[mm] = fmaf(xv, w1, acc1[mm]);
          }
        }
        for (int mm = 0; mm < rows; ++mm) {
          float* gp = a.g + (static_cast<int64_t>(blockIdx.y) * a.M + mm0 + mm) * a.N + n;
          if (kb == 0) {
            gp[0] = acc0[mm];
            gp[1] = acc1[mm];
          } else {
            gp[0] += acc0[mm];
            gp[1] += acc1[mm];
          }
        }
      }
    }
  }
}

hipError_t launch_gate_bf16(const GateArgs& a, hipStream_t s) {
  gate_kernel<<<dim3((a.N / 2 + 255) / 256, kGateSplit), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
