// Split combine + W_UV up-projection (+ sigmoid output gate) for the bf16 path.
//
// Combine: the splits of one (query, head) row carry (O_s / l_s, m_s, l_s), with
// O_s and l_s relative to their own running max m_s (base-2 units). The merge is
// the max-subtracted softmax of the interview guide §7.3 applied across splits:
//   M = max_s m_s,  L = Σ_s 2^(m_s - M) l_s,  o_lat = Σ_s 2^(m_s - M) l_s (O_s/l_s) / L,
//   lse = (M + log2 L) ln 2 (natural-log units).
// Up-projection (MLA tutorial page §3.1 and the `bhsc,hdc->bhsd` einsum of §5.1):
// out[m, i*128 + d] = o_lat[m, i, :] · W_UV_i[:, d], on v_mfma_f32_32x32x16_bf16.
// Gate (Gated-MLA page §2.6): out *= sigmoid(g), g = x · W_G per channel of the
// concatenated heads.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr int kGateSplit = 16;          // K-splits of the gate GEMM
constexpr int kHalf = 256;              // latent columns per workgroup (half of d_c)
constexpr int kSlotBytes = kHalf * 2;   // one staged half partial row (bf16)
constexpr int kSlots = 256;             // staged half rows per batch (128 KiB)
constexpr int kAStride = kHalf * 2 + 16;  // bytes per o_lat half row in LDS (padded)
}  // namespace

// grid (h, 2, ceil(M / rows_per_wg)), 256 threads. Workgroup (i, kh, mb) takes head i,
// latent columns [256 kh, 256 kh + 256) and query rows m in [mb R, mb R + R), R <= 32,
// and adds its share of the up-projection,
//   out[m][i*128 + d] += Σ_{c in half kh} o_lat[m][i][c] · W_UV_i[c][d],
// into the output with fp32 atomics (the output was zeroed by the query preparation of
// the same call). Each output element gets exactly two addends onto zero, so the sum
// does not depend on their order. Splitting the latent dimension, not the rows, reads
// each partial row and each W_UV_i once.
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  __shared__ __attribute__((aligned(1024))) char s_part[kSlots * kSlotBytes];
  __shared__ float s_w[kSlots];  // weight of each staged half row
  __shared__ int s_ns[32];       // per row: number of splits holding its tokens
  __shared__ float s_stat[32][2];  // per row: max M and 1 / L
  const int i = blockIdx.x, kh = blockIdx.y, mb = blockIdx.z;
  const int tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int M = a.batch * a.n_q;
  const int RPW = a.rows_per_wg, SB = a.splits_per_batch;
  const int m0 = mb * RPW;
  const int rows = min(RPW, M - m0);

  auto part_row = [&](int m, int sp) -> int64_t {  // row index of split sp of query row m, head i
    const int b = m / a.n_q, j = m % a.n_q;
    return ((static_cast<int64_t>(b) * a.n_splits + sp) * a.n_q + j) * a.h + i;
  };
  if (tid < rows) {
    const int kv = min(a.kv_lens[(m0 + tid) / a.n_q], a.max_kv_len);
    s_ns[tid] = kv >= a.n_q ? min((kv + a.chunk - 1) / a.chunk, a.n_splits) : 0;
  }
  __syncthreads();

  // ---- loads in the order they are needed: (m_s, l_s) of this wave's rows (rows w,
  //      w+4, ...; lane = split), then the W_UV_i fragments of this wave's 32 output
  //      columns for the 16 k-steps of half kh. Staging of the partial rows follows the
  //      statistics, so their weights are ready when the rows land.
  float2 ml0[8];
  int nsr[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int r = w + 4 * k;
    nsr[k] = r < rows ? s_ns[r] : 0;
    ml0[k] = l < nsr[k] ? *reinterpret_cast<const float2*>(a.ml_part + part_row(m0 + r, l) * 2)
                        : make_float2(-INFINITY, 0.f);
  }
  const u32x4* wv = reinterpret_cast<const u32x4*>(a.w_uv_pk) + ((static_cast<int64_t>(i) * 4 + w) * 32 + 16 * kh) * 64 + l;
  u32x4 bfr[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) bfr[ks] = wv[ks * 64];

  // ---- per row (one wave per row): M = max_s m_s, L = Σ_s 2^(m_s - M) l_s, the
  //      weights 2^(m_s - M) l_s / L of the first batch, lse. The eight rows of a wave
  //      are reduced together, so each cross-lane step has eight independent shuffles.
  float mx[8], L[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    mx[k] = ml0[k].x;
    const int r = w + 4 * k;
    for (int sp = l + 64; sp < nsr[k]; sp += 64) mx[k] = fmaxf(mx[k], a.ml_part[part_row(m0 + r, sp) * 2]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1)
#pragma unroll
    for (int k = 0; k < 8; ++k) mx[k] = fmaxf(mx[k], __shfl_xor(mx[k], o));
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float mref = mx[k] == -INFINITY ? 0.f : mx[k];
    L[k] = l < nsr[k] ? fast_exp2(ml0[k].x - mref) * ml0[k].y : 0.f;
    const int r = w + 4 * k;
    for (int sp = l + 64; sp < nsr[k]; sp += 64) {
      const int64_t pr = part_row(m0 + r, sp);
      L[k] += fast_exp2(a.ml_part[pr * 2] - mref) * a.ml_part[pr * 2 + 1];
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1)
#pragma unroll
    for (int k = 0; k < 8; ++k) L[k] += __shfl_xor(L[k], o);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int r = w + 4 * k;
    if (r >= rows) continue;
    const int m = m0 + r, ns = nsr[k];
    const float mref = mx[k] == -INFINITY ? 0.f : mx[k];
    for (int sp = l; sp < SB; sp += 64) {
      float wgt = 0.f;
      if (sp < ns && L[k] > 0.f) {
        const float2 v = sp < 64 ? ml0[k] : *reinterpret_cast<const float2*>(a.ml_part + part_row(m, sp) * 2);
        wgt = fast_exp2(v.x - mref) * v.y / L[k];
      }
      s_w[r * SB + sp] = wgt;
    }
    if (l == 0) {
      s_stat[r][0] = mref;
      s_stat[r][1] = L[k] > 0.f ? 1.f / L[k] : 0.f;
      if (kh == 0 && a.lse) a.lse[static_cast<int64_t>(m) * a.h + i] = L[k] > 0.f ? (mx[k] + __log2f(L[k])) * kLn2 : -INFINITY;
    }
  }
  int ns_max = 0;
  for (int r = 0; r < rows; ++r) ns_max = max(ns_max, s_ns[r]);

  // ---- o_lat half rows: Σ_s w_s (O_s / l_s). A wave takes two rows per pass (lanes
  //      0-31 row w + 8p, lanes 32-63 row w + 8p + 4), a lane 8 columns.
  float o[4][8];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[p][e] = 0.f;
  const int hl = l >> 5, cl = l & 31;
  for (int s0 = 0; s0 < ns_max; s0 += SB) {
    if (s0 > 0) {
      __syncthreads();  // every wave is done with the previous batch
      for (int slot = tid; slot < rows * SB; slot += 256) {  // later batches: weights
        const int r = slot / SB, sp = s0 + slot % SB;
        float wgt = 0.f;
        if (sp < s_ns[r]) {
          const int64_t pr = part_row(m0 + r, sp);
          wgt = fast_exp2(a.ml_part[pr * 2] - s_stat[r][0]) * a.ml_part[pr * 2 + 1] * s_stat[r][1];
        }
        s_w[slot] = wgt;
      }
    }
    // stage half rows (r, s0 + q) into slot r*SB + q: one wave load covers two slots
    for (int pair = w; pair * 2 < rows * SB; pair += 4) {
      const int slot = pair * 2 + hl;
      const int r = slot / SB, sp = s0 + slot % SB;
      if (slot < rows * SB && sp < s_ns[r])
        __builtin_amdgcn_global_load_lds(a.o_part + part_row(m0 + r, sp) * 512 + kh * kHalf + cl * 8,
                                         (lds_void*)(lds_ptr(s_part) + pair * 2 * kSlotBytes), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = w + 8 * p + 4 * hl;
      if (w + 8 * p >= rows) break;
      const int nq = r < rows ? min(SB, s_ns[r] - s0) : 0;
      for (int q = 0; q < nq; ++q) {
        const float wgt = s_w[r * SB + q];
        const u32x4 v = *(lds_u32x4*)(lds_ptr(s_part) + (r * SB + q) * kSlotBytes + cl * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[p][2 * e] += wgt * __uint_as_float(v[e] << 16);
          o[p][2 * e + 1] += wgt * __uint_as_float(v[e] & 0xFFFF0000u);
        }
      }
    }
  }
  __syncthreads();  // every wave is done with the staged rows

  // ---- o_lat as a hi + lo pair of bf16 rows (hi = bf16(o), lo = bf16(o - hi)), so
  //      the up-projection keeps about 16 significant bits of o_lat; rows past
  //      `rows` are zero
  char* s_hi = s_part;
  char* s_lo = s_part + 32 * kAStride;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = w + 8 * p + 4 * hl;
    u32x4 hv = {0u, 0u, 0u, 0u}, lv = {0u, 0u, 0u, 0u};
    if (r < rows) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = o[p][2 * e], x1 = o[p][2 * e + 1];
        const uint32_t h2 = pack_bf16x2(x0, x1);
        hv[e] = h2;
        lv[e] = pack_bf16x2(x0 - __uint_as_float(h2 << 16), x1 - __uint_as_float(h2 & 0xFFFF0000u));
      }
    }
    *(lds_u32x4*)(lds_ptr(s_hi) + r * kAStride + cl * 16) = hv;
    *(lds_u32x4*)(lds_ptr(s_lo) + r * kAStride + cl * 16) = lv;
  }
  __syncthreads();

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
  if (a.rows_per_wg < 1 || a.rows_per_wg > 32 || a.rows_per_wg * a.splits_per_batch > kSlots)
    return hipErrorInvalidValue;
  combine_kernel<<<dim3(a.h, 2, (M + a.rows_per_wg - 1) / a.rows_per_wg), 256, 0, s>>>(a);
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
