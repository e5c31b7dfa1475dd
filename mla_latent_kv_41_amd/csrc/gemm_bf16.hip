// Split-K bf16 product on the matrix cores (gate logits; fused-append projections).
#include "common.hpp"
#include "launch.hpp"

namespace mla {

// Split-K product g[ks][m][n] = Σ_{k in split ks} x[m][k] W[k][n], on the matrix
// cores as Dᵀ[n][m] = Σ_k Wᵀ[n][k] xᵀ[k][m]. Used for the gate logits (W = W_G) and
// for the fused append's down-projections (W = [W_DKV ‖ W_KR]).
// grid (ceil(N / 128), ksplit), 256 threads, two workgroups per CU. Workgroup (nb, ks)
// takes columns [128 nb, +128) and the K / ksplit k of split ks, 256 at a time. Its W
// block is staged row-major in LDS by direct-to-LDS loads (each 256-byte row's 16-byte
// chunk c at position c ^ 4 (row % 4), so both the loads and the reads below are
// free of bank conflicts). Wave w takes columns 32w .. 32w + 31: its A operand
// (32 columns x 16 k) comes from transposing reads (each 16-lane group reads a
// 4-row x 16-column block row-wise and receives it column-wise), two per k-step,
// the second 8 rows down; so the K index 8h + e (h = lane / 32) of k-step kk is
// k = 16 kk + 4h + (e % 4) + 8 (e / 4), and the B operand xᵀ follows that order.
// Rows m past M are zero; M is taken 32 rows at a time. When N is not a multiple of
// 128, the last block's staged rows run into the next row of W (or past its end,
// where the buffer bound reads zeros); the columns past N are computed and dropped.
constexpr int kGemmCols = 128;
__global__ __launch_bounds__(256) void splitk_gemm_kernel(GemmArgs a) {
  constexpr int kRowB = kGemmCols * 2;  // staged W_G row
  constexpr int kChunk = 256;           // staged rows (k) at a time
  __shared__ __attribute__((aligned(1024))) char s_wg[kChunk * kRowB];
  const int nb = blockIdx.x, ks = blockIdx.y;
  const int tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int kper = a.K / a.ksplit;  // a multiple of 16
  const int k0 = ks * kper, n0 = nb * kGemmCols;
  const u32x4 rs = buffer_rsrc(a.w, static_cast<uint32_t>(static_cast<int64_t>(a.K) * a.N * 2));
  // staging: wave load q fills LDS [1 KiB q, +1 KiB) = rows 4q .. 4q+3 of the chunk;
  // lane l takes row 4q + l/16, position l%16
  const int rsub = l >> 4, chunk = (l & 15) ^ (4 * rsub);  // rows 4q + rsub have row % 4 == rsub
  const uint32_t lane_off = static_cast<uint32_t>((static_cast<int64_t>(k0 + rsub) * a.N + n0 + 8 * chunk) * 2);
  // transposing-read offsets: 16-lane group g, lane i reads row 4(g/2) + i/4 (+8 for
  // the second read), columns 32w + 16(g%2) + 4(i%4) .. +3
  const int g = l >> 4, i = l & 15;
  const int rr = 4 * (g >> 1) + (i >> 2);
  const int cchunk = 4 * w + 2 * (g & 1) + ((i & 3) >> 1);
  const int off_lo = rr * kRowB + ((cchunk ^ (4 * (i >> 2))) << 4) + ((i & 1) << 3);
  const int h = l >> 5;

  for (int mm0 = 0; mm0 < a.M; mm0 += 32) {
    const int m = mm0 + (l & 31);
    const uint16_t* xr = a.x + static_cast<int64_t>(min(m, a.M - 1)) * a.K + k0 + 4 * h;
    f32x16 acc = {};
    for (int kc = 0; kc < kper; kc += kChunk) {
      const int rows = min(kChunk, kper - kc);
      if (kc > 0 || mm0 > 0) __syncthreads();  // every wave is done with the previous chunk
#pragma unroll 1
      for (int q = w; 4 * q < rows; q += 4)
        dma_b128(rs, lane_off, static_cast<uint32_t>(kc + 4 * q) * static_cast<uint32_t>(a.N) * 2u,
                 lds_addr(s_wg) + q * 1024);
      // B operand xᵀ for the chunk, loaded while the block lands: lane l holds row m,
      // k = kc + 16kk + 4h + 0..3 and + 8
      u32x4 bx[kChunk / 16];
#pragma unroll
      for (int kk = 0; kk < kChunk / 16; ++kk) {
        bx[kk] = u32x4{0u, 0u, 0u, 0u};
        if (kk < rows / 16 && m < a.M) {
          const u32x2 xl = *reinterpret_cast<const u32x2*>(xr + kc + 16 * kk);
          const u32x2 xh = *reinterpret_cast<const u32x2*>(xr + kc + 16 * kk + 8);
          bx[kk] = u32x4{xl[0], xl[1], xh[0], xh[1]};
        }
      }
      wait_vm<0>();
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kChunk / 16; ++kk) {
        if (kk < rows / 16) {  // uniform
          lds_char* tb = lds_ptr(s_wg) + kk * 16 * kRowB;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tb + off_lo));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tb + off_lo + 8 * kRowB));
          const i16x8 af = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af), as_bf16x8(bx[kk]), acc, 0, 0, 0);
        }
      }
    }
    // Dᵀ: lane l holds column m = mm0 + l%32 and rows n = 8j + 4h + 0..3 (values 4j .. 4j+3)
    if (m < a.M && n0 + 32 * w < a.N) {  // N is a multiple of 32
      float* gp = a.g + (static_cast<int64_t>(ks) * a.M + m) * a.N + n0 + 32 * w + 4 * h;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4*>(gp + 8 * j) = f32x4{acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]};
    }
  }
}

hipError_t launch_splitk_gemm_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.ksplit <= 0 || a.ksplit > 65535 || a.K % (a.ksplit * 16) != 0 || a.N <= 0 || a.N % 32 != 0)
    return hipErrorInvalidValue;
  if (static_cast<int64_t>(a.K) * a.N * 2 >= (int64_t(1) << 32)) return hipErrorInvalidValue;
  splitk_gemm_kernel<<<dim3((a.N + kGemmCols - 1) / kGemmCols, a.ksplit), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
