// Fused latent append: cache row [ gain ⊙ RMSNorm(h · W_DKV) ‖ RoPE(h · W_KR, pos) ]
// written straight from the hidden state h of each new token.
//
// The down-projection c_KV = h · W_DKV (tutorial page §2.2), an RMSNorm over the
// d_c latent right after it (tutorial page §6.3), and the decoupled key from its
// own d_model → d_rope projection of the same input (interview guide §6.2, `MLA`
// module), cached already rotated (linear-algebra page, "解耦 RoPE").
//
// bf16: the split-K matrix-core product (gemm_bf16.hip) writes fp32 partial sums
// of both projections side by side, [ksplit][M][d_c + d_r]; latent_finish_kernel
// adds the splits in a fixed order, normalises, rotates, rounds once and stores.
// fp32: latent_finish_kernel computes the products itself with fp32 FMAs.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr int kMaxRow = 1280;  // d_c + d_r: fp32 path d_c <= 1024, d_r <= 256

__device__ __forceinline__ void store_out(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_out(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16_bits(v); }
__device__ __forceinline__ void store_out(float* p, int64_t i, double v) { p[i] = static_cast<float>(v); }
__device__ __forceinline__ void store_out(uint16_t* p, int64_t i, double v) { p[i] = f64_to_bf16_bits(v); }
}  // namespace

// packed[k][n] = n < d_c ? w_dkv[k][n] : w_kr[k][n - d_c]; grid d_model, any block size.
template <typename T>
__global__ void pack_down_kernel(const T* __restrict__ w_dkv, const T* __restrict__ w_kr, T* __restrict__ packed,
                                 int d_c, int d_r) {
  const int64_t k = blockIdx.x;
  const int N = d_c + d_r;
  for (int n = threadIdx.x; n < N; n += blockDim.x)
    packed[k * N + n] = n < d_c ? w_dkv[k * d_c + n] : w_kr[k * d_r + (n - d_c)];
}

hipError_t launch_pack_down(int dtype, const void* w_dkv, const void* w_kr, void* packed, int d_model, int d_c,
                            int d_r, hipStream_t s) {
  if (d_model <= 0 || d_c + d_r <= 0) return hipErrorInvalidValue;
  if (dtype == 0)
    pack_down_kernel<float><<<d_model, 256, 0, s>>>(static_cast<const float*>(w_dkv),
                                                   static_cast<const float*>(w_kr), static_cast<float*>(packed),
                                                   d_c, d_r);
  else
    pack_down_kernel<uint16_t><<<d_model, 256, 0, s>>>(static_cast<const uint16_t*>(w_dkv),
                                                      static_cast<const uint16_t*>(w_kr),
                                                      static_cast<uint16_t*>(packed), d_c, d_r);
  return hipGetLastError();
}

// One workgroup (256 threads) per new token m = b * n_new + j, at position
// pos0[b] + j. Rows whose position or block id is out of range are skipped.
template <typename T>
__global__ __launch_bounds__(256) void latent_finish_kernel(ProjArgs a) {
  __shared__ float s_row[kMaxRow];
  __shared__ float s_red[4];
  const int m = blockIdx.x, b = m / a.n_new, j = m % a.n_new;
  const int tid = threadIdx.x;
  const int N = a.d_c + a.d_r;

  if constexpr (sizeof(T) == 4) {
    // fp32: the products, k ascending, one output column per thread at a time
    const float* h = static_cast<const float*>(a.hidden) + static_cast<int64_t>(m) * a.d_model;
    const float* w = static_cast<const float*>(a.w_down);
    for (int n = tid; n < N; n += 256) {
      float v = 0.f;
      for (int k = 0; k < a.d_model; ++k) v = fmaf(h[k], w[static_cast<int64_t>(k) * N + n], v);
      s_row[n] = v;
    }
  } else {
    // bf16: sum of the split partials, split 0 first
    for (int n = tid; n < N; n += 256) {
      float v = 0.f;
      for (int ks = 0; ks < a.ksplit; ++ks) v += a.part[(static_cast<int64_t>(ks) * a.M + m) * N + n];
      s_row[n] = v;
    }
  }
  __syncthreads();

  // mean square of the latent part
  float ss = 0.f;
  for (int n = tid; n < a.d_c; n += 256) ss = fmaf(s_row[n], s_row[n], ss);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if (tid % 64 == 0) s_red[tid / 64] = ss;
  __syncthreads();
  const float total = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
  const float inv = 1.0f / sqrtf(total / static_cast<float>(a.d_c) + a.eps);

  // destination slot (uniform per workgroup)
  const int64_t pos = static_cast<int64_t>(a.pos0[b]) + j;
  const CacheRef& c = a.cache;
  int64_t slot;
  if (c.block_table == nullptr) {
    if (pos < 0 || pos >= c.t_max) return;
    slot = static_cast<int64_t>(b) * c.t_max + pos;
  } else {
    if (pos < 0) return;
    const int64_t blk = pos / c.block_size;
    if (blk >= c.max_blocks) return;
    const int32_t id = c.block_table[static_cast<int64_t>(b) * c.max_blocks + blk];
    if (id < 0 || id >= c.n_blocks) return;
    slot = static_cast<int64_t>(id) * c.block_size + pos % c.block_size;
  }
  T* dst = static_cast<T*>(const_cast<void*>(c.data)) + slot * N;

  for (int n = tid; n < a.d_c; n += 256) {
    const float g = a.gain ? a.gain[n] : 1.0f;
    store_out(dst, n, g * (s_row[n] * inv));
  }
  // RoPE on the pairs (x[2k], x[2k+1]) with angle pos * base^(-2k/d_r), in fp64,
  // rounded once to the cache type
  for (int k = tid; k < a.d_r / 2; k += 256) {
    const double inv_freq = pow(a.rope_base, -2.0 * k / a.d_r);
    double sn, cs;
    sincos(static_cast<double>(pos) * inv_freq, &sn, &cs);
    const double x0 = s_row[a.d_c + 2 * k], x1 = s_row[a.d_c + 2 * k + 1];
    store_out(dst, a.d_c + 2 * k, x0 * cs - x1 * sn);
    store_out(dst, a.d_c + 2 * k + 1, x0 * sn + x1 * cs);
  }
}

hipError_t launch_latent_finish(int dtype, const ProjArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.d_c <= 0 || a.d_r < 0 || a.d_c + a.d_r > kMaxRow || a.n_new <= 0) return hipErrorInvalidValue;
  if (dtype == 0)
    latent_finish_kernel<float><<<a.M, 256, 0, s>>>(a);
  else
    latent_finish_kernel<uint16_t><<<a.M, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
