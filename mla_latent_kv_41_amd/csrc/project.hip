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
// A call moves the weights once (4.7 MB at d_model 4096) and little else, so it
// is bound by memory latency and launch overhead more than by bandwidth.
// fp32: latent_finish_kernel computes the products itself with fp32 FMAs.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr int kMaxRow = 1280;  // d_c + d_r: fp32 path d_c <= 1024, d_r <= 256

__device__ __forceinline__ void store_out(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_out(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16_bits(v); }
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

// One workgroup (512 threads) per new token m = b * n_new + j, at position
// pos0[b] + j. Rows whose position or block id is out of range are skipped.
//
// bf16: the row's split partials are G = N / 4 groups of four columns. Thread t < L G
// (L = 512 / G threads per group) takes group t % G and the splits p, p + L, p + 2L, ...
// (p = t / G), issuing them sixteen at a time as independent 16-byte loads; the L
// subtotals of a group are then added in the order p = 0, 1, .., L - 1. The order of
// every addition is fixed, so the result does not depend on timing.
constexpr int kFinishThreads = 512;
template <typename T>
__global__ __launch_bounds__(kFinishThreads) void latent_finish_kernel(ProjArgs a) {
  __shared__ float s_row[kMaxRow];
  __shared__ f32x4 s_sub[kFinishThreads];
  __shared__ float s_red[kFinishThreads / 64];
  const int m = blockIdx.x, b = m / a.n_new, j = m % a.n_new;
  const int tid = threadIdx.x;
  const int N = a.d_c + a.d_r;
  // the position, the destination block and the gain are loaded first, so that
  // their round trips overlap the partial sums' instead of following them
  const int64_t pos = static_cast<int64_t>(a.pos0[b]) + j;
  const CacheRef& c = a.cache;
  int64_t slot = -1;
  if (c.block_table == nullptr) {
    if (pos >= 0 && pos < c.t_max) slot = static_cast<int64_t>(b) * c.t_max + pos;
  } else if (pos >= 0 && pos / c.block_size < c.max_blocks) {
    const int32_t id = c.block_table[static_cast<int64_t>(b) * c.max_blocks + pos / c.block_size];
    if (id >= 0 && id < c.n_blocks) slot = static_cast<int64_t>(id) * c.block_size + pos % c.block_size;
  }
  float gain[kMaxRow / kFinishThreads + 1];
#pragma unroll
  for (int q = 0; q <= kMaxRow / kFinishThreads; ++q) {
    const int n = tid + q * kFinishThreads;
    gain[q] = (a.gain && n < a.d_c) ? a.gain[n] : 1.0f;
  }

  if constexpr (sizeof(T) == 4) {
    // fp32: the products, k ascending, one output column per thread at a time
    const float* h = static_cast<const float*>(a.hidden) + static_cast<int64_t>(m) * a.d_model;
    const float* w = static_cast<const float*>(a.w_down);
    for (int n = tid; n < N; n += kFinishThreads) {
      float v = 0.f;
      for (int k = 0; k < a.d_model; ++k) v = fmaf(h[k], w[static_cast<int64_t>(k) * N + n], v);
      s_row[n] = v;
    }
  } else {
    const int G = N / 4;  // N is a multiple of 32 on this path
    const int L = kFinishThreads / G;
    if (tid < L * G) {
      const int g = tid % G, p = tid / G;
      const f32x4* src = reinterpret_cast<const f32x4*>(a.part + static_cast<int64_t>(m) * N) + g;
      const int64_t split_stride = static_cast<int64_t>(a.M) * N / 4;  // in f32x4
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int base = p; base < a.ksplit; base += 16 * L) {  // once for up to 16 L splits
        f32x4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int ks = base + u * L;
          v[u] = ks < a.ksplit ? src[ks * split_stride] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) acc += v[u];
      }
      s_sub[tid] = acc;
    }
    __syncthreads();
    if (tid < G) {
      f32x4 v = s_sub[tid];
      for (int p = 1; p < L; ++p) v += s_sub[p * G + tid];
      *reinterpret_cast<f32x4*>(&s_row[4 * tid]) = v;
    }
  }
  __syncthreads();

  // mean square of the latent part
  float ss = 0.f;
  for (int n = tid; n < a.d_c; n += kFinishThreads) ss = fmaf(s_row[n], s_row[n], ss);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if (tid % 64 == 0) s_red[tid / 64] = ss;
  __syncthreads();
  float total = 0.f;
#pragma unroll
  for (int q = 0; q < kFinishThreads / 64; ++q) total += s_red[q];
  const float inv = 1.0f / sqrtf(total / static_cast<float>(a.d_c) + a.eps);

  if (slot < 0) return;  // uniform per workgroup
  T* dst = static_cast<T*>(a.cache_out) + slot * N;

#pragma unroll
  for (int q = 0; q <= kMaxRow / kFinishThreads; ++q) {
    const int n = tid + q * kFinishThreads;
    if (n < a.d_c) store_out(dst, n, gain[q] * (s_row[n] * inv));
  }
  // RoPE on the pairs (x[2k], x[2k+1]): the angle pos * inv_freq[k] formed and
  // reduced modulo 2π in fp64 (inv_freq = base^(-2k/d_r) from the host, in fp64),
  // sine and cosine of the reduced angle in fp32, the rotation in fp32
  for (int k = tid; k < a.d_r / 2; k += kFinishThreads) {
    const double theta = static_cast<double>(pos) * a.inv_freq[k];
    const double red = theta - 6.283185307179586 * rint(theta * 0.15915494309189535);
    float sn, cs;
    sincosf(static_cast<float>(red), &sn, &cs);
    const float x0 = s_row[a.d_c + 2 * k], x1 = s_row[a.d_c + 2 * k + 1];
    store_out(dst, a.d_c + 2 * k, x0 * cs - x1 * sn);
    store_out(dst, a.d_c + 2 * k + 1, x0 * sn + x1 * cs);
  }
}

hipError_t launch_latent_finish(int dtype, const ProjArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.d_c <= 0 || a.d_r < 0 || a.d_r > 2 * kMaxRopePairs || a.d_c + a.d_r > kMaxRow || a.n_new <= 0)
    return hipErrorInvalidValue;
  // bf16: four columns per thread group, at least one thread per group
  if (dtype != 0 && ((a.d_c + a.d_r) % 4 != 0 || (a.d_c + a.d_r) / 4 > kFinishThreads || a.ksplit <= 0))
    return hipErrorInvalidValue;
  if (dtype == 0)
    latent_finish_kernel<float><<<a.M, kFinishThreads, 0, s>>>(a);
  else
    latent_finish_kernel<uint16_t><<<a.M, kFinishThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
