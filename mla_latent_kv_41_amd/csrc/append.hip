// Latent append: write [c_KV ‖ RoPE(k_R, pos)] rows into a contiguous or paged cache.
//
// The cache holds only the latent row per token (MLA tutorial page §5.2 and §6.2:
// append at the position, never concatenate; cache c_kv, never decompressed K/V),
// and the decoupled key is stored already rotated (linear-algebra page, "解耦
// RoPE": the 64-wide k_R "with RoPE" next to the 512-wide c_KV).
#include "common.hpp"
#include "launch.hpp"

namespace mla {

template <typename T>
__device__ __forceinline__ double load_elem(const T* p, int64_t i);
template <>
__device__ __forceinline__ double load_elem<float>(const float* p, int64_t i) {
  return static_cast<double>(p[i]);
}
template <>
__device__ __forceinline__ double load_elem<uint16_t>(const uint16_t* p, int64_t i) {
  return static_cast<double>(bf16_bits_to_f32(p[i]));
}

__device__ __forceinline__ void store_elem(float* p, int64_t i, double v) { p[i] = static_cast<float>(v); }
__device__ __forceinline__ void store_elem(uint16_t* p, int64_t i, double v) { p[i] = f64_to_bf16_bits(v); }

// One workgroup per new token: grid = batch * n_new.
template <typename T>
__global__ void append_kernel(T* __restrict__ cache, CacheRef c, int n_new, int d_c, int d_r,
                              const T* __restrict__ c_kv, const T* __restrict__ k_r,
                              const int32_t* __restrict__ pos0, double rope_base) {
  const int b = blockIdx.x / n_new, j = blockIdx.x % n_new;
  const int64_t pos = static_cast<int64_t>(pos0[b]) + j;
  const int row = d_c + d_r;
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
  T* dst = cache + slot * row;
  const int64_t src = static_cast<int64_t>(b) * n_new + j;
  for (int e = threadIdx.x; e < d_c; e += blockDim.x) dst[e] = c_kv[src * d_c + e];
  // RoPE on the pairs (x[2k], x[2k+1]) with angle pos * base^(-2k/d_r), in fp64,
  // rounded once to the cache type.
  for (int k = threadIdx.x; k < d_r / 2; k += blockDim.x) {
    const double inv_freq = pow(rope_base, -2.0 * k / d_r);
    double sn, cs;
    sincos(static_cast<double>(pos) * inv_freq, &sn, &cs);
    const double x0 = load_elem(k_r, src * d_r + 2 * k), x1 = load_elem(k_r, src * d_r + 2 * k + 1);
    store_elem(dst, d_c + 2 * k, x0 * cs - x1 * sn);
    store_elem(dst, d_c + 2 * k + 1, x0 * sn + x1 * cs);
  }
}

hipError_t launch_append(int dtype, void* cache, const CacheRef& c, int batch, int n_new, int d_c,
                         int d_r, const void* c_kv, const void* k_r, const int32_t* pos0,
                         double rope_base, hipStream_t s) {
  const dim3 grid(batch * n_new), block(128);
  if (dtype == 0)
    append_kernel<float><<<grid, block, 0, s>>>(static_cast<float*>(cache), c, n_new, d_c, d_r,
                                                static_cast<const float*>(c_kv),
                                                static_cast<const float*>(k_r), pos0, rope_base);
  else
    append_kernel<uint16_t><<<grid, block, 0, s>>>(static_cast<uint16_t*>(cache), c, n_new, d_c, d_r,
                                                   static_cast<const uint16_t*>(c_kv),
                                                   static_cast<const uint16_t*>(k_r), pos0, rope_base);
  return hipGetLastError();
}

}  // namespace mla
