// fp32 absorbed-MLA decode for small layers: fp32 FMA arithmetic throughout.
//
// Same method as the bf16 matrix-core path (MLA tutorial page §3.1 and the
// einsums of §5.1; decoupled RoPE key of the interview guide §6.2): the query is
// absorbed, q_abs = q_nope · W_UK_iᵀ, scores are taken against the cached
// [c_KV ‖ k_R] rows, the softmax-weighted sum stays in latent space and W_UV is
// applied once per head. Three kernels: query preparation, attention (scores,
// max-subtracted softmax, latent sum), and the up-projection with the optional
// sigmoid gate (Gated-MLA page §2.6).
#include "common.hpp"
#include "launch.hpp"

namespace mla {

__device__ __forceinline__ const float* f32_row(const CacheRef& c, int b, int64_t t, int row) {
  const float* base = static_cast<const float*>(c.data);
  if (c.block_table == nullptr) return base + (static_cast<int64_t>(b) * c.t_max + t) * row;
  const int64_t blk = t / c.block_size;
  int32_t id = blk < c.max_blocks ? c.block_table[static_cast<int64_t>(b) * c.max_blocks + blk] : -1;
  if (id < 0 || id >= c.n_blocks) return nullptr;
  return base + (static_cast<int64_t>(id) * c.block_size + t % c.block_size) * row;
}

// q_cat[m][i] = qscale * [ q_nope · W_UK_iᵀ ‖ RoPE(q_R, pos) ];  grid M*h.
__global__ void f32_qprep(F32Args a) {
  const int m = blockIdx.x / a.h, i = blockIdx.x % a.h;
  const int b = m / a.n_q, j = m % a.n_q;
  const int row = a.d_c + a.d_r;
  const float* qn = a.q_nope + (static_cast<int64_t>(m) * a.h + i) * a.d_n;
  float* dst = a.q_cat + (static_cast<int64_t>(m) * a.h + i) * row;
  for (int c = threadIdx.x; c < a.d_c; c += blockDim.x) {
    const float* w = a.w_uk + static_cast<int64_t>(c) * a.h * a.d_n + static_cast<int64_t>(i) * a.d_n;
    float acc = 0.f;
    for (int e = 0; e < a.d_n; ++e) acc = fmaf(qn[e], w[e], acc);
    dst[c] = acc * a.qscale;
  }
  const int kv = min(a.kv_lens[b], a.max_kv_len);
  const int64_t pos = static_cast<int64_t>(kv) - a.n_q + j;
  const float* qr = a.q_rope + (static_cast<int64_t>(m) * a.h + i) * a.d_r;
  for (int k = threadIdx.x; k < a.d_r / 2; k += blockDim.x) {
    double sn, cs;
    sincos(static_cast<double>(pos) * pow(a.rope_base, -2.0 * k / a.d_r), &sn, &cs);
    const double x0 = qr[2 * k], x1 = qr[2 * k + 1];
    dst[a.d_c + 2 * k] = static_cast<float>((x0 * cs - x1 * sn) * a.qscale);
    dst[a.d_c + 2 * k + 1] = static_cast<float>((x0 * sn + x1 * cs) * a.qscale);
  }
}

__device__ float block_reduce(float v, bool is_max, float* red) {
  for (int o = 32; o > 0; o >>= 1) {
    const float w = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, w) : v + w;
  }
  const int wv = threadIdx.x / 64, nw = blockDim.x / 64;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wv] = v;
  __syncthreads();
  v = red[0];
  for (int k = 1; k < nw; ++k) v = is_max ? fmaxf(v, red[k]) : v + red[k];
  return v;
}

// Scores (log2 units: q_cat carries scale*log2 e), softmax, latent sum; grid M*h.
__global__ void f32_attn(F32Args a) {
  __shared__ float red[16];
  const int m = blockIdx.x / a.h, i = blockIdx.x % a.h;
  const int b = m / a.n_q, j = m % a.n_q;
  const int row = a.d_c + a.d_r;
  const int kv = min(a.kv_lens[b], a.max_kv_len);
  const int n_vis = kv - a.n_q + j + 1;  // causal: query j sees 0 .. kv - n_q + j
  const float* q = a.q_cat + (static_cast<int64_t>(m) * a.h + i) * row;
  float* sc = a.scores + (static_cast<int64_t>(m) * a.h + i) * a.max_kv_len;
  float mx = -INFINITY;
  for (int t = threadIdx.x; t < n_vis; t += blockDim.x) {
    const float* r = f32_row(a.cache, b, t, row);
    float s = -INFINITY;
    if (r) {
      s = 0.f;
      for (int c = 0; c < row; ++c) s = fmaf(q[c], r[c], s);
    }
    sc[t] = s;
    mx = fmaxf(mx, s);
  }
  mx = block_reduce(mx, true, red);
  const float mref = mx == -INFINITY ? 0.f : mx;
  float sum = 0.f;
  for (int t = threadIdx.x; t < n_vis; t += blockDim.x) {
    const float p = exp2f(sc[t] - mref);
    sc[t] = p;
    sum += p;
  }
  sum = block_reduce(sum, false, red);
  __syncthreads();
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  float* o = a.o_lat + (static_cast<int64_t>(m) * a.h + i) * a.d_c;
  for (int c = threadIdx.x; c < a.d_c; c += blockDim.x) {
    float acc = 0.f;
    for (int t = 0; t < n_vis; ++t) {
      const float* r = f32_row(a.cache, b, t, row);
      if (r) acc = fmaf(sc[t], r[c], acc);
    }
    o[c] = acc * inv;
  }
  if (a.lse && threadIdx.x == 0) a.lse[static_cast<int64_t>(m) * a.h + i] = (mref + log2f(sum)) * kLn2;
}

// out[m][i*d_v + d] = o_lat · W_UV_i (times sigmoid(x · W_G) when gated); grid M*h.
__global__ void f32_up(F32Args a) {
  const int m = blockIdx.x / a.h, i = blockIdx.x % a.h;
  const float* o = a.o_lat + (static_cast<int64_t>(m) * a.h + i) * a.d_c;
  const int64_t width = static_cast<int64_t>(a.h) * a.d_v;
  for (int d = threadIdx.x; d < a.d_v; d += blockDim.x) {
    const int64_t col = static_cast<int64_t>(i) * a.d_v + d;
    float acc = 0.f;
    for (int c = 0; c < a.d_c; ++c) acc = fmaf(o[c], a.w_uv[c * width + col], acc);
    if (a.gate_x) {
      float g = 0.f;
      for (int k = 0; k < a.d_model; ++k)
        g = fmaf(a.gate_x[static_cast<int64_t>(m) * a.d_model + k], a.w_gate[k * width + col], g);
      acc *= 1.f / (1.f + expf(-g));
    }
    a.out[m * width + col] = acc;
  }
}

hipError_t launch_decode_f32(const F32Args& a, hipEvent_t ev0, hipEvent_t ev1, hipStream_t s) {
  const int M = a.batch * a.n_q;
  const dim3 grid(M * a.h);
  f32_qprep<<<grid, 256, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev0 && hipEventRecord(ev0, s) != hipSuccess) return hipErrorUnknown;
  f32_attn<<<grid, 256, 0, s>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev1 && hipEventRecord(ev1, s) != hipSuccess) return hipErrorUnknown;
  f32_up<<<grid, 128, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
