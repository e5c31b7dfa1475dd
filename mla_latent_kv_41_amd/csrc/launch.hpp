// Host-side launchers for the kernels of libmla (one per translation unit).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Cache addressing shared by the kernels: contiguous when block_table == nullptr.
struct CacheRef {
  const void* data;
  const int32_t* block_table;
  int32_t t_max;       // contiguous: slots per sequence
  int32_t block_size;  // paged
  int32_t max_blocks;  // paged: table row length
  int32_t n_blocks;    // paged: pool size
};

// ---------------------------------------------------------------- bf16 (MFMA) path
hipError_t launch_pack_bf16(const uint16_t* w_uk, const uint16_t* w_uv, uint16_t* packed, int h,
                            hipStream_t s);
hipError_t launch_append(int dtype, void* cache, const CacheRef& c, int batch, int n_new, int d_c,
                         int d_r, const void* c_kv, const void* k_r, const int32_t* pos0,
                         double rope_base, hipStream_t s);

struct QPrepArgs {
  const uint16_t* q_nope;   // [M][h][128]
  const uint16_t* q_rope;   // [M][h][64] or nullptr
  const uint16_t* w_uk_pk;  // packed W_UK
  const int32_t* kv_lens;
  uint16_t* q_cat;          // fragment order of the attention kernel (see qprep_kernel)
  int32_t M, n_q, h, d_r, max_kv_len;
  int32_t rows_per_wg;      // query rows per attention workgroup (32 per wave)
  float* out;               // [M][h*128] output, zeroed for the combine's atomic adds
  float qscale;             // scale * log2(e)
  double inv_freq[32];      // rope_base^(-2k/d_r), computed on the host in fp64
};
hipError_t launch_qprep_bf16(const QPrepArgs& a, hipStream_t s);

struct DecodeArgs {
  CacheRef cache;
  const int32_t* kv_lens;
  const uint16_t* q_cat;  // fragment order (written by qprep_kernel)
  uint16_t* o_part;       // [B][S][n_q][h][512] bf16, normalised O / l
  float* ml_part;         // [B][S][n_q][h][2]
  int32_t batch, n_q, h, d_r, n_splits, chunk, max_kv_len;
  int32_t role_split;   // 1: role-split 64-row workgroups (h n_q % 128 == 64); 0: 128-row workgroups
};
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);

struct CombineArgs {
  const uint16_t* o_part;  // [B][S][n_q][h][512] bf16
  const float* ml_part;    // [B][S][n_q][h][2] (m, l)
  const int32_t* kv_lens;
  const uint16_t* w_uv_pk;  // packed W_UV
  const float* gate;        // [M][h*128] pre-activation gate logits or nullptr
  float* out;               // [M][h*128], zeroed beforehand: halves are added atomically
  float* lse;               // [M][h] or nullptr
  int32_t batch, n_q, h, n_splits, chunk, max_kv_len;
  int32_t rows_per_wg;       // query rows per workgroup, 1..32
  int32_t splits_per_batch;  // half partial rows staged per row and batch (rows * splits <= slots)
  int32_t slots;             // staged half rows per batch: 256, or 128 (two workgroups per CU)
  int32_t lengths_first;     // 1: wait for the sequence lengths before staging, and skip the
                             // partial rows of splits past each row's last one (ragged batches)
};
hipError_t launch_combine_bf16(const CombineArgs& a, hipStream_t s);

// g[ks][m][n] = Σ_{k in split ks} x[m][k] w[k][n]; K a multiple of 16 ksplit, N of 32
struct GemmArgs {
  const uint16_t* x;  // [M][K]
  const uint16_t* w;  // [K][N]
  float* g;           // [ksplit][M][N]
  int32_t M, K, N, ksplit;
};
hipError_t launch_splitk_gemm_bf16(const GemmArgs& a, hipStream_t s);

// ---------------------------------------------------------------- fused append
// Cache row [gain ⊙ RMSNorm(h · W_DKV) ‖ RoPE(h · W_KR, pos)] of each new token.
constexpr int kMaxRopePairs = 128;  // d_r <= 256
hipError_t launch_pack_down(int dtype, const void* w_dkv, const void* w_kr, void* packed, int d_model, int d_c,
                            int d_r, hipStream_t s);
struct ProjArgs {
  CacheRef cache;        // addressing of the destination (its data pointer is not written through)
  void* cache_out;       // the cache itself, written
  const int32_t* pos0;   // [batch]: position of each sequence's first new token
  const void* hidden;    // fp32 path: [M][d_model]
  const void* w_down;    // fp32 path: packed [d_model][d_c + d_r]
  const float* part;     // bf16 path: [ksplit][M][d_c + d_r] split partial sums
  const float* gain;     // [d_c] or nullptr (ones)
  int32_t M, n_new, d_model, d_c, d_r, ksplit;
  float eps;
  double inv_freq[kMaxRopePairs];  // rope_base^(-2k/d_r), computed on the host in fp64
};
hipError_t launch_latent_finish(int dtype, const ProjArgs& a, hipStream_t s);

// ---------------------------------------------------------------- fp32 path
struct F32Args {
  CacheRef cache;
  const int32_t* kv_lens;
  const float* q_nope;  // [M][h][d_n]
  const float* q_rope;  // [M][h][d_r] or nullptr
  const float* w_uk;    // [d_c][h*d_n]
  const float* w_uv;    // [d_c][h*d_v]
  const float* gate_x;  // [M][d_model] or nullptr
  const float* w_gate;  // [d_model][h*d_v]
  float* q_cat;         // ws [M][h][d_c + d_r]
  float* scores;        // ws [M][h][max_kv_len]
  float* o_lat;         // ws [M][h][d_c]
  float* out;           // [M][h*d_v]
  float* lse;           // [M][h] or nullptr
  int32_t batch, n_q, h, d_c, d_r, d_n, d_v, d_model, max_kv_len;
  float qscale;
  double rope_base;
};
hipError_t launch_decode_f32(const F32Args& a, hipEvent_t ev0, hipEvent_t ev1, hipStream_t s);

}  // namespace mla
