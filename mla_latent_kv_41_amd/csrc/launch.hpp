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

// One (sequence, token range) pair of the split-K attention. The query
// preparation writes the pairs of each class into a list on the device.
struct WorkItem {
  int32_t b;   // sequence
  int32_t s;   // range s of the sequence's ceil(kv / chunk), its tiles dealt out evenly
  int32_t p;   // partial index: the range's partial rows are (p * n_q + j) * h + head
  int32_t kv;  // the sequence's length, clamped to max_kv_len
};

// Split plan built on the device (by the query preparation's first workgroup) from
// kv_lens: a sequence with fewer than precise_below tokens goes to the precise list
// and holds ns_b = ceil(kv_b / chunk_precise) ranges, else to the fast list with
// ceil(kv_b / chunk_fast) ranges (none if kv_b < n_q); its partials take indices
// seq_off[b] .. seq_off[b] + ns_b - 1, compactly. Pairs past `cap` are dropped
// (only possible when the host lengths the plan was sized from disagree with kv_lens).
struct PlanArgs {
  const int32_t* kv_lens;
  int32_t batch, n_q, max_kv_len, chunk_fast, chunk_precise, precise_below, cap;
  int32_t* counts;    // [0] pairs in the fast list, [1] in the precise list
  int32_t* seq_off;   // [batch + 1]
  WorkItem* fast;     // [cap + kListPad]: the pairs, then entries with b = -1
  WorkItem* precise;  // [cap + kListPad]
};
constexpr int kListPad = 8;  // list entries past cap (grids are padded to 8 workgroups)

struct QPrepArgs {
  const uint16_t* q_nope;   // [M][h][128]
  const uint16_t* q_rope;   // [M][h][64] or nullptr
  const uint16_t* w_uk_pk;  // packed W_UK
  const int32_t* kv_lens;
  uint16_t* q_cat;          // block order (see qprep_kernel): bf16 of the scaled query
  uint16_t* q_lo;           // same order: bf16 of what q_cat's rounding left, or nullptr
  const float* q_abs;       // latent mode: the absorbed query [M][h][512] fp32 given (no W_UK product), or nullptr
  int32_t M, n_q, h, d_r, max_kv_len;
  float qscale;             // scale * log2(e)
  double inv_freq[32];      // rope_base^(-2k/d_r), computed on the host in fp64
  PlanArgs plan;
};
hipError_t launch_qprep_bf16(const QPrepArgs& a, hipStream_t s);

// Attention kernel forms
enum DecodeForm : int32_t {
  kForm128 = 0,       // 128 query rows per workgroup, one bf16 query (fast)
  kFormRoles = 1,     // role-split 64-row workgroups, one bf16 query (fast)
  kFormPrecise = 2,   // role-split 64-row workgroups, query and probabilities as hi + lo bf16
  kFormPingPong = 3,  // eight-wave 64-row workgroups (a score and a value wave per SIMD), one bf16 query (fast)
};

struct DecodeArgs {
  CacheRef cache;
  const uint16_t* q_cat;   // block order (written by qprep_kernel)
  const uint16_t* q_lo;    // kFormPrecise: the low halves, same order
  const WorkItem* list;    // the pairs this launch takes, then entries with b = -1
  float* o_part;           // [pairs][n_q][h][512] fp32, O relative to the row's reference m
  float* ml_part;          // [pairs][n_q][h][2] (m, l), base-2 units
  int32_t n_q, h, d_r, chunk;
  int32_t form;            // DecodeForm
  int32_t units;           // workgroups launched: pairs the list may hold x head groups
  uint64_t* stamps;        // instrumented builds: the phase stamp buffer (set by the launcher)
};
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);
// One grid for a call's fast launch (fast: kForm128, units a multiple of 8, q_lo
// set) and its precise launch, whose arguments are fast's but for the
// list, range length and unit count given: the fast units first.
hipError_t launch_decode_mixed_bf16(const DecodeArgs& fast, const WorkItem* prec_list, int prec_chunk,
                                    int prec_units, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);

struct CombineArgs {
  const float* o_part;      // [pairs][n_q][h][512]
  const float* ml_part;     // [pairs][n_q][h][2] (m, l)
  const int32_t* seq_off;   // [batch + 1] first partial index of each sequence
  const uint16_t* w_uv_pk;  // packed W_UV
  const float* gate;        // [16][M][h*128] pre-activation gate logit splits, or nullptr
  float* out;               // [M][h*128]: one plain store per element
  float* o_lat;             // latent mode: [M][h][512] merged latent output (no W_UV), or nullptr
  float* lse;               // [M][h] or nullptr
  int32_t batch, n_q, h;
  int32_t rows_per_wg;      // query rows per workgroup: 32, 16, 8, 4, 2 or 1
};
hipError_t launch_combine_bf16(const CombineArgs& a, hipStream_t s);

// g[ks][m][n] = Σ_{k in split ks} x[m][k] w[k][n]; K a multiple of 16 ksplit, N of 32
// K splits of the gate logits g = x · W_G: the split-K product writes
// [kGateSplit][M][h * 128] fp32 sums, which the combine kernels add in order
constexpr int kGateSplit = 4;

struct GemmArgs {
  const uint16_t* x;  // [M][K]
  const uint16_t* w;  // [K][N]
  float* g;           // [ksplit][M][N]
  int32_t M, K, N, ksplit;
};
hipError_t launch_splitk_gemm_bf16(const GemmArgs& a, hipStream_t s);

// ---------------------------------------------------------------- non-absorbed form
struct ExpandArgs {
  CacheRef cache;             // the latent cache (bf16)
  const int32_t* kv_lens;     // [batch]
  const uint16_t* w_uk;       // [d_c][h*128] formula layout
  const uint16_t* w_uv;       // [d_c][h*128]
  const uint16_t* packed;     // workspace: both matrices in B-fragment order (written first)
  float* k_out;               // [batch][max_kv_len][h][128]
  float* v_out;               // [batch][max_kv_len][h][128]
  int32_t batch, max_kv_len, h, d_c, d_r;
};
hipError_t launch_expand(const ExpandArgs& a, hipStream_t s);

struct ExplicitArgs {
  CacheRef cache;             // the latent cache, for the rotated keys k_R
  const int32_t* kv_lens;
  const float* k;             // [batch][max_kv_len][h][128]
  const float* v;             // [batch][max_kv_len][h][128]
  const uint16_t* q_nope;     // [batch][n_q][h][128]
  const uint16_t* q_rope;     // [batch][n_q][h][d_r] or nullptr
  const float* gate;          // [16][M][h*128] gate logit splits, or nullptr
  float* part;                // [batch][n_splits][n_q][h][130] (O, m, l) per token range
  float* out;                 // [M][h*128]
  float* lse;                 // [M][h] or nullptr
  int32_t batch, n_q, h, d_r, max_kv_len, n_splits, chunk;
  float qscale;               // scale * log2(e)
  double inv_freq[32];        // rope_base^(-2k/d_r)
};
hipError_t launch_explicit_decode(const ExplicitArgs& a, hipEvent_t ev0, hipEvent_t ev1, hipStream_t s);

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
