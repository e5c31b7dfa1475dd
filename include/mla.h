/*
 * mla.h — C ABI of the MI355X (gfx950) absorbed Multi-head Latent Attention
 * decode library (libmla.so).
 *
 * The method (pages: "MLA多头潜在注意力机制：低秩压缩与矩阵吸收实现高效推理"
 * §2.2, §3.1, §3.2, §5.1, §5.2; the interview guide §6.2; the linear-algebra
 * page, "潜在向量的压缩与上投影" and "解耦 RoPE"; the Gated-MLA page §2.6, §3.3):
 *
 *   Each cached token stores one row [ c_KV (d_c) ‖ RoPE(k_R, pos) (d_rope) ].
 *   W_UK is absorbed into the query: q_abs = q_nope · W_UK_iᵀ (length d_c), so the
 *   score of head i against token t is scale · (q_abs · c_t + RoPE(q_R) · k_R,t).
 *   The softmax-weighted sum stays in latent space, o_lat = Σ_t p_t c_t, and W_UV
 *   is applied once per head afterwards: out_i = o_lat · W_UV_i. With a gate,
 *   out ⊙= sigmoid(x · W_G) channel-wise over the concatenated heads.
 *
 * Conventions shared by every entry point
 *   - Pointers named as device pointers must be device memory of the current
 *     HIP device; "host" pointers are ordinary host memory.
 *   - All tensors are dense row-major in the order their shape is written.
 *   - bf16 means IEEE bfloat16; every conversion to bf16 rounds to nearest even.
 *   - Weight layouts follow the formula orientation: W_UK is [d_c][h*d_qk_nope]
 *     and head i owns columns i*d_qk_nope .. (i+1)*d_qk_nope-1; W_UV likewise.
 *   - RoPE rotates the pairs (x[2k], x[2k+1]) by pos * rope_base^(-2k/d_rope).
 *   - Calls are asynchronous and ordered on `stream` (0 = the null stream). The
 *     library never allocates, frees or synchronises, and keeps no state besides
 *     a cached device-property query; it is safe to call from several threads.
 *     Buffers passed in must stay alive until the stream has run the work.
 *   - Errors: arguments are checked on the host before any launch, and a failed
 *     check returns a status without touching the device. A launch failure
 *     returns MLA_E_HIP. Device-side ranges that the host cannot see (kv_lens
 *     contents, block-table entries) are bounds-checked in the kernels: an
 *     out-of-range entry is skipped instead of being read or written, and the
 *     result for that sequence is then undefined.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mla_status;
#define MLA_OK 0
#define MLA_E_NULL 1        /* a required pointer is NULL */
#define MLA_E_SHAPE 2       /* sizes inconsistent with each other */
#define MLA_E_DTYPE 3       /* unknown dtype code */
#define MLA_E_UNSUPPORTED 4 /* valid shape that the library has no kernel for */
#define MLA_E_WORKSPACE 5   /* workspace too small */
#define MLA_E_HIP 6         /* a HIP call or launch failed */

#define MLA_F32 0  /* cache, weights and queries in fp32 (fp32 arithmetic throughout) */
#define MLA_BF16 1 /* cache, weights and queries in bf16 (bf16 MFMA, fp32 accumulation) */

/* Attention dimensions (per layer). */
typedef struct {
  int32_t n_heads;   /* h */
  int32_t d_c;       /* latent width of the cached c_KV */
  int32_t d_rope;    /* decoupled RoPE key width (0: no positional key) */
  int32_t d_qk_nope; /* per-head query/key width without position */
  int32_t d_v;       /* per-head value width */
  float scale;       /* score scale; 0 selects 1/sqrt(d_qk_nope + d_rope) */
  float rope_base;   /* 0 selects 10000 */
  int32_t dtype;     /* MLA_F32 or MLA_BF16 */
} mla_dims;

/*
 * Supported shapes. MLA_F32: any h <= 1024, d_c <= 1024, d_rope <= 256 and even,
 * d_qk_nope <= 256, d_v <= 256 (a plain fp32 path for small layers).
 * MLA_BF16: d_c = 512, d_rope in {0, 64}, d_qk_nope = 128, d_v = 128, n_heads a
 * multiple of 32 with n_heads * n_q a multiple of 64 (the DeepSeek-V2/V3 attention
 * shape and its position-free gated variant); with a gate, d_model a multiple of
 * 64. Paged caches need block_size a multiple of 32. Other shapes return
 * MLA_E_UNSUPPORTED (or MLA_E_SHAPE).
 *
 * Precision of the bf16 decode: the cache, weights and queries are bf16; products
 * accumulate in fp32; the split partials and their merge are fp32; the absorbed,
 * scaled query and the softmax probabilities enter the matrix cores as bf16 for
 * sequences of 4096 tokens or more, and as hi + lo bf16 pairs (about 16 significant
 * bits) for shorter sequences, where single bf16 roundings do not average out.
 */
/*
 * One-time weight absorption / packing (tutorial §3.2: "preprocess the absorbed
 * weights once at load time"; the einsums `bhsd,hcd->bhsc` and `bhsc,hdc->bhsd`
 * of §5.1).
 *   w_uk   device [d_c][h*d_qk_nope], dims->dtype
 *   w_uv   device [d_c][h*d_v],       dims->dtype
 *   packed device buffer of *packed_bytes bytes, owned by the caller; its layout
 *          is private to the library (per-head blocks in matrix-core fragment
 *          order) and is what mla_decode / mla_decode_paged read.
 * With packed == NULL the call only writes the needed size to *packed_bytes and
 * returns MLA_OK (no device access). Otherwise *packed_bytes must hold at least
 * that size (MLA_E_WORKSPACE if not).
 */
mla_status mla_absorb_weights(const mla_dims* dims, const void* w_uk, const void* w_uv,
                              void* packed, size_t* packed_bytes, hipStream_t stream);

/* Where the latent cache lives. Row width is d_c + d_rope elements of dims->dtype. */
typedef struct {
  const int32_t* block_table; /* device [batch][max_blocks] physical block ids; NULL = contiguous */
  int32_t t_max;              /* contiguous: token slots per sequence, cache is [batch][t_max][row] */
  int32_t block_size;         /* paged: tokens per block, pool is [n_blocks][block_size][row] */
  int32_t max_blocks;         /* paged: entries per block-table row */
  int32_t n_blocks;           /* paged: blocks in the pool (ids must lie in [0, n_blocks)) */
} mla_cache_layout;

/*
 * Latent append (tutorial §5.2: append each new c_kv at its position instead of
 * concatenating; interview guide §8.2; linear-algebra page "解耦 RoPE": the row
 * is c_KV followed by the RoPE-rotated k_R).
 *   cache  device buffer laid out as `layout` describes
 *   c_kv   device [batch][n_new][d_c]    (already normalised by the caller)
 *   k_r    device [batch][n_new][d_rope] unrotated; NULL iff d_rope == 0
 *   pos0   device [batch]: slot of the first new token of each sequence; token j
 *          goes to position pos0[b] + j and its k_R is rotated by that position
 * The call writes only those n_new rows per sequence. Rows whose position falls
 * outside the layout (or whose block id is out of range) are skipped. The caller
 * owns the lengths and advances them once per step for all layers.
 */
mla_status mla_append_latent(const mla_dims* dims, void* cache, const mla_cache_layout* layout,
                             int32_t batch, int32_t n_new, const void* c_kv, const void* k_r,
                             const int32_t* pos0, hipStream_t stream);

/* Per-call decode arguments. */
typedef struct {
  int32_t batch;               /* B */
  int32_t n_q;                 /* new (query) tokens per sequence, >= 1 */
  const int32_t* kv_lens;      /* device [B]: visible tokens per sequence, the n_q new ones
                                  included (they must already be appended); query j of
                                  sequence b is at position kv_lens[b] - n_q + j and
                                  attends to positions 0 .. kv_lens[b] - n_q + j */
  const int32_t* kv_lens_host; /* optional host copy of kv_lens: validated, and used to plan
                                  the split of long sequences; NULL = plan from max_kv_len */
  int32_t max_kv_len;          /* bound on every kv_lens[b] (required, >= n_q) */
  const void* q_nope;          /* device [B][n_q][h][d_qk_nope], dims->dtype */
  const void* q_rope;          /* device [B][n_q][h][d_rope] unrotated, NULL iff d_rope == 0 */
  const void* packed_w;        /* device, from mla_absorb_weights */
  const void* gate_x;          /* device [B][n_q][d_model] or NULL (no gate) */
  const void* w_gate;          /* device [d_model][h*d_v] or NULL; both or neither */
  int32_t d_model;             /* gate input width */
  float* out;                  /* device [B][n_q][h*d_v] fp32, heads concatenated */
  float* lse;                  /* device [B][n_q][h] fp32 log-sum-exp of the scores, or NULL */
  void* workspace;             /* device scratch, or NULL to query its size */
  size_t* workspace_bytes;     /* in: size of workspace; out (when workspace == NULL): needed */
  int32_t num_splits;          /* 0: the planner chooses; > 0 forces token splits per sequence */
  hipEvent_t ev_attn_begin;    /* optional timing events (both or neither, else MLA_E_NULL): */
  hipEvent_t ev_attn_end;      /* bf16 path: stamped by the split-K attention dispatch itself
                                  (start and end of that kernel); fp32 path: recorded on
                                  `stream` before and after its attention kernels */
} mla_decode_args;

/*
 * Absorbed decode over a contiguous cache [batch][t_max][d_c + d_rope] (tutorial
 * §3.1 and §5.1; linear-algebra page "解耦 RoPE"; Gated-MLA page §2.6 for the
 * gate). Writes args->out (and args->lse). Needs a workspace (query its size
 * with workspace == NULL); MLA_E_WORKSPACE if *workspace_bytes is too small.
 */
mla_status mla_decode(const mla_dims* dims, const void* cache, int32_t t_max,
                      const mla_decode_args* args, hipStream_t stream);

/* The same over a paged pool [n_blocks][block_size][d_c + d_rope] addressed through
 * block_table (device [batch][max_blocks]); block_size must be a multiple of 32. */
mla_status mla_decode_paged(const mla_dims* dims, const void* pool, const int32_t* block_table,
                            int32_t block_size, int32_t max_blocks, int32_t n_blocks,
                            const mla_decode_args* args, hipStream_t stream);

/*
 * Decode with the absorption folded into the weights (tutorial §2.2 and §5.1: W_UK
 * can be absorbed into the query's up-projection W_UQ, and W_UV into the output
 * projection W_O, so neither is applied at run time). The caller forms the absorbed
 * query itself, q_abs = c_Q · (W_UQ_i · W_UK_iᵀ), and applies the folded output
 * weights (W_UV_i · W_O_i) to the result; this call runs the attention between:
 *   args->q_nope  device [B][n_q][h][d_c] fp32: the absorbed query q_abs (not q_nope),
 *                 rounded once by the call, with the score scale, to the matrix cores'
 *                 bf16 (a hi + lo pair for the sequences the precise form takes)
 *   args->q_rope  device [B][n_q][h][d_rope] unrotated, as for mla_decode
 *   args->out     device [B][n_q][h][d_c] fp32: the merged latent output
 *                 o_lat = Σ_t p_t c_t of each (query, head), not yet up-projected
 * The scores are scale · (q_abs · c_t + RoPE(q_R) · k_R,t) with the same attention
 * kernels and plan as mla_decode; args->packed_w is not used; args->lse as there.
 * `layout` selects the cache form (contiguous when block_table is NULL). The gate
 * acts on the heads' outputs, which this form never forms: a gated call returns
 * MLA_E_UNSUPPORTED. MLA_BF16 only.
 */
mla_status mla_decode_latent(const mla_dims* dims, const void* cache, const mla_cache_layout* layout,
                             const mla_decode_args* args, hipStream_t stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and kernels as mla_decode / mla_decode_paged, with the
 * workspace taken from a 64 MiB array that the library holds on each GPU it runs
 * on (from its first use on that GPU until the process ends) instead of from the
 * caller. `layout` selects the cache form as for mla_append_latent: contiguous
 * [batch][t_max][row] when layout->block_table is NULL, else the paged pool with
 * block_size a multiple of 32. args->workspace and args->workspace_bytes are
 * ignored. MLA_E_WORKSPACE if the call would need more than 64 MiB of workspace
 * (the DeepSeek-shaped step, 32 sequences of 4097 tokens, needs about 43 MB).
 * The call allocates and frees nothing and clears nothing: every call rewrites the
 * parts of the array it reads. All calls on one GPU share its array, so calls that
 * overlap on one GPU (on different streams, or from different threads without
 * ordering) race and their results are undefined; calls ordered on one stream are
 * safe.
 */
mla_status mla_decode_noalloc(const mla_dims* dims, const void* cache, const mla_cache_layout* layout,
                              const mla_decode_args* args, hipStream_t stream);

/*
 * The non-absorbed form, for comparison with the absorbed decode (tutorial §3.2:
 * the training-time forward up-projects the cached latent into per-head keys and
 * values, k = c_KV · W_UK and v = c_KV · W_UV, and runs standard attention; §3.3
 * compares the two forms at decode). MLA_BF16 only, d_qk_nope = d_v = 128.
 *
 * mla_expand_kv writes, for every cached token t < kv_lens[b] of every sequence,
 *   k_out[b][t][i][e] = Σ_c c_t[c] · W_UK[c][i*128 + e]
 *   v_out[b][t][i][e] = Σ_c c_t[c] · W_UV[c][i*128 + e]
 * in fp32 (bf16 products on the matrix cores, fp32 accumulation), with k_out and
 * v_out device [batch][max_kv_len][h][128] fp32 (rows past kv_lens[b] untouched).
 *   cache, layout  the latent cache, as for mla_append_latent
 *   kv_lens        device [batch]; values above max_kv_len are clamped to it
 *   w_uk, w_uv     device [d_c][h*128] bf16, the formula layout (not packed)
 *   workspace      device scratch for the weights in matrix-core order, or NULL to
 *                  query its size (2 * d_c * h * 128 * 2 bytes, rounded up)
 */
mla_status mla_expand_kv(const mla_dims* dims, const void* cache, const mla_cache_layout* layout, int32_t batch,
                         const int32_t* kv_lens, int32_t max_kv_len, const void* w_uk, const void* w_uv,
                         float* k_out, float* v_out, void* workspace, size_t* workspace_bytes,
                         hipStream_t stream);

/*
 * Standard attention over explicit keys and values (the non-absorbed decode): for
 * query j of sequence b and head i, the scores
 *   scale · ( q_nope · k[b][t][i] + RoPE(q_R, p_j) · k_R,t ),  t <= p_j = kv_len - n_q + j,
 * with k_R the rotated key stored in the latent cache rows (one per token, shared by
 * the heads), a max-subtracted softmax and out = Σ_t p_t v[b][t][i]; the gate as in
 * mla_decode. fp32 arithmetic throughout. k, v are [batch][args->max_kv_len][h][128]
 * fp32, as mla_expand_kv writes them for the same max_kv_len. args as for mla_decode
 * (packed_w is not used; n_q <= 4); the workspace holds the token ranges' partial
 * results (size query with workspace == NULL). Timing events, when given, are
 * recorded on `stream` around the attention kernel.
 */
mla_status mla_decode_explicit(const mla_dims* dims, const float* k, const float* v, const void* cache,
                               const mla_cache_layout* layout, const mla_decode_args* args, hipStream_t stream);

/*
 * Fused latent append from the hidden state: the cache row of each new token,
 *   [ gain ⊙ c / sqrt(mean(c²) + eps)  ‖  RoPE(h · W_KR, pos) ],  c = h · W_DKV,
 * computed and stored in one call (tutorial §2.2: c_KV = h · W_DKV with W_DKV of
 * d_model × d_c; §6.3: an RMSNorm over the latent right after the
 * down-projection; interview guide §6.2 `MLA` module: k_R from its own
 * d_model → d_rope projection of the same input; linear-algebra page "解耦 RoPE":
 * k_R is cached rotated). It replaces the caller's projections + normalisation +
 * mla_append_latent.
 *
 * mla_pack_down_weights packs the two projections once into one matrix:
 *   w_dkv  device [d_model][d_c],    dims->dtype
 *   w_kr   device [d_model][d_rope], dims->dtype; NULL iff d_rope == 0
 *   packed device buffer of *packed_bytes bytes owned by the caller, laid out as
 *          [d_model][d_c + d_rope] (W_DKV's columns, then W_KR's).
 * With packed == NULL it only writes the needed size (no device access).
 */
mla_status mla_pack_down_weights(const mla_dims* dims, int32_t d_model, const void* w_dkv,
                                 const void* w_kr, void* packed, size_t* packed_bytes,
                                 hipStream_t stream);

typedef struct {
  int32_t batch;              /* sequences */
  int32_t n_new;              /* new tokens per sequence */
  int32_t d_model;            /* hidden width; bf16: a multiple of 16 */
  const void* hidden;         /* device [batch][n_new][d_model], dims->dtype */
  const void* packed_down;    /* device, from mla_pack_down_weights with the same d_model */
  const float* norm_gain;     /* device [d_c] fp32 RMSNorm gain, or NULL for all ones */
  float norm_eps;             /* RMSNorm epsilon, >= 0 (added to the mean square) */
  const int32_t* pos0;        /* device [batch]: position (and slot) of each sequence's first
                                 new token; token j goes to pos0[b] + j, as in
                                 mla_append_latent */
  void* workspace;            /* device scratch, or NULL to query its size */
  size_t* workspace_bytes;    /* in: size of workspace; out (when workspace == NULL): needed */
  int32_t k_splits;           /* bf16: 0 lets the library choose; > 0 forces the number of
                                 d_model splits of the product (d_model must be a multiple
                                 of 16 * k_splits) */
} mla_project_args;

/*
 * Writes the n_new rows per sequence into `cache` (laid out as `layout` says),
 * exactly where mla_append_latent would. bf16: the products run on the matrix
 * cores with fp32 accumulation, split over d_model and summed in a fixed order;
 * normalisation in fp32; RoPE angles formed and reduced modulo 2π in fp64, their
 * sine, cosine and the rotation in fp32; one rounding to bf16 per element. fp32:
 * the same in fp32 arithmetic, without the matrix cores. Rows whose position falls outside the layout
 * (or whose block id is out of range) are skipped. MLA_E_WORKSPACE if
 * *workspace_bytes is too small; MLA_E_UNSUPPORTED for a bf16 d_model that is not
 * a multiple of 16 (or of 16 * k_splits).
 */
mla_status mla_project_append(const mla_dims* dims, void* cache, const mla_cache_layout* layout,
                              const mla_project_args* args, hipStream_t stream);

/* Static description of a status code. */
const char* mla_status_string(mla_status s);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
