// libmla C ABI: argument checking, split planning, workspace layout and launches.
//
// Every check below runs on the host before any HIP call, so a rejected call
// never touches the device.
#include <math.h>
#include <string.h>

#include <algorithm>

#include "mla.h"
#include "launch.hpp"

using namespace mla;

namespace {

constexpr size_t kAlign = 256;
constexpr int kTile = 32;       // tokens per attention tile; split ranges are multiples of it
constexpr int kGateSplit = 16;  // K-splits of the gate logits; must match the combine kernel

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Resolved {
  int h, d_c, d_r, d_n, d_v, dtype;
  float scale;
  double rope_base;
};

mla_status resolve(const mla_dims* d, Resolved* r) {
  if (!d) return MLA_E_NULL;
  if (d->dtype != MLA_F32 && d->dtype != MLA_BF16) return MLA_E_DTYPE;
  if (d->n_heads <= 0 || d->d_c <= 0 || d->d_rope < 0 || d->d_qk_nope <= 0 || d->d_v <= 0) return MLA_E_SHAPE;
  if (d->d_rope % 2) return MLA_E_SHAPE;
  if (!(d->scale >= 0.f) || !(d->rope_base >= 0.f)) return MLA_E_SHAPE;  // also rejects NaN
  r->h = d->n_heads;
  r->d_c = d->d_c;
  r->d_r = d->d_rope;
  r->d_n = d->d_qk_nope;
  r->d_v = d->d_v;
  r->dtype = d->dtype;
  r->scale = d->scale > 0.f ? d->scale : 1.f / sqrtf(static_cast<float>(d->d_qk_nope + d->d_rope));
  r->rope_base = d->rope_base > 0.f ? d->rope_base : 10000.0;
  if (r->dtype == MLA_F32) {
    if (r->h > 1024 || r->d_c > 1024 || r->d_r > 256 || r->d_n > 256 || r->d_v > 256) return MLA_E_UNSUPPORTED;
  } else {
    if (r->d_c != 512 || (r->d_r != 0 && r->d_r != 64) || r->d_n != 128 || r->d_v != 128) return MLA_E_UNSUPPORTED;
  }
  return MLA_OK;
}

size_t elem_bytes(int dtype) { return dtype == MLA_F32 ? 4 : 2; }

// Split plan for the bf16 path.
struct Plan {
  int nw;        // 32-row blocks per attention workgroup (rows = 32 * nw)
  bool roles;    // role-split 64-row form (rows not a multiple of 128)
  int hgroups;   // workgroups per (sequence, split)
  int n_splits;  // token ranges per sequence
  int chunk;     // tokens per range, a multiple of kTile
  int comb_rows;    // combine: query rows per workgroup (<= 32)
  int comb_splits;  // combine: partial half rows staged per row and batch
  int comb_slots;   // combine: staged half rows per batch (256, or 128 with two workgroups per CU)
  bool ragged;      // host lengths given and not all equal
};

Plan plan_bf16(const Resolved& r, const mla_decode_args* a) {
  Plan p;
  const int rows = r.h * a->n_q;
  // 128-row workgroups when the rows come in 128s; else role-split 64-row workgroups
  // (two score waves, two value waves)
  p.roles = rows % 128 != 0;
  p.nw = p.roles ? 2 : 4;
  p.hgroups = rows / (32 * p.nw);
  // one workgroup per CU either way: four tile buffers take most of the LDS
  const int64_t target = 256;
  const int L = a->max_kv_len;
  const int64_t units = static_cast<int64_t>(a->batch) * p.hgroups;
  // one workgroup per slot when every sequence is as long as the longest
  int64_t split_target = std::max<int64_t>(1, (target + units - 1) / units);
  if (a->num_splits > 0) {
    split_target = a->num_splits;
  } else if (a->kv_lens_host) {
    int64_t total = 0;
    for (int b = 0; b < a->batch; ++b) total += std::min(a->kv_lens_host[b], L);
    if (total * 5 < static_cast<int64_t>(a->batch) * L * 4) {
      // ragged batch: ranges sized so the batch yields about three workgroups per slot
      // (measured on the ragged two-query workload: 1, 2, 3, 4 per slot give an
      // attention kernel of 370, 332, 323, 335 us; more ranges balance the lengths
      // better until the combine's extra partial rows outweigh it)
      const int64_t per_wg = std::max<int64_t>(kTile, (total * p.hgroups + 3 * target - 1) / (3 * target));
      split_target = std::max<int64_t>(1, (L + per_wg - 1) / per_wg);
    }
  }
  split_target = std::min<int64_t>(split_target, (L + kTile - 1) / kTile);
  split_target = std::max<int64_t>(split_target, 1);
  int64_t chunk = (L + split_target - 1) / split_target;
  chunk = (chunk + kTile - 1) / kTile * kTile;
  p.chunk = static_cast<int>(chunk);
  p.n_splits = static_cast<int>((L + chunk - 1) / chunk);
  // combine grid: (h, 2 latent halves, M / rows); halve the rows until the grid fills
  // the CUs; splits staged per batch fill the 256 half-row slots
  // with 16 or more query rows, workgroups of up to 16 rows that stage 128 half rows,
  // two per CU (one stages while the other computes: measured faster at every such
  // shape); else up to 32 rows and 256 half rows, so few rows take many splits at once
  const int M = a->batch * a->n_q;
  p.comb_slots = M >= 16 ? 128 : 256;
  p.comb_rows = std::min(p.comb_slots == 128 ? 16 : 32, M);
  while (p.comb_rows > 1 && 2LL * r.h * ((M + p.comb_rows - 1) / p.comb_rows) < 256) p.comb_rows = (p.comb_rows + 1) / 2;
  p.comb_splits = std::min(p.n_splits, p.comb_slots / p.comb_rows);
  // ragged lengths: the combine reads the lengths before staging partial rows, so the
  // rows of short sequences load only the splits that hold their tokens
  p.ragged = false;
  if (a->kv_lens_host)
    for (int b = 1; b < a->batch; ++b) p.ragged |= a->kv_lens_host[b] != a->kv_lens_host[0];
  return p;
}

struct Workspace {
  size_t q_cat, o_part, ml_part, gate, scores, o_lat, total;
};

Workspace layout_ws(const Resolved& r, const mla_decode_args* a, const Plan* p) {
  Workspace w{};
  const size_t M = static_cast<size_t>(a->batch) * a->n_q;
  size_t off = 0;
  if (r.dtype == MLA_BF16) {
    const size_t row = 512 + r.d_r;
    w.q_cat = off;
    off = align_up(off + M * r.h * row * 2);
    const size_t prow = static_cast<size_t>(a->batch) * p->n_splits * a->n_q * r.h;
    w.o_part = off;
    off = align_up(off + prow * 512 * 2);
    w.ml_part = off;
    off = align_up(off + prow * 2 * 4);
    if (a->gate_x) {
      w.gate = off;
      off = align_up(off + static_cast<size_t>(kGateSplit) * M * r.h * 128 * 4);
    }
  } else {
    w.q_cat = off;
    off = align_up(off + M * r.h * (r.d_c + r.d_r) * 4);
    w.scores = off;
    off = align_up(off + M * r.h * static_cast<size_t>(a->max_kv_len) * 4);
    w.o_lat = off;
    off = align_up(off + M * r.h * r.d_c * 4);
  }
  w.total = off;
  return w;
}

mla_status check_decode(const Resolved& r, const mla_decode_args* a) {
  if (!a) return MLA_E_NULL;
  if (a->batch <= 0 || a->n_q <= 0 || a->max_kv_len < a->n_q) return MLA_E_SHAPE;
  if (!a->workspace_bytes) return MLA_E_NULL;
  if ((a->gate_x == nullptr) != (a->w_gate == nullptr)) return MLA_E_NULL;
  if ((a->ev_attn_begin == nullptr) != (a->ev_attn_end == nullptr)) return MLA_E_NULL;
  if (a->gate_x && a->d_model <= 0) return MLA_E_SHAPE;
  if (a->num_splits < 0) return MLA_E_SHAPE;
  if (a->kv_lens_host) {
    for (int b = 0; b < a->batch; ++b)
      if (a->kv_lens_host[b] < a->n_q || a->kv_lens_host[b] > a->max_kv_len) return MLA_E_SHAPE;
  }
  if (r.dtype == MLA_BF16) {
    const int rows = r.h * a->n_q;
    if (rows % 64 != 0) return MLA_E_UNSUPPORTED;
    const int R = rows % 128 == 0 ? 128 : 64;
    if (R % a->n_q != 0 || r.h % (R / a->n_q) != 0) return MLA_E_UNSUPPORTED;
    if (a->gate_x && (a->d_model % (kGateSplit * 16) != 0 || (r.h * 128) % 128 != 0)) return MLA_E_UNSUPPORTED;
  }
  return MLA_OK;
}

mla_status decode_impl(const mla_dims* dims, const CacheRef& cache, const mla_decode_args* a,
                       hipStream_t stream) {
  Resolved r;
  mla_status st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  st = check_decode(r, a);
  if (st != MLA_OK) return st;
  Plan p{};
  if (r.dtype == MLA_BF16) p = plan_bf16(r, a);
  const Workspace ws = layout_ws(r, a, &p);
  if (!a->workspace) {
    *a->workspace_bytes = ws.total;
    return MLA_OK;
  }
  if (*a->workspace_bytes < ws.total) return MLA_E_WORKSPACE;
  if (!cache.data || !a->kv_lens || !a->q_nope || !a->packed_w || !a->out) return MLA_E_NULL;
  if (r.d_r > 0 && !a->q_rope) return MLA_E_NULL;
  char* wsb = static_cast<char*>(a->workspace);
  const int M = a->batch * a->n_q;
  const float qscale = r.scale * 1.4426950408889634f;

  if (r.dtype == MLA_F32) {
    F32Args f{};
    f.cache = cache;
    f.kv_lens = a->kv_lens;
    f.q_nope = static_cast<const float*>(a->q_nope);
    f.q_rope = static_cast<const float*>(a->q_rope);
    f.w_uk = static_cast<const float*>(a->packed_w);
    f.w_uv = f.w_uk + static_cast<size_t>(r.d_c) * r.h * r.d_n;
    f.gate_x = static_cast<const float*>(a->gate_x);
    f.w_gate = static_cast<const float*>(a->w_gate);
    f.q_cat = reinterpret_cast<float*>(wsb + ws.q_cat);
    f.scores = reinterpret_cast<float*>(wsb + ws.scores);
    f.o_lat = reinterpret_cast<float*>(wsb + ws.o_lat);
    f.out = a->out;
    f.lse = a->lse;
    f.batch = a->batch;
    f.n_q = a->n_q;
    f.h = r.h;
    f.d_c = r.d_c;
    f.d_r = r.d_r;
    f.d_n = r.d_n;
    f.d_v = r.d_v;
    f.d_model = a->d_model;
    f.max_kv_len = a->max_kv_len;
    f.qscale = qscale;
    f.rope_base = r.rope_base;
    return launch_decode_f32(f, a->ev_attn_begin, a->ev_attn_end, stream) == hipSuccess ? MLA_OK : MLA_E_HIP;
  }

  const uint16_t* w_uk_pk = static_cast<const uint16_t*>(a->packed_w);
  const uint16_t* w_uv_pk = w_uk_pk + static_cast<size_t>(r.h) * 8192 * 8;
  QPrepArgs q{};
  q.q_nope = static_cast<const uint16_t*>(a->q_nope);
  q.q_rope = static_cast<const uint16_t*>(a->q_rope);
  q.w_uk_pk = w_uk_pk;
  q.kv_lens = a->kv_lens;
  q.q_cat = reinterpret_cast<uint16_t*>(wsb + ws.q_cat);
  q.M = M;
  q.n_q = a->n_q;
  q.h = r.h;
  q.d_r = r.d_r;
  q.max_kv_len = a->max_kv_len;
  q.rows_per_wg = 32 * p.nw;
  q.out = a->out;  // zeroed here: the combine adds its two latent halves into it
  q.qscale = qscale;
  for (int k = 0; k < r.d_r / 2 && k < 32; ++k) q.inv_freq[k] = pow(r.rope_base, -2.0 * k / r.d_r);
  if (launch_qprep_bf16(q, stream) != hipSuccess) return MLA_E_HIP;

  if (a->gate_x) {
    GemmArgs g{};
    g.x = static_cast<const uint16_t*>(a->gate_x);
    g.w = static_cast<const uint16_t*>(a->w_gate);
    g.g = reinterpret_cast<float*>(wsb + ws.gate);
    g.M = M;
    g.K = a->d_model;
    g.N = r.h * 128;
    g.ksplit = kGateSplit;
    if (launch_splitk_gemm_bf16(g, stream) != hipSuccess) return MLA_E_HIP;
  }

  DecodeArgs d{};
  d.cache = cache;
  d.kv_lens = a->kv_lens;
  d.q_cat = q.q_cat;
  d.o_part = reinterpret_cast<uint16_t*>(wsb + ws.o_part);
  d.ml_part = reinterpret_cast<float*>(wsb + ws.ml_part);
  d.batch = a->batch;
  d.n_q = a->n_q;
  d.h = r.h;
  d.d_r = r.d_r;
  d.n_splits = p.n_splits;
  d.chunk = p.chunk;
  d.max_kv_len = a->max_kv_len;
  d.role_split = p.roles ? 1 : 0;
  if (launch_decode_bf16(d, stream, a->ev_attn_begin, a->ev_attn_end) != hipSuccess) return MLA_E_HIP;

  CombineArgs c{};
  c.o_part = d.o_part;
  c.ml_part = d.ml_part;
  c.kv_lens = a->kv_lens;
  c.w_uv_pk = w_uv_pk;
  c.gate = a->gate_x ? reinterpret_cast<const float*>(wsb + ws.gate) : nullptr;
  c.out = a->out;
  c.lse = a->lse;
  c.batch = a->batch;
  c.n_q = a->n_q;
  c.h = r.h;
  c.n_splits = p.n_splits;
  c.chunk = p.chunk;
  c.max_kv_len = a->max_kv_len;
  c.rows_per_wg = p.comb_rows;
  c.splits_per_batch = p.comb_splits;
  c.slots = p.comb_slots;
  c.lengths_first = p.ragged ? 1 : 0;
  return launch_combine_bf16(c, stream) == hipSuccess ? MLA_OK : MLA_E_HIP;
}

}  // namespace

extern "C" {

mla_status mla_absorb_weights(const mla_dims* dims, const void* w_uk, const void* w_uv, void* packed,
                              size_t* packed_bytes, hipStream_t stream) {
  Resolved r;
  mla_status st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  if (!packed_bytes) return MLA_E_NULL;
  const size_t eb = elem_bytes(r.dtype);
  const size_t uk = static_cast<size_t>(r.d_c) * r.h * r.d_n * eb;
  const size_t uv = static_cast<size_t>(r.d_c) * r.h * r.d_v * eb;
  const size_t need = uk + uv;
  if (!packed) {
    *packed_bytes = need;
    return MLA_OK;
  }
  if (*packed_bytes < need) return MLA_E_WORKSPACE;
  if (!w_uk || !w_uv) return MLA_E_NULL;
  if (r.dtype == MLA_F32) {
    // fp32 path reads the formula layout directly
    if (hipMemcpyAsync(packed, w_uk, uk, hipMemcpyDeviceToDevice, stream) != hipSuccess) return MLA_E_HIP;
    if (hipMemcpyAsync(static_cast<char*>(packed) + uk, w_uv, uv, hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return MLA_E_HIP;
    return MLA_OK;
  }
  return launch_pack_bf16(static_cast<const uint16_t*>(w_uk), static_cast<const uint16_t*>(w_uv),
                          static_cast<uint16_t*>(packed), r.h, stream) == hipSuccess
             ? MLA_OK
             : MLA_E_HIP;
}

mla_status mla_append_latent(const mla_dims* dims, void* cache, const mla_cache_layout* layout,
                             int32_t batch, int32_t n_new, const void* c_kv, const void* k_r,
                             const int32_t* pos0, hipStream_t stream) {
  Resolved r;
  mla_status st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  if (!layout) return MLA_E_NULL;
  if (batch < 0 || n_new < 0) return MLA_E_SHAPE;
  if (layout->block_table) {
    if (layout->block_size <= 0 || layout->max_blocks <= 0 || layout->n_blocks <= 0) return MLA_E_SHAPE;
  } else if (layout->t_max <= 0) {
    return MLA_E_SHAPE;
  }
  if (batch == 0 || n_new == 0) return MLA_OK;
  if (!cache || !c_kv || !pos0) return MLA_E_NULL;
  if (r.d_r > 0 && !k_r) return MLA_E_NULL;
  CacheRef c{cache, layout->block_table, layout->t_max, layout->block_size, layout->max_blocks, layout->n_blocks};
  return launch_append(r.dtype, cache, c, batch, n_new, r.d_c, r.d_r, c_kv, k_r, pos0, r.rope_base, stream) ==
                 hipSuccess
             ? MLA_OK
             : MLA_E_HIP;
}

mla_status mla_decode(const mla_dims* dims, const void* cache, int32_t t_max, const mla_decode_args* args,
                      hipStream_t stream) {
  if (t_max <= 0 || (args && t_max < args->max_kv_len)) return MLA_E_SHAPE;
  CacheRef c{cache, nullptr, t_max, 0, 0, 0};
  return decode_impl(dims, c, args, stream);
}

mla_status mla_decode_paged(const mla_dims* dims, const void* pool, const int32_t* block_table,
                            int32_t block_size, int32_t max_blocks, int32_t n_blocks,
                            const mla_decode_args* args, hipStream_t stream) {
  if (block_size <= 0 || block_size % kTile != 0 || max_blocks <= 0 || n_blocks <= 0) return MLA_E_SHAPE;
  if (args && static_cast<int64_t>(max_blocks) * block_size < args->max_kv_len) return MLA_E_SHAPE;
  if (args && args->workspace && !block_table) return MLA_E_NULL;
  CacheRef c{pool, block_table, 0, block_size, max_blocks, n_blocks};
  return decode_impl(dims, c, args, stream);
}

mla_status mla_pack_down_weights(const mla_dims* dims, int32_t d_model, const void* w_dkv, const void* w_kr,
                                 void* packed, size_t* packed_bytes, hipStream_t stream) {
  Resolved r;
  mla_status st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  if (!packed_bytes) return MLA_E_NULL;
  if (d_model <= 0) return MLA_E_SHAPE;
  const size_t need = static_cast<size_t>(d_model) * (r.d_c + r.d_r) * elem_bytes(r.dtype);
  if (!packed) {
    *packed_bytes = need;
    return MLA_OK;
  }
  if (*packed_bytes < need) return MLA_E_WORKSPACE;
  if (!w_dkv || (r.d_r > 0 && !w_kr)) return MLA_E_NULL;
  return launch_pack_down(r.dtype == MLA_F32 ? 0 : 1, w_dkv, w_kr, packed, d_model, r.d_c, r.d_r, stream) ==
                 hipSuccess
             ? MLA_OK
             : MLA_E_HIP;
}

mla_status mla_project_append(const mla_dims* dims, void* cache, const mla_cache_layout* layout,
                              const mla_project_args* a, hipStream_t stream) {
  Resolved r;
  mla_status st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  if (!layout || !a || !a->workspace_bytes) return MLA_E_NULL;
  if (a->batch < 0 || a->n_new < 0 || a->d_model <= 0 || a->k_splits < 0) return MLA_E_SHAPE;
  if (!(a->norm_eps >= 0.f) || !(a->norm_eps < INFINITY)) return MLA_E_SHAPE;
  if (layout->block_table) {
    if (layout->block_size <= 0 || layout->max_blocks <= 0 || layout->n_blocks <= 0) return MLA_E_SHAPE;
  } else if (layout->t_max <= 0) {
    return MLA_E_SHAPE;
  }
  const int N = r.d_c + r.d_r;
  const int64_t M = static_cast<int64_t>(a->batch) * a->n_new;
  if (M > (int64_t(1) << 30)) return MLA_E_UNSUPPORTED;
  int ks = 1;
  size_t need = kAlign;
  if (r.dtype == MLA_BF16) {
    // split-K product: K in 16s per split, W under 4 GiB (32-bit buffer offsets)
    if (a->d_model % 16 != 0 || static_cast<int64_t>(a->d_model) * N * 2 >= (int64_t(1) << 32))
      return MLA_E_UNSUPPORTED;
    if (a->k_splits > 0) {
      ks = a->k_splits;
      if (ks > 1024 || a->d_model % (16 * ks) != 0) return MLA_E_UNSUPPORTED;
    } else {
      ks = 32;  // about 160 workgroups for the DeepSeek widths at d_model = 4096
      while (ks > 1 && a->d_model % (16 * ks) != 0) ks /= 2;
    }
    need = std::max(need, align_up(static_cast<size_t>(ks) * M * N * 4));
  }
  if (!a->workspace) {
    *a->workspace_bytes = need;
    return MLA_OK;
  }
  if (*a->workspace_bytes < need) return MLA_E_WORKSPACE;
  if (M == 0) return MLA_OK;
  if (!cache || !a->hidden || !a->packed_down || !a->pos0) return MLA_E_NULL;

  ProjArgs p{};
  p.cache = CacheRef{cache, layout->block_table, layout->t_max, layout->block_size, layout->max_blocks,
                     layout->n_blocks};
  p.cache_out = cache;
  p.pos0 = a->pos0;
  p.hidden = a->hidden;
  p.w_down = a->packed_down;
  p.part = static_cast<const float*>(a->workspace);
  p.gain = a->norm_gain;
  p.M = static_cast<int32_t>(M);
  p.n_new = a->n_new;
  p.d_model = a->d_model;
  p.d_c = r.d_c;
  p.d_r = r.d_r;
  p.ksplit = ks;
  p.eps = a->norm_eps;
  for (int k = 0; k < r.d_r / 2 && k < kMaxRopePairs; ++k) p.inv_freq[k] = pow(r.rope_base, -2.0 * k / r.d_r);
  if (r.dtype == MLA_BF16) {
    GemmArgs g{};
    g.x = static_cast<const uint16_t*>(a->hidden);
    g.w = static_cast<const uint16_t*>(a->packed_down);
    g.g = static_cast<float*>(a->workspace);
    g.M = p.M;
    g.K = a->d_model;
    g.N = N;
    g.ksplit = ks;
    if (launch_splitk_gemm_bf16(g, stream) != hipSuccess) return MLA_E_HIP;
  }
  return launch_latent_finish(r.dtype == MLA_F32 ? 0 : 1, p, stream) == hipSuccess ? MLA_OK : MLA_E_HIP;
}

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_E_NULL: return "a required pointer is NULL";
    case MLA_E_SHAPE: return "inconsistent sizes";
    case MLA_E_DTYPE: return "unknown dtype";
    case MLA_E_UNSUPPORTED: return "shape not supported by the library's kernels";
    case MLA_E_WORKSPACE: return "workspace too small";
    case MLA_E_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
