// libmla C ABI: argument checking, split planning, workspace layout and launches.
//
// Every check below runs on the host before any HIP call, so a rejected call
// never touches the device.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "mla.h"
#include "launch.hpp"

using namespace mla;

// The allocation-free decode's workspace: one array on each GPU the library runs
// on, held until the process ends. kScratchBytes covers the DeepSeek-shaped step
// (32 sequences of 4097 tokens: about 43 MB without host lengths) and anything that
// needs as much workspace.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr size_t kAlign = 256;
constexpr int kTile = 32;       // tokens per attention tile; split ranges are multiples of it

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
//
// Sequences shorter than kPreciseBelow tokens take the precise attention form (query
// and probabilities as hi + lo bf16 pairs); longer ones the fast form (one bf16
// query). Over a few thousand tokens the bf16 roundings of the query and of P
// average out to well inside the error bar of the fp32 reference; below that they do
// not, and a short sequence costs little either way.
constexpr int kPreciseBelow = 4096;
constexpr int kMaxSplitsPerSeq = 1024;  // bound on a sequence's token ranges
constexpr int kMinRaggedChunk = 256;   // tokens per range at least, ragged batches
constexpr int kRaggedPerSlot = 1;      // ragged batches: workgroups per CU slot
constexpr int kRowsRangeMin = 1024;     // see the fast form's choice below
#ifndef MLA_FAST64_FORM
#define MLA_FAST64_FORM kFormPingPong
#endif
constexpr int kFast64Form = MLA_FAST64_FORM;  // the fast form of 64-row workgroups

struct Plan {
  int fast_form;     // kForm128 (rows a multiple of 128) or kFormRoles
  int fast_groups;   // head groups (workgroups) per pair in the fast form
  int prec_groups;   // ... in the precise form (64-row workgroups)
  int chunk;         // tokens per range of the fast form's sequences, a multiple of kTile
  int chunk_precise; // ... of the precise form's sequences
  int64_t cap;       // pairs the workspace holds: a bound on Σ_b ceil(kv_b / chunk)
  int64_t fast_pairs, prec_pairs;  // bounds on the pairs of each list (0: not launched)
  int comb_rows;     // combine: query rows per workgroup (32, 16, 8, 4, 2 or 1)
};

int64_t ceil_div(int64_t x, int64_t y) { return (x + y - 1) / y; }

Plan plan_bf16(const Resolved& r, const mla_decode_args* a) {
  Plan p{};
  const int rows = r.h * a->n_q;
  const int64_t L = a->max_kv_len;
  const int64_t target = 256;  // workgroups per wave of the chip: one per CU
  // The fast form: 128-row workgroups run the attention's steady state faster, but
  // each range writes 128 partial rows of 2 KB. When the longest sequences would get
  // ranges shorter than kRowsRangeMin tokens in that form (one range per CU, as on
  // the DeepSeek-shaped and the long paged workloads), the role-split 64-row form,
  // which needs half as many ranges, moves fewer bytes in all: measured per step
  // 78.6 against 84.4 us (DeepSeek-shaped) and 75.9 against 82.3 us (paged), while
  // the ragged two-query workload keeps 128-row ranges of ~1.5K tokens (455 against
  // 557 us).
  p.fast_form = kFast64Form;
#ifndef MLA_NO_FORM128
  if (rows % 128 == 0 && a->num_splits == 0) {
#else
  if (false) {
#endif
    const int64_t units = static_cast<int64_t>(a->batch) * (rows / 128);
    const int64_t c128 = ceil_div(L, std::min(ceil_div(target, units), ceil_div(L, kTile)));
    if (c128 >= kRowsRangeMin) p.fast_form = kForm128;
  } else if (rows % 128 == 0) {
    p.fast_form = kForm128;
  }
  p.fast_groups = rows / (p.fast_form == kForm128 ? 128 : 64);
  p.prec_groups = rows / 64;
  auto groups_of = [&](int64_t kv) { return kv < kPreciseBelow ? p.prec_groups : p.fast_groups; };
  bool ragged = false;
  int64_t total = 0, total_units = 0;  // tokens, and tokens x head groups
  if (a->kv_lens_host) {
    for (int b = 0; b < a->batch; ++b) {
      const int64_t kv = std::min<int64_t>(a->kv_lens_host[b], L);
      total += kv;
      total_units += kv * groups_of(kv);
    }
    ragged = total * 5 < static_cast<int64_t>(a->batch) * L * 4;
  }
  // with host lengths: the precise form's tokens, and whether both forms run (the
  // precise launch then gets ranges of its own, below)
  int64_t prec_units = 0;
  bool any_fast = false;
  if (a->kv_lens_host) {
    for (int b = 0; b < a->batch; ++b) {
      const int64_t kv = std::min<int64_t>(a->kv_lens_host[b], L);
      if (kv < kPreciseBelow) prec_units += kv * p.prec_groups;
      else any_fast = true;
    }
  }
  const bool own_precise = a->kv_lens_host && a->num_splits == 0 && any_fast && prec_units > 0;
  // workgroups of a launch with ranges of ch tokens over the fast form's sequences
  // (which 0), the precise form's (1) or all (2), from the host lengths
  auto workgroups = [&](int64_t ch, int which) {
    int64_t n = 0;
    for (int b = 0; b < a->batch; ++b) {
      const int64_t kv = std::min<int64_t>(a->kv_lens_host[b], L);
      const bool prec = kv < kPreciseBelow;
      if (kv < a->n_q || (which == 0 && prec) || (which == 1 && !prec)) continue;
      n += ceil_div(kv, ch) * groups_of(kv);
    }
    return n;
  };
  // The shortest range length from `base` (a multiple of kTile) whose launch fits in
  // `limit` workgroups. Every sequence's last range is a remainder, so ranges sized
  // from the token total alone can leave a launch a few workgroups past its last full
  // wave of the chip, and those run as one more wave (the ragged two-query workload's
  // precise launch: 276 workgroups of at most 14 tiles, against 248 of at most 16 at
  // 512-token ranges). Taken when under twice `base`, since two waves of `base`-token
  // ranges cost no more.
  auto fit = [&](int64_t base, int64_t limit, int which) -> int64_t {
    const int64_t top = ceil_div(L, kTile) * kTile;
    if (base >= top || workgroups(base, which) <= limit) return base;
    int64_t lo = base / kTile, hi = top / kTile;  // workgroups(lo * kTile) > limit
    if (workgroups(hi * kTile, which) > limit) return base;
    while (hi - lo > 1) {
      const int64_t mid = (lo + hi) / 2;
      if (workgroups(mid * kTile, which) <= limit) hi = mid;
      else lo = mid;
    }
    return hi * kTile < 2 * base ? hi * kTile : base;
  };
  int64_t chunk;
  if (a->num_splits > 0) {
    chunk = ceil_div(L, a->num_splits);
  } else if (ragged) {
    // ranges sized so the batch yields about one workgroup per slot, fitted below to
    // one whole wave: more ranges balance the lengths better, but every range writes
    // fp32 partial rows that the combine reads back (on the ragged two-query workload
    // two per slot make the attention 8 us shorter and the combine 13 us longer), at
    // least kMinRaggedChunk tokens, so the partials of a range stay well below the
    // cache bytes it reads
    chunk = std::max<int64_t>(kMinRaggedChunk, ceil_div(total_units, kRaggedPerSlot * target));
  } else {
    // at most one workgroup per slot when every sequence is as long as the longest:
    // as many ranges per sequence as fit the chip whole (a few past it would run as
    // a second wave)
    const int64_t units = static_cast<int64_t>(a->batch) * groups_of(L);
    chunk = ceil_div(L, std::min(std::max<int64_t>(1, target / units), ceil_div(L, kTile)));
  }
  chunk = std::max(chunk, ceil_div(L, kMaxSplitsPerSeq));
  chunk = std::min(ceil_div(chunk, kTile) * kTile, ceil_div(L, kTile) * kTile);
  if (ragged && a->num_splits == 0) chunk = fit(chunk, kRaggedPerSlot * target, own_precise ? 0 : 2);
  p.chunk = static_cast<int>(chunk);
  p.chunk_precise = p.chunk;
  if (own_precise) {
    // the precise launch follows the fast one on its own: its ranges are sized so its
    // sequences' units fill the chip once (at least kMinRaggedChunk tokens), rather
    // than by the fast form's ranges
    const int64_t c = std::max<int64_t>(kMinRaggedChunk, ceil_div(prec_units, target));
    p.chunk_precise = static_cast<int>(fit(std::min<int64_t>(ceil_div(c, kTile) * kTile, ceil_div(L, kTile) * kTile), target, 1));
  }
  if (a->kv_lens_host) {
    for (int b = 0; b < a->batch; ++b) {
      const int64_t kv = std::min<int64_t>(a->kv_lens_host[b], L);
      const bool prec = kv < kPreciseBelow;
      const int64_t ns = kv >= a->n_q ? ceil_div(kv, prec ? p.chunk_precise : p.chunk) : 0;
      p.cap += ns;
      (prec ? p.prec_pairs : p.fast_pairs) += ns;
    }
  } else {
    // any length up to max_kv_len: both lists may fill
    p.cap = static_cast<int64_t>(a->batch) * ceil_div(L, p.chunk);
    p.fast_pairs = L >= kPreciseBelow ? p.cap : 0;
    p.prec_pairs = p.cap;
  }
  // combine grid: (h, M / rows), rows 32, 16, 8, 4, 2 or 1: halved until the grid has a
  // workgroup per CU
  const int M = a->batch * a->n_q;
  p.comb_rows = 32;
  while (p.comb_rows > 1 && static_cast<int64_t>(r.h) * ceil_div(M, p.comb_rows) < target) p.comb_rows /= 2;
  return p;
}

struct Workspace {
  size_t counts, seq_off, fast_list, prec_list, q_cat, q_lo, o_part, ml_part, gate, scores, o_lat, total;
};

Workspace layout_ws(const Resolved& r, const mla_decode_args* a, const Plan* p) {
  Workspace w{};
  const size_t M = static_cast<size_t>(a->batch) * a->n_q;
  size_t off = 0;
  if (r.dtype == MLA_BF16) {
    const size_t row = 512 + r.d_r;
    const size_t cap = static_cast<size_t>(std::max<int64_t>(p->cap, 1));
    w.counts = off;
    off = align_up(off + 2 * sizeof(int32_t));
    w.seq_off = off;
    off = align_up(off + (static_cast<size_t>(a->batch) + 1) * sizeof(int32_t));
    // both lists always exist (the device plan may fill either), each with kListPad
    // entries past cap: a launch's grid, padded to 8 workgroups, reads up to there
    w.fast_list = off;
    off = align_up(off + (cap + kListPad) * sizeof(WorkItem));
    w.prec_list = off;
    off = align_up(off + (cap + kListPad) * sizeof(WorkItem));
    w.q_cat = off;
    off = align_up(off + M * r.h * row * 2);
    if (p->prec_pairs > 0) {
      w.q_lo = off;
      off = align_up(off + M * r.h * row * 2);
    }
    const size_t prow = cap * a->n_q * r.h;
    w.o_part = off;
    off = align_up(off + prow * 512 * 4);
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
    // 32-head query blocks, 64 or 128 rows per attention workgroup
    if (r.h % 32 != 0 || (static_cast<int64_t>(r.h) * a->n_q) % 64 != 0) return MLA_E_UNSUPPORTED;
    if (a->gate_x && a->d_model % (kGateSplit * 16) != 0) return MLA_E_UNSUPPORTED;
    // every grid dimension and element offset the kernels form stays in range
    if (static_cast<int64_t>(a->batch) * a->n_q > (int64_t(1) << 24) || r.h > 4096) return MLA_E_UNSUPPORTED;
  }
  return MLA_OK;
}

// latent: the absorbed query is given in args->q_nope ([B][n_q][h][d_c] fp32) and the
// merged latent output goes to args->out ([B][n_q][h][d_c] fp32): no W_UK, W_UV or gate.
mla_status decode_impl(const mla_dims* dims, const CacheRef& cache, const mla_decode_args* a,
                       hipStream_t stream, bool latent = false) {
  Resolved r;
  mla_status st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  st = check_decode(r, a);
  if (st != MLA_OK) return st;
  if (latent && (r.dtype != MLA_BF16 || a->gate_x)) return MLA_E_UNSUPPORTED;
  Plan p{};
  if (r.dtype == MLA_BF16) p = plan_bf16(r, a);
  const Workspace ws = layout_ws(r, a, &p);
  if (!a->workspace) {
    *a->workspace_bytes = ws.total;
    return MLA_OK;
  }
  if (*a->workspace_bytes < ws.total) return MLA_E_WORKSPACE;
  if (!cache.data || !a->kv_lens || !a->q_nope || (!a->packed_w && !latent) || !a->out) return MLA_E_NULL;
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

  const uint16_t* w_uk_pk = latent ? nullptr : static_cast<const uint16_t*>(a->packed_w);
  const uint16_t* w_uv_pk = latent ? nullptr : w_uk_pk + static_cast<size_t>(r.h) * 8192 * 8;
  // grids: the pairs a list may hold x head groups, padded to a multiple of 8 (one
  // run of units per XCD; the extra workgroups find no pair and return)
  auto grid_units = [](int64_t pairs, int groups) -> int64_t {
    const int64_t u = pairs * groups;
    return u >= 8 ? (u + 7) / 8 * 8 : u;
  };
  const int64_t fast_units = grid_units(p.fast_pairs, p.fast_groups);
  const int64_t prec_units = grid_units(p.prec_pairs, p.prec_groups);
  if (fast_units > INT32_MAX || prec_units > INT32_MAX || p.cap > INT32_MAX) return MLA_E_UNSUPPORTED;

  int32_t* counts = reinterpret_cast<int32_t*>(wsb + ws.counts);
  WorkItem* fast_list = reinterpret_cast<WorkItem*>(wsb + ws.fast_list);
  WorkItem* prec_list = reinterpret_cast<WorkItem*>(wsb + ws.prec_list);
  QPrepArgs q{};
  q.q_nope = static_cast<const uint16_t*>(a->q_nope);
  q.q_rope = static_cast<const uint16_t*>(a->q_rope);
  q.w_uk_pk = w_uk_pk;
  q.kv_lens = a->kv_lens;
  q.q_cat = reinterpret_cast<uint16_t*>(wsb + ws.q_cat);
  q.q_lo = p.prec_pairs > 0 ? reinterpret_cast<uint16_t*>(wsb + ws.q_lo) : nullptr;
  q.q_abs = latent ? static_cast<const float*>(a->q_nope) : nullptr;
  q.M = M;
  q.n_q = a->n_q;
  q.h = r.h;
  q.d_r = r.d_r;
  q.max_kv_len = a->max_kv_len;
  q.qscale = qscale;
  for (int k = 0; k < r.d_r / 2 && k < 32; ++k) q.inv_freq[k] = pow(r.rope_base, -2.0 * k / r.d_r);
  q.plan.kv_lens = a->kv_lens;
  q.plan.batch = a->batch;
  q.plan.n_q = a->n_q;
  q.plan.max_kv_len = a->max_kv_len;
  q.plan.chunk_fast = p.chunk;
  q.plan.chunk_precise = p.chunk_precise;
  q.plan.precise_below = kPreciseBelow;
  q.plan.cap = static_cast<int32_t>(p.cap);
  q.plan.counts = counts;
  q.plan.seq_off = reinterpret_cast<int32_t*>(wsb + ws.seq_off);
  q.plan.fast = fast_list;
  q.plan.precise = prec_list;
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

  // the attention launches: the fast form over the long sequences' pairs, then the
  // precise form over the short ones'; the timing events bracket both
  DecodeArgs d{};
  d.cache = cache;
  d.q_cat = q.q_cat;
  d.q_lo = q.q_lo;
  d.o_part = reinterpret_cast<float*>(wsb + ws.o_part);
  d.ml_part = reinterpret_cast<float*>(wsb + ws.ml_part);
  d.n_q = a->n_q;
  d.h = r.h;
  d.d_r = r.d_r;
  d.chunk = p.chunk;
  const bool two = fast_units > 0 && prec_units > 0;
  if (two && p.fast_form == kForm128 && fast_units % 8 == 0) {
    // both forms in one grid (their block shapes agree): the precise units fill
    // the CUs that the shorter fast ranges leave first, rather than waiting for the
    // longest of them
    d.list = fast_list;
    d.form = p.fast_form;
    d.units = static_cast<int32_t>(fast_units);
    if (launch_decode_mixed_bf16(d, prec_list, p.chunk_precise, static_cast<int32_t>(prec_units), stream,
                                 a->ev_attn_begin, a->ev_attn_end) != hipSuccess)
      return MLA_E_HIP;
  } else {
    if (fast_units > 0) {
      d.list = fast_list;
      d.form = p.fast_form;
      d.units = static_cast<int32_t>(fast_units);
      if (launch_decode_bf16(d, stream, a->ev_attn_begin, two ? nullptr : a->ev_attn_end) != hipSuccess)
        return MLA_E_HIP;
    }
    if (prec_units > 0) {
      d.list = prec_list;
      d.chunk = p.chunk_precise;
      d.form = kFormPrecise;
      d.units = static_cast<int32_t>(prec_units);
      if (launch_decode_bf16(d, stream, two ? nullptr : a->ev_attn_begin, a->ev_attn_end) != hipSuccess)
        return MLA_E_HIP;
    }
  }

  CombineArgs c{};
  c.o_part = d.o_part;
  c.ml_part = d.ml_part;
  c.seq_off = q.plan.seq_off;
  c.w_uv_pk = w_uv_pk;
  c.gate = a->gate_x ? reinterpret_cast<const float*>(wsb + ws.gate) : nullptr;
  c.out = latent ? nullptr : a->out;
  c.o_lat = latent ? a->out : nullptr;
  c.lse = a->lse;
  c.batch = a->batch;
  c.n_q = a->n_q;
  c.h = r.h;
  c.rows_per_wg = p.comb_rows;
  return launch_combine_bf16(c, stream) == hipSuccess ? MLA_OK : MLA_E_HIP;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // the array's device address on each GPU, once looked up

// The current device's copy of `scratch`. The host-side name of the array is not a
// device address: host code only ever passes on the address looked up here, once per
// device, with that device current.
mla_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
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

mla_status mla_decode_latent(const mla_dims* dims, const void* cache, const mla_cache_layout* layout,
                             const mla_decode_args* args, hipStream_t stream) {
  if (!layout || !args) return MLA_E_NULL;
  CacheRef c{cache, layout->block_table, layout->t_max, layout->block_size, layout->max_blocks, layout->n_blocks};
  if (layout->block_table) {
    if (layout->block_size <= 0 || layout->block_size % kTile != 0 || layout->max_blocks <= 0 || layout->n_blocks <= 0)
      return MLA_E_SHAPE;
    if (static_cast<int64_t>(layout->max_blocks) * layout->block_size < args->max_kv_len) return MLA_E_SHAPE;
  } else if (layout->t_max <= 0 || layout->t_max < args->max_kv_len) {
    return MLA_E_SHAPE;
  }
  return decode_impl(dims, c, args, stream, true);
}

mla_status mla_decode_noalloc(const mla_dims* dims, const void* cache, const mla_cache_layout* layout,
                              const mla_decode_args* args, hipStream_t stream) {
  if (!layout || !args) return MLA_E_NULL;
  CacheRef c{cache, layout->block_table, layout->t_max, layout->block_size, layout->max_blocks, layout->n_blocks};
  if (layout->block_table) {
    if (layout->block_size <= 0 || layout->block_size % kTile != 0 || layout->max_blocks <= 0 || layout->n_blocks <= 0)
      return MLA_E_SHAPE;
    if (static_cast<int64_t>(layout->max_blocks) * layout->block_size < args->max_kv_len) return MLA_E_SHAPE;
  } else if (layout->t_max <= 0 || layout->t_max < args->max_kv_len) {
    return MLA_E_SHAPE;
  }
  // the workspace this call needs, on the host; then the same call on the scratch array
  mla_decode_args la = *args;
  size_t need = 0;
  la.workspace = nullptr;
  la.workspace_bytes = &need;
  mla_status st = decode_impl(dims, c, &la, stream);
  if (st != MLA_OK) return st;
  if (need > kScratchBytes) return MLA_E_WORKSPACE;  // past the library's scratch
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MLA_OK) return st;
  size_t have = kScratchBytes;
  la.workspace = ws;
  la.workspace_bytes = &have;
  return decode_impl(dims, c, &la, stream);
}

mla_status mla_expand_kv(const mla_dims* dims, const void* cache, const mla_cache_layout* layout, int32_t batch,
                         const int32_t* kv_lens, int32_t max_kv_len, const void* w_uk, const void* w_uv,
                         float* k_out, float* v_out, void* workspace, size_t* workspace_bytes,
                         hipStream_t stream) {
  Resolved r;
  mla_status st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  if (!layout || !workspace_bytes) return MLA_E_NULL;
  if (r.dtype != MLA_BF16) return MLA_E_UNSUPPORTED;
  if (batch <= 0 || max_kv_len <= 0) return MLA_E_SHAPE;
  if (layout->block_table) {
    if (layout->block_size <= 0 || layout->max_blocks <= 0 || layout->n_blocks <= 0) return MLA_E_SHAPE;
    if (static_cast<int64_t>(layout->max_blocks) * layout->block_size < max_kv_len) return MLA_E_SHAPE;
  } else if (layout->t_max < max_kv_len) {
    return MLA_E_SHAPE;
  }
  if (static_cast<int64_t>(batch) * ceil_div(max_kv_len, 128) > INT32_MAX || r.h > 65535) return MLA_E_UNSUPPORTED;
  const size_t need = align_up(2 * static_cast<size_t>(r.h) * 128 * r.d_c * 2);
  if (!workspace) {
    *workspace_bytes = need;
    return MLA_OK;
  }
  if (*workspace_bytes < need) return MLA_E_WORKSPACE;
  if (!cache || !kv_lens || !w_uk || !w_uv || !k_out || !v_out) return MLA_E_NULL;
  ExpandArgs e{};
  e.cache = CacheRef{cache, layout->block_table, layout->t_max, layout->block_size, layout->max_blocks,
                     layout->n_blocks};
  e.kv_lens = kv_lens;
  e.w_uk = static_cast<const uint16_t*>(w_uk);
  e.w_uv = static_cast<const uint16_t*>(w_uv);
  e.packed = static_cast<const uint16_t*>(workspace);
  e.k_out = k_out;
  e.v_out = v_out;
  e.batch = batch;
  e.max_kv_len = max_kv_len;
  e.h = r.h;
  e.d_c = r.d_c;
  e.d_r = r.d_r;
  return launch_expand(e, stream) == hipSuccess ? MLA_OK : MLA_E_HIP;
}

mla_status mla_decode_explicit(const mla_dims* dims, const float* k, const float* v, const void* cache,
                               const mla_cache_layout* layout, const mla_decode_args* a, hipStream_t stream) {
  Resolved r;
  mla_status st = resolve(dims, &r);
  if (st != MLA_OK) return st;
  if (!a || !layout || !a->workspace_bytes) return MLA_E_NULL;
  if (r.dtype != MLA_BF16) return MLA_E_UNSUPPORTED;
  if (a->batch <= 0 || a->n_q <= 0 || a->max_kv_len < a->n_q || a->num_splits < 0) return MLA_E_SHAPE;
  if (a->n_q > 4) return MLA_E_UNSUPPORTED;
  if ((a->gate_x == nullptr) != (a->w_gate == nullptr)) return MLA_E_NULL;
  if ((a->ev_attn_begin == nullptr) != (a->ev_attn_end == nullptr)) return MLA_E_NULL;
  if (a->gate_x && (a->d_model <= 0 || a->d_model % (kGateSplit * 16) != 0)) return MLA_E_UNSUPPORTED;
  if (a->kv_lens_host)
    for (int b = 0; b < a->batch; ++b)
      if (a->kv_lens_host[b] < a->n_q || a->kv_lens_host[b] > a->max_kv_len) return MLA_E_SHAPE;
  if (layout->block_table) {
    if (layout->block_size <= 0 || layout->max_blocks <= 0 || layout->n_blocks <= 0) return MLA_E_SHAPE;
    if (static_cast<int64_t>(layout->max_blocks) * layout->block_size < a->max_kv_len) return MLA_E_SHAPE;
  } else if (layout->t_max < a->max_kv_len) {
    return MLA_E_SHAPE;
  }
  // token ranges: enough (sequence, head, range) workgroups to fill the chip a few times
  const int64_t L = a->max_kv_len, M = static_cast<int64_t>(a->batch) * a->n_q;
  int64_t splits = a->num_splits > 0 ? a->num_splits
                                     : std::min(ceil_div(2048, static_cast<int64_t>(a->batch) * r.h), ceil_div(L, 256));
  splits = std::max<int64_t>(1, std::min(splits, L));
  const int64_t chunk = ceil_div(ceil_div(L, splits), 8) * 8;
  splits = ceil_div(L, chunk);
  if (static_cast<int64_t>(a->batch) * splits * r.h > INT32_MAX) return MLA_E_UNSUPPORTED;
  size_t off = 0;
  const size_t part_off = off;
  off = align_up(off + static_cast<size_t>(a->batch) * splits * a->n_q * r.h * 130 * 4);
  const size_t gate_off = off;
  if (a->gate_x) off = align_up(off + static_cast<size_t>(kGateSplit) * M * r.h * 128 * 4);
  if (!a->workspace) {
    *a->workspace_bytes = off;
    return MLA_OK;
  }
  if (*a->workspace_bytes < off) return MLA_E_WORKSPACE;
  if (!k || !v || !cache || !a->kv_lens || !a->q_nope || !a->out) return MLA_E_NULL;
  if (r.d_r > 0 && !a->q_rope) return MLA_E_NULL;
  char* wsb = static_cast<char*>(a->workspace);
  if (a->gate_x) {
    GemmArgs g{};
    g.x = static_cast<const uint16_t*>(a->gate_x);
    g.w = static_cast<const uint16_t*>(a->w_gate);
    g.g = reinterpret_cast<float*>(wsb + gate_off);
    g.M = static_cast<int32_t>(M);
    g.K = a->d_model;
    g.N = r.h * 128;
    g.ksplit = kGateSplit;
    if (launch_splitk_gemm_bf16(g, stream) != hipSuccess) return MLA_E_HIP;
  }
  ExplicitArgs e{};
  e.cache = CacheRef{cache, layout->block_table, layout->t_max, layout->block_size, layout->max_blocks,
                     layout->n_blocks};
  e.kv_lens = a->kv_lens;
  e.k = k;
  e.v = v;
  e.q_nope = static_cast<const uint16_t*>(a->q_nope);
  e.q_rope = static_cast<const uint16_t*>(a->q_rope);
  e.gate = a->gate_x ? reinterpret_cast<const float*>(wsb + gate_off) : nullptr;
  e.part = reinterpret_cast<float*>(wsb + part_off);
  e.out = a->out;
  e.lse = a->lse;
  e.batch = a->batch;
  e.n_q = a->n_q;
  e.h = r.h;
  e.d_r = r.d_r;
  e.max_kv_len = a->max_kv_len;
  e.n_splits = static_cast<int32_t>(splits);
  e.chunk = static_cast<int32_t>(chunk);
  e.qscale = r.scale * 1.4426950408889634f;
  for (int q = 0; q < r.d_r / 2 && q < 32; ++q) e.inv_freq[q] = pow(r.rope_base, -2.0 * q / r.d_r);
  return launch_explicit_decode(e, a->ev_attn_begin, a->ev_attn_end, stream) == hipSuccess ? MLA_OK : MLA_E_HIP;
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
