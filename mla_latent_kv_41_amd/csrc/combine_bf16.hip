// Split combine + W_UV up-projection (+ sigmoid output gate) for the bf16 path.
//
// Combine: the splits of one (query, head) row carry (O_s / l_s, m_s, l_s), with
// O_s and l_s relative to their own running max m_s (base-2 units). The merge is
// the max-subtracted softmax of the interview guide §7.3 applied across splits:
//   M = max_s m_s,  L = Σ_s 2^(m_s - M) l_s,  o_lat = Σ_s 2^(m_s - M) l_s (O_s/l_s) / L,
//   lse = (M + log2 L) ln 2 (natural-log units).
// Up-projection (MLA tutorial page §3.1 and the `bhsc,hdc->bhsd` einsum of §5.1):
// out[m, i*128 + d] = o_lat[m, i, :] · W_UV_i[:, d], on v_mfma_f32_32x32x16_bf16.
// Gate (Gated-MLA page §2.6): out *= sigmoid(g), g = x · W_G per channel of the
// concatenated heads.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {
constexpr int kGateSplit = 16;          // K-splits of the gate GEMM
constexpr int kHalf = 256;              // latent columns per workgroup (half of d_c)
constexpr int kSlotBytes = kHalf * 2;   // one staged half partial row (bf16)
constexpr int kAStride = kHalf * 2 + 16;  // bytes per o_lat half row in LDS (padded)
// SLOTS staged half rows per batch: 256 (128 KiB, one workgroup per CU) or 128 (two
// workgroups per CU, for many row blocks: one stages while the other computes)
template <int SLOTS>
struct CombCfg {
  static constexpr int kSlots = SLOTS;
  static constexpr int kMlCap = SLOTS == 256 ? 3072 : 1024;  // (m, l) pairs staged in LDS
  static constexpr int kStageLoads = SLOTS / 2 / 4;          // partial-row loads per wave and batch
};
}  // namespace

// grid (h, 2, ceil(M / rows_per_wg)), 256 threads. Workgroup (i, kh, mb) takes head i,
// latent columns [256 kh, 256 kh + 256) and query rows m in [mb R, mb R + R), R <= 32,
// and adds its share of the up-projection,
//   out[m][i*128 + d] += Σ_{c in half kh} o_lat[m][i][c] · W_UV_i[c][d],
// into the output with fp32 atomics (the output was zeroed by the query preparation of
// the same call). Each output element gets exactly two addends onto zero, so the sum
// does not depend on their order. Splitting the latent dimension, not the rows, reads
// each partial row and each W_UV_i once.
//
// Loads go out in the order they are needed, and each wave waits with explicit
// vmcnt bounds (loads complete in issue order): the sequence lengths and every
// (m_s, l_s) of the rows, then this batch's partial half rows, all straight into
// LDS; the statistics wait for the first two only. The W_UV_i fragments follow once
// the statistics are done, and the merge waits for the partial rows only. Partial
// rows of splits past a sequence's end are staged too (the merge skips them), so
// every wave issues a fixed number of loads; slots past the rows read zeros.
template <int SLOTS>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  using CC = CombCfg<SLOTS>;
  constexpr int kSlots = CC::kSlots, kMlCap = CC::kMlCap, kStageLoads = CC::kStageLoads;
  static_assert(32 * kAStride * 2 <= kSlots * kSlotBytes, "o_lat staging fits the slots");
  __shared__ __attribute__((aligned(1024))) char s_part[kSlots * kSlotBytes];
  __shared__ __attribute__((aligned(16))) float s_ml[kMlCap * 2];  // (m, l) of (row, split)
  __shared__ float s_w[kSlots];     // weight of each staged half row
  __shared__ int s_kv[64];          // per row: sequence length (the load writes all 64 lanes)
  __shared__ int s_ns[32];          // per row: number of splits holding its tokens
  __shared__ float s_stat[32][2];   // per row: max M and 1 / L
  const int i = blockIdx.x, kh = blockIdx.y, mb = blockIdx.z;
  const int tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int M = a.batch * a.n_q;
  const int RPW = a.rows_per_wg, SB = a.splits_per_batch, NS = a.n_splits;
  const int m0 = mb * RPW;
  const int rows = min(RPW, M - m0);
  const int hl = l >> 5, cl = l & 31;

  auto part_row = [&](int m, int sp) -> int64_t {  // row index of split sp of query row m, head i
    const int b = m / a.n_q, j = m - b * a.n_q;
    return ((static_cast<int64_t>(b) * NS + sp) * a.n_q + j) * a.h + i;
  };
  const u32x4 rs_part = buffer_rsrc(a.o_part, static_cast<uint32_t>(
      static_cast<int64_t>(a.batch) * NS * a.n_q * a.h * 512 * 2));
  // one batch of partial half rows (r, s0 + q) into slot r*SB + q: wave load k of
  // wave w covers slots 2p, 2p + 1 with p = w + 4k (lanes 0-31 and 32-63). The lane's
  // slot advances by 8 per load; its row r, split q and the row's (b, j) = (m / n_q,
  // m % n_q) are stepped, not divided, per load.
  const int64_t split_stride = static_cast<int64_t>(a.n_q) * a.h * 1024;  // bytes per split
  auto stage = [&](int s0) __attribute__((always_inline)) {
    int r = (2 * w + hl) / SB, q = (2 * w + hl) - r * SB;
    int b = (m0 + r) / a.n_q, j = (m0 + r) - b * a.n_q;
#pragma unroll 1
    for (int k = 0; k < kStageLoads; ++k) {  // a loop: this code runs once per workgroup,
                                              // so its size costs instruction fetches
      const int sp = s0 + q;
      bool ok = r < rows && sp < NS;
      if (a.lengths_first && ok) {  // uniform; the row's length is in LDS already
        const int kv = min(s_kv[r], a.max_kv_len);
        ok = kv >= a.n_q && sp * a.chunk < kv;
      }
      const int64_t row0 = ((static_cast<int64_t>(b) * NS) * a.n_q + j) * a.h + i;  // split 0
      const uint32_t off = ok ? static_cast<uint32_t>(row0 * 1024 + sp * split_stride + kh * kHalf * 2 + cl * 16) : kOobOffset;
      dma_b128(rs_part, off, 0u, lds_addr(s_part) + (w + 4 * k) * 2 * kSlotBytes);
      for (q += 8; q >= SB; q -= SB) {
        ++r;
        if (++j == a.n_q) { j = 0; ++b; }
      }
    }
  };

  // ---- loads: sequence lengths (wave 0), (m_s, l_s) of all rows x splits, batch 0.
  //      Ragged batches wait for the lengths first, so that the partial rows of
  //      splits past a row's last one are not loaded at all (they read as zeros).
  {
    const u32x4 rs_ml = buffer_rsrc(a.ml_part, static_cast<uint32_t>(
        static_cast<int64_t>(a.batch) * NS * a.n_q * a.h * 2 * 4));
    if (w == 0) {
      const u32x4 rs_kv = buffer_rsrc(a.kv_lens, static_cast<uint32_t>(a.batch * 4));
      dma_b32(rs_kv, l < rows ? static_cast<uint32_t>(((m0 + l) / a.n_q) * 4) : kOobOffset, lds_addr(s_kv));
    }
    const int nf = rows * NS * 2;  // floats
    for (int q = w; 64 * q < nf; q += 4) {  // uniform
      const int f = 64 * q + l, pi = f >> 1;
      const int r = pi / NS, sp = pi - r * NS;
      const uint32_t off = f < nf ? static_cast<uint32_t>((part_row(m0 + r, sp) * 2 + (f & 1)) * 4) : kOobOffset;
      dma_b32(rs_ml, off, lds_addr(s_ml) + 64 * q * 4);
    }
    if (a.lengths_first) {
      wait_vm<0>();
      lds_barrier();  // the lengths, for every wave
    }
    stage(0);
  }
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kStageLoads) : "memory");  // lengths and (m, l) landed
  lds_barrier();

  // ---- per row (wave w: rows w + 4k): splits holding tokens, M = max_s m_s,
  //      L = Σ_s 2^(m_s - M) l_s, batch 0 weights 2^(m_s - M) l_s / L, lse. Lanes work
  //      in parallel: lane l holds row l's split count, lane sp split sp of each row
  //      (sp >= 64: a loop); the reductions run on DPP, not through LDS, which the
  //      partial rows are streaming into.
  int ns_lane = 0;  // lane l < rows: splits holding tokens of row l
  if (l < rows) {
    const int kv = min(s_kv[l], a.max_kv_len);
    ns_lane = kv >= a.n_q ? min((kv + a.chunk - 1) / a.chunk, NS) : 0;
  }
  const int ns_max = wave_max_i(ns_lane);
  float lse_v[8];  // lse of row w + 4k (general path) or of this thread's row (lane sp == 0)
  if (NS <= 8) {  // uniform: thread t takes (row t / 8, split t % 8), one pass
    const int r = tid >> 3, sp = tid & 7;
    const bool live = r < rows;
    int ns = 0;
    if (live) {
      const int kv = min(s_kv[r], a.max_kv_len);
      ns = kv >= a.n_q ? min((kv + a.chunk - 1) / a.chunk, NS) : 0;
    }
    f32x2 v = *reinterpret_cast<const f32x2*>(s_ml + (min(r, rows - 1) * NS + min(sp, NS - 1)) * 2);
    if (sp >= ns) v = f32x2{-INFINITY, 0.f};
    // reductions over the 8 lanes of the row (quad permutes, then the mirrored half row)
    float mx = v[0];
    mx = fmaxf(mx, __int_as_float(dpp_mov<0xB1>(__float_as_int(mx))));
    mx = fmaxf(mx, __int_as_float(dpp_mov<0x4E>(__float_as_int(mx))));
    mx = fmaxf(mx, __int_as_float(dpp_mov<0x141>(__float_as_int(mx))));
    const float mref = mx == -INFINITY ? 0.f : mx;
    float L = sp < ns ? fast_exp2(v[0] - mref) * v[1] : 0.f;
    L += __int_as_float(dpp_mov<0xB1>(__float_as_int(L)));
    L += __int_as_float(dpp_mov<0x4E>(__float_as_int(L)));
    L += __int_as_float(dpp_mov<0x141>(__float_as_int(L)));
    const float inv_l = L > 0.f ? 1.f / L : 0.f;
    lse_v[0] = L > 0.f ? (mx + __log2f(L)) * kLn2 : -INFINITY;
    if (live && sp < SB) s_w[r * SB + sp] = sp < ns ? fast_exp2(v[0] - mref) * v[1] * inv_l : 0.f;
    if (live && sp == 0) {
      s_ns[r] = ns;
      s_stat[r][0] = mref;
      s_stat[r][1] = inv_l;
    }
  } else {
    // general: wave w takes rows w + 4k, lane sp split sp (sp >= 64: a loop), the eight
    // rows of a wave reduced together
    int nsr[8];
    float mx[8], L[8];
    f32x2 v0[8];  // (m, l) of split l of each row
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = w + 4 * k;
      nsr[k] = r < rows ? __builtin_amdgcn_readlane(ns_lane, r) : 0;
      v0[k] = *reinterpret_cast<const f32x2*>(s_ml + (min(r, rows - 1) * NS + min(l, NS - 1)) * 2);
      if (l >= nsr[k]) v0[k] = f32x2{-INFINITY, 0.f};
      mx[k] = v0[k][0];
    }
    if (NS > 64) {  // uniform
#pragma unroll
      for (int k = 0; k < 8; ++k)
        for (int sp = l + 64; sp < nsr[k]; sp += 64) mx[k] = fmaxf(mx[k], s_ml[((w + 4 * k) * NS + sp) * 2]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) mx[k] = wave_max(mx[k]);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float mref = mx[k] == -INFINITY ? 0.f : mx[k];
      L[k] = l < nsr[k] ? fast_exp2(v0[k][0] - mref) * v0[k][1] : 0.f;
    }
    if (NS > 64) {  // uniform
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float mref = mx[k] == -INFINITY ? 0.f : mx[k];
        for (int sp = l + 64; sp < nsr[k]; sp += 64) {
          const f32x2 v = *reinterpret_cast<const f32x2*>(s_ml + ((w + 4 * k) * NS + sp) * 2);
          L[k] += fast_exp2(v[0] - mref) * v[1];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) L[k] = wave_sum(L[k]);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = w + 4 * k;
      const float mref = mx[k] == -INFINITY ? 0.f : mx[k];
      const float inv_l = L[k] > 0.f ? 1.f / L[k] : 0.f;
      lse_v[k] = L[k] > 0.f ? (mx[k] + __log2f(L[k])) * kLn2 : -INFINITY;
      if (r >= rows) continue;  // uniform
      for (int sp = l; sp < SB; sp += 64) {
        float wgt = 0.f;
        if (sp < nsr[k]) {
          const f32x2 v = sp < 64 ? v0[k] : *reinterpret_cast<const f32x2*>(s_ml + (r * NS + sp) * 2);
          wgt = fast_exp2(v[0] - mref) * v[1] * inv_l;
        }
        s_w[r * SB + sp] = wgt;
      }
      if (l == 0) {
        s_ns[r] = nsr[k];
        s_stat[r][0] = mref;
        s_stat[r][1] = inv_l;
      }
    }
  }

  // ---- W_UV_i fragments of this wave's 32 output columns, 16 k-steps of half kh
  //      (the compiler waits for these before the MFMAs)
  const u32x4* wv = reinterpret_cast<const u32x4*>(a.w_uv_pk) + ((static_cast<int64_t>(i) * 4 + w) * 32 + 16 * kh) * 64 + l;
  u32x4 bfr[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) bfr[ks] = wv[ks * 64];
  asm volatile("s_waitcnt vmcnt(16)" ::: "memory");  // this wave's partial rows landed
  lds_barrier();  // every wave's rows, weights and counts

  // ---- o_lat half rows: Σ_s w_s (O_s / l_s). A wave takes two rows per pass (lanes
  //      0-31 row w + 8p, lanes 32-63 row w + 8p + 4), a lane 8 columns.
  float o[4][8];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[p][e] = 0.f;
  // slots of splits past a row's last split hold stale rows (staged anyway, so every
  // wave issues a fixed number of loads): zero them, so the merge can take every
  // slot of a batch with weight 0 there
  auto clear_stale = [&](int s0) __attribute__((always_inline)) {
    if (a.lengths_first) return;  // those slots were loaded as zeros
    if (!__builtin_amdgcn_ballot_w64(l < rows && ns_lane < s0 + min(SB, NS - s0))) return;  // uniform
    for (int e = tid; e < rows * SB * 32; e += 256) {  // 16-byte pieces
      const int slot = e >> 5, r = slot / SB, sp = s0 + slot - r * SB;
      if (sp >= s_ns[r]) *(lds_u32x4*)(lds_ptr(s_part) + slot * kSlotBytes + (e & 31) * 16) = u32x4{0u, 0u, 0u, 0u};
    }
    lds_barrier();
  };
  for (int s0 = 0; s0 < ns_max; s0 += SB) {
    if (s0 > 0) {  // later batches (more splits than one batch stages)
      lds_barrier();  // every wave is done with the previous batch
      for (int slot = tid; slot < rows * SB; slot += 256) {
        const int r = slot / SB, sp = s0 + slot % SB;
        float wgt = 0.f;
        if (sp < s_ns[r]) {
          const f32x2 v = *reinterpret_cast<const f32x2*>(s_ml + (r * NS + sp) * 2);
          wgt = fast_exp2(v[0] - s_stat[r][0]) * v[1] * s_stat[r][1];
        }
        s_w[slot] = wgt;
      }
      stage(s0);
      wait_vm<0>();
      lds_barrier();
    }
    clear_stale(s0);
    // every slot of the batch, 8 at a time with the reads ahead of the arithmetic
    const int nb_s = min(SB, NS - s0);  // staged splits of this batch
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = w + 8 * p + 4 * hl;
      if (w + 8 * p >= rows) break;  // uniform
      const bool row_ok = r < rows;
      for (int q0 = 0; q0 < nb_s; q0 += 8) {
        float wq[8];
        u32x4 vq[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const bool ok = row_ok && q0 + u < nb_s;
          const int slot = ok ? r * SB + q0 + u : 0;
          wq[u] = ok ? s_w[slot] : 0.f;
          vq[u] = *(lds_u32x4*)(lds_ptr(s_part) + slot * kSlotBytes + cl * 16);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[p][2 * e] += wq[u] * __uint_as_float(vq[u][e] << 16);
            o[p][2 * e + 1] += wq[u] * __uint_as_float(vq[u][e] & 0xFFFF0000u);
          }
      }
    }
  }
  lds_barrier();  // every wave is done with the staged rows

  // ---- o_lat as a hi + lo pair of bf16 rows (hi = bf16(o), lo = bf16(o - hi)), so
  //      the up-projection keeps about 16 significant bits of o_lat; rows past
  //      `rows` are zero
  char* s_hi = s_part;
  char* s_lo = s_part + 32 * kAStride;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = w + 8 * p + 4 * hl;
    u32x4 hv = {0u, 0u, 0u, 0u}, lv = {0u, 0u, 0u, 0u};
    if (r < rows) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = o[p][2 * e], x1 = o[p][2 * e + 1];
        const uint32_t h2 = pack_bf16x2(x0, x1);
        hv[e] = h2;
        lv[e] = pack_bf16x2(x0 - __uint_as_float(h2 << 16), x1 - __uint_as_float(h2 & 0xFFFF0000u));
      }
    }
    *(lds_u32x4*)(lds_ptr(s_hi) + r * kAStride + cl * 16) = hv;
    *(lds_u32x4*)(lds_ptr(s_lo) + r * kAStride + cl * 16) = lv;
  }
  lds_barrier();

  // ---- out[m][i*128 + 32w + ..] += (o_hi + o_lo)[m][half kh] · W_UV_i[half kh][32w + ..]
  f32x16 acc = {};
  const int arow = (l & 31) * kAStride + (l >> 5) * 16;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const u32x4 ah = *(lds_u32x4*)(lds_ptr(s_hi) + arow + ks * 32);
    const u32x4 al = *(lds_u32x4*)(lds_ptr(s_lo) + arow + ks * 32);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ah), as_bf16x8(bfr[ks]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(al), as_bf16x8(bfr[ks]), acc, 0, 0, 0);
  }
  const int width = a.h * 128;
  const int col = i * 128 + 32 * w + (l & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = 8 * (v / 4) + 4 * (l >> 5) + (v & 3);
    if (r >= rows) continue;
    const int m = m0 + r;
    float ov = acc[v];
    if (a.gate) {  // out = sigmoid(g) (o_0 + o_1): each half carries its factor
      float g = 0.f;
      for (int ks = 0; ks < kGateSplit; ++ks) g += a.gate[(static_cast<int64_t>(ks) * M + m) * width + col];
      ov *= 1.f / (1.f + __expf(-g));
    }
    atomicAdd(a.out + static_cast<int64_t>(m) * width + col, ov);
  }
  if (kh == 0 && a.lse) {
    if (NS <= 8) {
      if ((tid & 7) == 0 && (tid >> 3) < rows) a.lse[static_cast<int64_t>(m0 + (tid >> 3)) * a.h + i] = lse_v[0];
    } else if (l == 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (w + 4 * k < rows) a.lse[static_cast<int64_t>(m0 + w + 4 * k) * a.h + i] = lse_v[k];
    }
  }
}

hipError_t launch_combine_bf16(const CombineArgs& a, hipStream_t s) {
  const int M = a.batch * a.n_q;
  const bool half = a.rows_per_wg <= 16 && a.rows_per_wg * a.splits_per_batch <= CombCfg<128>::kSlots &&
                    a.rows_per_wg * a.n_splits <= CombCfg<128>::kMlCap && a.slots == 128;
  const int slots = half ? CombCfg<128>::kSlots : CombCfg<256>::kSlots;
  const int ml_cap = half ? CombCfg<128>::kMlCap : CombCfg<256>::kMlCap;
  if (a.rows_per_wg < 1 || a.rows_per_wg > 32 || a.rows_per_wg * a.splits_per_batch > slots ||
      a.rows_per_wg * a.n_splits > ml_cap)
    return hipErrorInvalidValue;
  // buffer offsets are 32-bit
  if (static_cast<int64_t>(a.batch) * a.n_splits * a.n_q * a.h * 512 * 2 >= (int64_t(1) << 32) - 16)
    return hipErrorInvalidValue;
  const dim3 grid(a.h, 2, (M + a.rows_per_wg - 1) / a.rows_per_wg);
  if (half)
    combine_kernel<128><<<grid, 256, 0, s>>>(a);
  else
    combine_kernel<256><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
