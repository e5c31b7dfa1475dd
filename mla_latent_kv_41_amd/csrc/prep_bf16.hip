// Weight absorption packing and query preparation for the bf16 matrix-core path.
//
// Absorption (MLA tutorial page §3.1, §3.2 and the `bhsd,hcd->bhsc` einsum of
// §5.1): W_UK is folded into the query, q_abs[m, i, :] = q_nope[m, i, :] · W_UK_iᵀ,
// a [1 x 128] · [128 x 512] product per head, batched over all M = B * n_q query
// rows so each W_UK_i is read once per step. The decoupled query key is rotated
// (interview guide §6.2; linear-algebra page "解耦 RoPE"). Both parts are scaled
// by scale * log2(e), so the attention kernel works in base-2 exponent units.
//
// Packing (done once at load, tutorial §3.2): W_UK and W_UV are re-laid out per
// head in the exact per-lane fragment order of the matrix-core instruction that
// consumes them (v_mfma_f32_32x32x16_bf16 for W_UK, v_mfma_f32_16x16x32_bf16 for
// W_UV), so every weight load in the hot kernels is one contiguous 1 KiB wave
// transaction.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

// Fragment order (64 lanes x 8 bf16 = 1 KiB per fragment):
//   W_UK (B operand of D[m][c] = q_nope[m][:] · W_UK_i[c][:]):
//     frag (i, nb < 16, ks < 8), lane l: W_UK[32nb + l%32][i*128 + 16ks + 8(l/32) + e]
//   W_UV (B operand of the 16x16x32 product D[m][d] = o_lat[m][:] · W_UV_i[:][d]):
//     frag (i, nb < 8, ks < 16), lane l: W_UV[32ks + 8(l/16) + e][i*128 + 16nb + l%16]
__global__ void pack_kernel(const uint16_t* __restrict__ w_uk, const uint16_t* __restrict__ w_uv,
                            uint16_t* __restrict__ packed, int h) {
  const int64_t per = static_cast<int64_t>(h) * 8192;  // lanes per region
  const int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= 2 * per) return;
  const int64_t width = static_cast<int64_t>(h) * 128;
  uint16_t v[8];
  if (g < per) {
    const int l = g % 64;
    const int64_t f = g / 64;
    const int ks = f % 8, nb = (f / 8) % 16, i = static_cast<int>(f / 128);
    const int64_t r = 32 * nb + l % 32;
    const int64_t c0 = static_cast<int64_t>(i) * 128 + 16 * ks + 8 * (l / 32);
    for (int e = 0; e < 8; ++e) v[e] = w_uk[r * width + c0 + e];
  } else {
    const int64_t gg = g - per;
    const int l = gg % 64;
    const int64_t f = gg / 64;
    const int ks = f % 16, nb = (f / 16) % 8, i = static_cast<int>(f / 128);
    const int64_t col = static_cast<int64_t>(i) * 128 + 16 * nb + l % 16;
    for (int e = 0; e < 8; ++e) v[e] = w_uv[(32 * ks + 8 * (l / 16) + e) * width + col];
  }
  u32x4 o;
  for (int e = 0; e < 4; ++e) o[e] = static_cast<uint32_t>(v[2 * e]) | (static_cast<uint32_t>(v[2 * e + 1]) << 16);
  *reinterpret_cast<u32x4*>(packed + g * 8) = o;
}

hipError_t launch_pack_bf16(const uint16_t* w_uk, const uint16_t* w_uv, uint16_t* packed, int h,
                            hipStream_t s) {
  const int64_t n = static_cast<int64_t>(h) * 8192 * 2;
  pack_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), 256, 0, s>>>(w_uk, w_uv, packed, h);
  return hipGetLastError();
}

// Q_cat is written in the attention kernels' B-fragment order, in blocks of 32
// query rows: block (m, i / 32) holds query row m (= b * n_q + j) of heads
// 32 (i / 32) .. + 31. Within a block, column c of head i sits at k-step c / 16,
// lane (i % 32) + 32 ((c / 8) % 2), element c % 8, so each of an attention wave's
// fragment loads is one contiguous 1 KiB read. An attention workgroup takes
// consecutive blocks of one sequence; blocks of one query are consecutive.
//
// Precise mode (q_lo != nullptr): q_lo holds bf16(x - bf16(x)) of each scaled value
// x, in the same order, so q_cat + q_lo carries about 16 significant bits of x. Only
// the rows of sequences the precise form takes (fewer than precise_below tokens)
// are written; no other kernel reads q_lo.

// Split plan of one decode call (see PlanArgs), built by one wave: lane l takes a
// contiguous run of sequences, the wave scans the runs' totals, then every lane
// writes its sequences' offsets and list entries.
__device__ void build_plan(const PlanArgs& p, int l) {
  const int per = (p.batch + 63) / 64;
  const int b0 = min(p.batch, l * per), b1 = min(p.batch, b0 + per);
  auto splits = [&](int b, int* kv_out) __attribute__((always_inline)) {
    const int kv = min(max(p.kv_lens[b], 0), p.max_kv_len);
    *kv_out = kv;
    const int chunk = kv < p.precise_below ? p.chunk_precise : p.chunk_fast;
    return kv >= p.n_q ? (kv + chunk - 1) / chunk : 0;
  };
  int tot = 0, nf = 0, np = 0;
  for (int b = b0; b < b1; ++b) {
    int kv;
    const int ns = splits(b, &kv);
    tot += ns;
    if (kv < p.precise_below) np += ns;
    else nf += ns;
  }
  // exclusive scans over the lanes
  int it = tot, ifa = nf, ipr = np;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t0 = __shfl_up(it, d), t1 = __shfl_up(ifa, d), t2 = __shfl_up(ipr, d);
    if (l >= d) {
      it += t0;
      ifa += t1;
      ipr += t2;
    }
  }
  int ot = it - tot, of = ifa - nf, op = ipr - np;
  for (int b = b0; b < b1; ++b) {
    int kv;
    int ns = splits(b, &kv);
    ns = max(0, min(ns, p.cap - ot));  // never past the partial buffers
    p.seq_off[b] = min(ot, p.cap);
    const bool prec = kv < p.precise_below;
    WorkItem* dst = prec ? p.precise + op : p.fast + of;
    for (int s = 0; s < ns; ++s) dst[s] = WorkItem{b, s, ot + s, kv};
    ot += ns;
    if (prec) op += ns;
    else of += ns;
  }
  if (l == 63) {
    p.seq_off[p.batch] = min(ot, p.cap);
    p.counts[0] = min(of, p.cap);
    p.counts[1] = min(op, p.cap);
  }
  // the rest of both lists, up to cap + kListPad, holds b = -1: a workgroup reads its
  // pair's entry and stops there, without waiting for the counts first
  const int nf_all = __shfl(of, 63), np_all = __shfl(op, 63);
  for (int k = nf_all + l; k < p.cap + kListPad; k += 64) p.fast[k] = WorkItem{-1, 0, 0, 0};
  for (int k = np_all + l; k < p.cap + kListPad; k += 64) p.precise[k] = WorkItem{-1, 0, 0, 0};
}

// grid (ceil(h / 4), 8), 8 waves: group g of 4 heads (4g .. 4g + 3), block nb of 64
// latent columns. No wave waits for another.
//
// Waves 0-3 (the product): wave w computes head 4g + w for those columns (two
// 32-column MFMA blocks) over every 32-row block of M, as Dᵀ = W_UK-block · q_nopeᵀ
// so each lane holds one query row and runs of 4 adjacent columns. q_nope rows are
// read whole (16 lanes per 256-byte row: a wave load touches 8 cache lines, where
// fragment-shaped loads touch 32) and become MFMA fragments through the wave's own
// LDS area, which then stages the result into 16-byte chunks of 8 columns. LDS
// operations of one wave execute in order, so the area needs no barrier. The chunks
// of the 4 heads at one (row, column chunk) are adjacent lanes of the block order
// above; the 4 waves' pieces of a line meet in the L2 of this workgroup's XCD.
//
// Waves 4-7 (side work, concurrent with the product's loads): rotate the q_R of
// query rows m = nb (mod 8) of these heads. The rotation angle depends on
// the row and the pair only: each half wave takes one row, lane k forms the sine and
// cosine of pair k once, and the 4 heads' chunks fetch them by lane shuffles. Wave 7
// of workgroup (0, 0) first builds the split plan.
constexpr int kQHeads = 4;
constexpr int kQColBlocks = 8;

__global__ __launch_bounds__(512) void qprep_kernel(QPrepArgs a) {
  constexpr int kQnB = 256 + 16;  // row of a wave's area (q_nope row, or 64 result columns hi + lo), padded
  __shared__ __attribute__((aligned(16))) char s_area[kQHeads][32 * kQnB];
  const int g = blockIdx.x, nb = blockIdx.y;
  const int tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int i0 = kQHeads * g;
  const int nh = min(kQHeads, a.h - i0);  // heads in this group
  const bool lo_out = a.q_lo != nullptr;
  // the low halves are read only by the precise form, which takes the sequences the
  // plan puts in its list (the same rule as build_plan), so only their rows get them
  auto precise_len = [&](int kv) __attribute__((always_inline)) {
    return min(max(kv, 0), a.max_kv_len) < a.plan.precise_below;
  };

  // query row m, head i -> offset of the block-order element (m, i, column 0)
  // (the column adds col_off(c))
  const int KS = (512 + a.d_r) / 16;
  const int HB = a.h / 32;
  auto row_off = [&](int m, int i) __attribute__((always_inline)) -> int64_t {
    return ((static_cast<int64_t>(m) * HB + (i >> 5)) * KS * 64 + (i & 31)) * 8;
  };
  auto col_off = [](int c) __attribute__((always_inline)) -> int { return ((c >> 4) * 64 + 32 * ((c >> 3) & 1)) * 8 + (c & 7); };

  if (w >= kQHeads) {
    // ================= side work: waves 4-7 =================
    const int sw = w - kQHeads;
    const int srows = a.M > nb ? (a.M - nb + kQColBlocks - 1) / kQColBlocks : 0;
    // RoPE of q_R: half wave hf of wave sw takes side row t = 8u + 2sw + hf (u = 0, 1, ..),
    // query row m = nb + 8t. Pair k (columns 2k, 2k + 1) turns by pos * inv_freq[k], the
    // angle formed and reduced modulo 2π in fp64, sine and cosine in fp32. Lane hl of
    // the half forms pair hl, then writes chunk hl / 4 (4 pairs) of head hl % 4.
    const int npair = a.d_r / 2, rchunks = a.d_r / 8;
    const int hf = l >> 5, hl = l & 31;
    const int hh = hl % kQHeads, ch = hl / kQHeads;
    // the loads of a wave's next row are issued before its current row is rotated
    auto side_loads = [&](int t_base, u32x4& x, int& kvl) __attribute__((always_inline)) {
      const int t = t_base + hf;
      const int m = nb + kQColBlocks * t;
      x = u32x4{0u, 0u, 0u, 0u};
      kvl = 0;
      if (t < srows && ch < rchunks && hh < nh)
        x = *reinterpret_cast<const u32x4*>(a.q_rope + (static_cast<int64_t>(m) * a.h + i0 + hh) * a.d_r + 8 * ch);
      if (t < srows) kvl = a.kv_lens[m / a.n_q];
    };
    u32x4 x_next;
    int kvl_next;
    if (a.d_r > 0 && 2 * sw < srows) side_loads(2 * sw, x_next, kvl_next);
    // the plan goes to the side wave with the fewest rotation rows (wave 7 takes rows
    // from t = 6 on, none when M <= 48), after its first row's loads are issued, so
    // no wave builds the plan and then waits on the loads of its rows
    if (g == 0 && nb == 0 && sw == kQHeads - 1) build_plan(a.plan, l);
    for (int t_base = 2 * sw; a.d_r > 0 && t_base < srows; t_base += 2 * kQHeads) {  // uniform
      const int t = t_base + hf;
      const bool row_ok = t < srows;
      const int m = nb + kQColBlocks * t;
      const bool item = row_ok && ch < rchunks && hh < nh;
      const u32x4 x = x_next;
      const int kvl = kvl_next;
      if (t_base + 2 * kQHeads < srows) side_loads(t_base + 2 * kQHeads, x_next, kvl_next);
      float cs = 1.f, sn = 0.f;
      if (row_ok && hl < npair) {
        const double pos = static_cast<double>(min(kvl, a.max_kv_len) - a.n_q + m % a.n_q);
        const double theta = pos * a.inv_freq[hl];
        const double red = theta - 6.283185307179586 * rint(theta * 0.15915494309189535);
        sincosf(static_cast<float>(red), &sn, &cs);
      }
      u32x4 o, ol;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int src = 32 * hf + ((4 * ch + p) & 31);  // every lane takes part
        const float c = __shfl(cs, src), sv = __shfl(sn, src);
        const float x0 = bf16_bits_to_f32(static_cast<uint16_t>(x[p] & 0xFFFFu));
        const float x1 = bf16_bits_to_f32(static_cast<uint16_t>(x[p] >> 16));
        const float y0 = (x0 * c - x1 * sv) * a.qscale, y1 = (x0 * sv + x1 * c) * a.qscale;
        o[p] = pack_bf16x2(y0, y1);
        ol[p] = pack_bf16x2(y0 - __uint_as_float(o[p] << 16), y1 - __uint_as_float(o[p] & 0xFFFF0000u));
      }
      if (item) {
        const int64_t off = row_off(m, i0 + hh) + col_off(512 + 8 * ch);
        *reinterpret_cast<u32x4*>(a.q_cat + off) = o;
        if (lo_out && precise_len(kvl)) *reinterpret_cast<u32x4*>(a.q_lo + off) = ol;
      }
    }
    return;
  }

  // ================= the product: waves 0-3, head hw =================
  const int hw = min(i0 + w, a.h - 1);  // past h: a discarded copy
  char* area = s_area[w];
  // q_nope rows 32mb .. +31 of head hw, whole rows: load i, lane l -> row 4i + l/16,
  // 16-byte chunk l%16 -> area[row][chunk]
  u32x4 rows[8];
  auto load_rows = [&](int mb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = 32 * mb + 4 * i + (l >> 4);
      rows[i] = m < a.M ? *reinterpret_cast<const u32x4*>(a.q_nope + (static_cast<int64_t>(m) * a.h + hw) * 128 + 8 * (l & 15))
                        : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // latent mode: the absorbed query is given; its columns 64nb .. 64nb + 63 of head hw
  // enter the staging below in the product's lane layout (row l%32, columns
  // 32cb + 8j + 4(l/32) .. + 3 in values 4j .. 4j + 3)
  const bool given = a.q_abs != nullptr;
  auto load_given = [&](int mb, f32x16* acc) __attribute__((always_inline)) {
    const int m = 32 * mb + (l & 31);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (m < a.M)
          v = *reinterpret_cast<const f32x4*>(a.q_abs + (static_cast<int64_t>(m) * a.h + hw) * 512 + 64 * nb +
                                              32 * cb + 8 * j + 4 * (l >> 5));
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[cb][4 * j + e] = v[e];
      }
  };
  // the first block's rows go out before the weights, so they land first and the
  // products can follow the weights as they arrive
  if (!given) load_rows(0);
  // W_UK fragments of head hw: column blocks 2nb, 2nb + 1, 8 k-steps each
  u32x4 bfr[2][8];
  if (!given) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const u32x4* wk = reinterpret_cast<const u32x4*>(a.w_uk_pk) + ((static_cast<int64_t>(hw) * 16 + 2 * nb + cb) * 8) * 64 + l;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) bfr[cb][ks] = wk[ks * 64];
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // every weight load issued before the rows' wait
  for (int mb = 0; mb * 32 < a.M; ++mb) {
    // lengths of the sequences of this lane's stored rows, loaded ahead of the
    // products (they decide which rows get low halves)
    int kv_row[4] = {0, 0, 0, 0};
    if (lo_out) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int m = 32 * mb + (l >> 3) + 8 * k;
        if (m < a.M) kv_row[k] = a.kv_lens[m / a.n_q];
      }
    }
    f32x16 acc[2];
    if (given) {
      load_given(mb, acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) *(lds_u32x4*)(lds_ptr(area) + (4 * i + (l >> 4)) * kQnB + (l & 15) * 16) = rows[i];
      // B fragment k-step ks: row l%32, k = 16ks + 8(l/32) + e
      u32x4 af[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) af[ks] = *(lds_u32x4*)(lds_ptr(area) + (l & 31) * kQnB + (2 * ks + (l >> 5)) * 16);
      // the next block's rows are in flight during this block's products and stores
      if ((mb + 1) * 32 < a.M) load_rows(mb + 1);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        acc[cb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(bfr[cb][ks]), as_bf16x8(af[ks]), acc[cb], 0, 0, 0);
      }
    }
    // stage in the area (its fragments are in registers): lane l holds row l%32 and
    // columns 32cb + 8j + 4(l/32) + 0..3 in values 4j .. 4j+3; the high halves take
    // bytes 0..127 of the row, the low halves (precise mode) bytes 128..255
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16& o = acc[cb];
        const float x0 = o[4 * j] * a.qscale, x1 = o[4 * j + 1] * a.qscale;
        const float x2 = o[4 * j + 2] * a.qscale, x3 = o[4 * j + 3] * a.qscale;
        const u32x2 v = {pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
        const int boff = (l & 31) * kQnB + (32 * cb + 8 * j + 4 * (l >> 5)) * 2;
        *(lds_u32x2*)(lds_ptr(area) + boff) = v;
        if (lo_out) {
          const u32x2 vl = {pack_bf16x2(x0 - __uint_as_float(v[0] << 16), x1 - __uint_as_float(v[0] & 0xFFFF0000u)),
                            pack_bf16x2(x2 - __uint_as_float(v[1] << 16), x3 - __uint_as_float(v[1] & 0xFFFF0000u))};
          *(lds_u32x2*)(lds_ptr(area) + boff + 128) = vl;
        }
      }
    // 32 rows x 8 chunks of 8 columns: chunk q = l + 64k -> row q/8, column chunk q%8
    const int cc = l & 7;
    const int64_t coff = col_off(64 * nb + 8 * cc);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = (l >> 3) + 8 * k, m = 32 * mb + r;
      const u32x4 v = *(lds_u32x4*)(lds_ptr(area) + r * kQnB + cc * 16);
      if (m < a.M && w < nh) *reinterpret_cast<u32x4*>(a.q_cat + row_off(m, hw) + coff) = v;
      if (lo_out && m < a.M && w < nh && precise_len(kv_row[k])) {
        const u32x4 vl = *(lds_u32x4*)(lds_ptr(area) + r * kQnB + 128 + cc * 16);
        *reinterpret_cast<u32x4*>(a.q_lo + row_off(m, hw) + coff) = vl;
      }
    }
  }
}

hipError_t launch_qprep_bf16(const QPrepArgs& a, hipStream_t s) {
  if (a.d_r % 8 != 0 || a.d_r > 64 || a.h % 32 != 0) return hipErrorInvalidValue;  // whole 16-byte q_R chunks
  qprep_kernel<<<dim3((a.h + kQHeads - 1) / kQHeads, kQColBlocks), 512, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
