// Split-K flash-decode over the bf16 latent cache (the hot loop of absorbed MLA).
//
// For one sequence b, one token range [t_begin, t_end) and R = 32*NW query rows
// (pairs (query j, head i) that share the sequence's latent cache), each 32-token
// tile of cache rows [c_KV ‖ k_R] is staged HBM -> LDS once and used by every row:
//
//   Sᵀ[t][r] = Σ_k C[t][k] · Q_cat[r][k]              (scores; MLA tutorial page §3.1:
//                                                      q·kᵀ = (q·W_UKᵀ)·c_KVᵀ, plus the
//                                                      decoupled RoPE term)
//   online softmax over t with the running max subtracted (interview guide §7.3)
//   Oᵀ[c][r] += Σ_t C[t][c] · P[r][t]                  (latent-space sum, tutorial
//                                                      §3.1: attn·v = (attn·c_KV)·W_UV)
//
// Both contractions run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation. The
// 128 heads sharing one latent make them dense: each bf16 cache element loaded
// from HBM feeds 2*R multiply-adds.
//
// Work split inside a workgroup (one wave per SIMD): for the scores and the
// softmax, wave w owns query rows 32w .. 32w+31 (their Q_cat fragments stay in
// VGPRs, their softmax state in lanes). For the value contraction it owns latent
// columns 32*CBW*w .. +32*CBW of every row (Oᵀ accumulators, 16 blocks of 32x32
// fp32 = 256 registers per lane, in AGPRs), so each cache element is transposed
// out of LDS once per workgroup rather than once per wave. P travels between the
// two through LDS, written in the B-operand order of the value MFMA: the value
// MFMA takes the tile's 32 tokens in the order the score MFMA leaves them in its
// accumulator.
//
// Pipelining: a workgroup (one per CU) keeps four tile buffers. Step i runs tile
// i's scores and softmax together with tile i - 1's value MFMAs, with tile i + 1
// in flight and tile i + 2 issued at its start; P is double-buffered by tile
// parity, so each step needs one barrier. Query rows that do not come in 128s
// take the role-split 64-row form further down.
//
// LDS tile layout: the 576 (or 512) columns are cut into groups of 64 (128 bytes,
// eight 16-byte chunks); group G holds all 32 rows, row t at G*4096 + t*128, and
// chunk k of the group at position k ^ swz(t), swz(t) = ((u & 1) << 2) | (u >> 1)
// with u = (t >> 1) & 7. The 16-row column reads of the score operand and the
// 4-row transposed reads of the value operand are then free of bank conflicts,
// and each 1 KiB wave load (8 rows x one group) has a per-lane offset that takes
// only two values.
//
// Softmax state is kept in base-2 units (Q_cat carries scale * log2 e). Each row's
// reference max is fixed at the first tile where the row sees a token, so the
// accumulators never need rescaling: later P values may exceed 1, which is exact
// in floating point as long as they stay in range. If a score ever exceeds the
// reference by more than 64 (P > 2^64), the wave flags it; the waves exchange
// their flags through LDS once after the range, and if any is set the workgroup
// drains its loads and restarts the range with the largest score seen as every
// row's reference (at most 8 times). The decision is workgroup-uniform, so every
// wave takes the same barriers.
//
// Output per (b, split): the normalised partial O/l as bf16 rows of 512 (written
// coalesced through LDS) and (m, l) in fp32; the combine kernel merges splits.
#include "common.hpp"
#include "launch.hpp"
#include <hip/hip_ext.h>

namespace mla {

namespace {

constexpr int kTileT = 32;    // tokens per tile
constexpr float kHeadroom = 64.0f;  // largest score - reference allowed (base-2 units)
constexpr int kMaxRestarts = 8;

__device__ __forceinline__ int swz(int t) {
  const int u = (t >> 1) & 7;
  return ((u & 1) << 2) | (u >> 1);
}

template <int NW, int DR>
struct Cfg {
  static constexpr int NBUF = 4;                           // tile buffers
  static constexpr int ROW = 512 + DR;                     // elements per cache row
  static constexpr int ROWB = ROW * 2;                     // bytes per cache row
  static constexpr int CH = ROW / 8;                       // 16-byte chunks per row
  static constexpr int KS = ROW / 16;                      // score k-steps (K=16 each)
  static constexpr int R = 32 * NW;                        // query rows per workgroup
  static constexpr int TILE_BYTES = kTileT * ROWB;
  static constexpr int LOADS = (kTileT * CH) / (64 * NW);  // 16-B loads per lane per tile
  static constexpr int CBW = 16 / NW;                      // value column blocks per wave
  static constexpr int RB = NW;                            // row blocks of 32 query rows
  static_assert((kTileT * CH) % (64 * NW) == 0, "tile loads per wave");
  static_assert(32 * CBW * R * 2 <= TILE_BYTES, "epilogue staging fits a tile buffer");
};

template <int V>
struct Ic {
  static constexpr int value = V;
};

// Score MFMA in VGPR form: Sᵀ += A · B with the accumulator in VGPRs. (The
// compiler selects the AGPR form for every builtin MFMA of this kernel, whose AGPRs
// hold the value accumulators.) The leading s_nop gives the 2 wait states a VALU
// write of an operand needs before an MFMA reads it; back-to-back accumulation into
// the same registers needs none.
__device__ __forceinline__ void mfma_v(f32x16& c, const u32x4& a, const u32x4& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// Last MFMA of a chain: also waits out the 8-pass result latency (> 11 wait states)
// before any VALU instruction may read or write the accumulator.
__device__ __forceinline__ void mfma_v_last(f32x16& c, const u32x4& a, const u32x4& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 4"
      : "+v"(c) : "v"(a), "v"(b));
}

}  // namespace

template <int NW, int DR>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  using C = Cfg<NW, DR>;
  constexpr int NBUF = C::NBUF, CBW = C::CBW, RB = C::RB;
  // Tile buffers as distinct arrays: reads of one are provably independent of the
  // direct-to-LDS loads landing in another, so they need no load wait.
  __shared__ __attribute__((aligned(1024))) char s_tile0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char s_tile1[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char s_tile2[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char s_tile3[C::TILE_BYTES];
  // P fragments [parity][row block][k-step][lane]: P of tile i goes into buffer i % 2,
  // so publishing it never waits for readers of tile i - 1's P. After the last step's
  // barrier, the buffer the last tile did not use holds 1 / l per row.
  constexpr int PBUF = RB * 2 * 1024;
  __shared__ __attribute__((aligned(16))) char s_p[2 * PBUF];
  static_assert(4 * C::TILE_BYTES + 2 * PBUF <= 160 * 1024, "LDS");
  static_assert(16 + 4 * C::R <= PBUF, "1 / l fits a P buffer");

  const int tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);  // wave index, uniform
  const int hgroups = (a.h * a.n_q) / C::R;
  const int units = a.batch * a.n_splits * hgroups;

  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous
  // range of units so one sequence's splits (and head groups) share an L2.
  int u = blockIdx.x;
  if ((units & 7) == 0) u = (blockIdx.x & 7) * (units >> 3) + (blockIdx.x >> 3);
  const int hg = u % hgroups;
  const int s = (u / hgroups) % a.n_splits;
  const int b = u / (hgroups * a.n_splits);

  const int kv = min(a.kv_lens[b], a.max_kv_len);
  const int t_begin = s * a.chunk;
  const int t_end = min(t_begin + a.chunk, kv);
  if (t_begin >= t_end || kv < a.n_q) return;  // empty split: the combine skips it
  const int n_tiles = (t_end - t_begin + kTileT - 1) / kTileT;

  const int HG = C::R / a.n_q;  // heads per workgroup
  // this lane's score row r = 32w + l%32 (lanes l and l^32 hold the same row)
  const int r_own = 32 * w + (l & 31);
  const int j_own = r_own / HG;
  const int head_own = hg * HG + r_own % HG;
  const int vis_own = kv - a.n_q + j_own;  // last visible position of this row

  // ---- tile loads: wave load n' = n*NW + w fills LDS [n'*1024, +1024) = column
  //      group G = n'/4, rows 8(n'%4) + l/8, chunk position l%8. Its source is
  //      row t = 8(n'%4) + l/8, logical chunk 8G + ((l%8) ^ swz(t)); swz(t) only
  //      depends on n'%2 and l, so the per-lane part of the offset takes two values.
  uint32_t ld_lane[2];
#pragma unroll
  for (int odd = 0; odd < 2; ++odd) {
    const int t = 8 * odd + (l >> 3);
    ld_lane[odd] = static_cast<uint32_t>(t * C::ROWB + (((l & 7) ^ swz(t)) << 4));
  }

  const char* cache = static_cast<const char*>(a.cache.data);
  const bool paged = a.cache.block_table != nullptr;
  // physical block of tile `it` (paged cache); out-of-range entries read block 0.
  // The table is read-only here: reading it through the constant address space
  // makes the uniform lookup a scalar load, which does not wait on tile loads.
  const __attribute__((address_space(4))) int32_t* table =
      (const __attribute__((address_space(4))) int32_t*)(a.cache.block_table);
  auto page_id = [&](int it) __attribute__((always_inline)) -> int {
    const int blk = (t_begin + it * kTileT) / a.cache.block_size;
    const int id = table[static_cast<int64_t>(b) * a.cache.max_blocks + blk];
    return (id < 0 || id >= a.cache.n_blocks) ? 0 : id;
  };
  int pg_next = paged ? page_id(0) : 0;  // block of the next tile to issue, read one issue ahead

  // Buffer resource of tile `it`: base at the tile's first row, size bound covering
  // only the tile's rows inside the range, so loads of rows past the range end return
  // zeros (those tokens are masked). A 32-token tile never straddles a block (ranges
  // start at multiples of 32, blocks hold multiples of 32 tokens). Tiles are taken in
  // order, so the block of tile it + 1 is fetched here, one tile ahead.
  auto tile_rsrc = [&](int it) __attribute__((always_inline)) -> u32x4 {
    const int t0 = t_begin + it * kTileT;
    const char* base;
    if (!paged) {
      base = cache + (static_cast<int64_t>(b) * a.cache.t_max + t0) * C::ROWB;
    } else {
      base = cache + (static_cast<int64_t>(pg_next) * a.cache.block_size + t0 % a.cache.block_size) * C::ROWB;
      if (it + 1 < n_tiles) pg_next = page_id(it + 1);
    }
    const uint64_t ba = reinterpret_cast<uint64_t>(base);
    const uint32_t rows = static_cast<uint32_t>(min(kTileT, t_end - t0));
    return u32x4{static_cast<uint32_t>(ba), static_cast<uint32_t>(ba >> 32) & 0xFFFFu,
                 rows * static_cast<uint32_t>(C::ROWB), 0x00020000u};
  };
  // Load n of this wave's share of a tile: wave load n' = n*NW + w fills LDS
  // [n'*1024, +1024) from column group n'/4, rows 8(n'%4) .. +7; the whole byte
  // offset is per lane (soffset 0) so the size bound applies to all of it.
  auto issue_load = [&](const u32x4& rsrc, char* tile, int n) __attribute__((always_inline)) {
    const int np = n * NW + w;  // wave-uniform
    const int G = np >> 2, rq = np & 3;
    dma_b128(rsrc, ld_lane[rq & 1], static_cast<uint32_t>(G * 128 + (rq >> 1) * 16 * C::ROWB),
             static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_ptr(tile) + np * 1024)));
  };
  auto issue_tile = [&](int it, char* tile) __attribute__((always_inline)) {
    const u32x4 rsrc = tile_rsrc(it);
#pragma unroll
    for (int n = 0; n < C::LOADS; ++n) issue_load(rsrc, tile, n);
  };

  // ---- per-lane LDS read offsets
  // score A operand: row t = l%32, logical chunk k = 2ks + l/32: group ks/4,
  // position (2(ks%4) + l/32) ^ swz(t)
  int sa_off[4];
  {
    const int t = l & 31, sw = swz(t);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) sa_off[kk] = t * 128 + (((2 * kk + (l >> 5)) ^ sw) << 4);
  }
  // value A operand (transposed reads). K index 8h + e (h = l/32) of value k-step
  // kk stands for token 16kk + 4h + (e%4) + 8(e/4): the tokens the score
  // accumulator holds in lane l's values 8kk .. 8kk+7. 16-lane group g, lane i
  // reads rows 4(g/2) + i/4 (+8) and columns 16(g%2) + 4(i%4) of a 32-column
  // block, i.e. chunk 4(blk%2) + 2(g%2) + (i%4)/2 of group blk/2, half (i%2).
  int va_off[2][2];
  {
    const int g = l >> 4, i = l & 15;
#pragma unroll
    for (int sec = 0; sec < 2; ++sec) {
      const int t = 4 * (g >> 1) + (i >> 2) + 8 * sec;
      const int sw = swz(t);
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const int low = 2 * (g & 1) + ((i & 3) >> 1);  // chunk within the 4-chunk half group
        va_off[sec][par] = t * 128 + (((4 * par + low) ^ sw) << 4) + ((i & 1) << 3);
      }
    }
  }

  u32x4 qf[C::KS];  // this row's Q_cat fragments (loaded below)

  // Oᵀ accumulators: column block CBW*w + cbl (32 latent columns) x row block rb
  // (32 query rows), acc[cbl * RB + rb]
  f32x16 acc[CBW * RB];
  float m_ref = -INFINITY;   // this row's fixed reference max
  float m_seen = -INFINITY;  // largest score this row has seen
  float l_run = 0.f;

  // ---- scores: Sᵀ[32 tokens][32 rows of this wave], SDEPTH fragments in flight
  constexpr int SDEPTH = 6;
  auto scores = [&](const char* tile, auto hook) __attribute__((always_inline)) {
    f32x16 sc = {};
    u32x4 fa[SDEPTH];
    // k-step ks: column group ks/4, chunk pair ks%4
    auto frag = [&](int ks) __attribute__((always_inline)) {
      return *(lds_u32x4*)(lds_ptr(tile) + sa_off[ks & 3] + (ks >> 2) * 4096);
    };
#pragma unroll
    for (int ks = 0; ks < SDEPTH; ++ks) fa[ks] = frag(ks);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      if (ks + 1 < C::KS) mfma_v(sc, fa[ks % SDEPTH], qf[ks]);
      else mfma_v_last(sc, fa[ks % SDEPTH], qf[ks]);
      hook(ks);
      if (ks + SDEPTH < C::KS) fa[ks % SDEPTH] = frag(ks + SDEPTH);
    }
    return sc;
  };

  // ---- softmax of a tile for row r_own against the fixed reference: P as 8 packed
  //      bf16 pairs (values 2k, 2k+1 of the score accumulator) and whether a score
  //      overran the reference by more than the headroom. Written as 26 short
  //      micro-steps (max and reference, one probability each, row sum).
  struct Soft {
    u32x4 p[2];
    bool overrun;
  };
  struct SoftState {
    float mxa[5], t0, t1, mx, mref, pa;
    float ps[4];
    Soft r;
  };
  // tokens a row must not see (past the range end or its causal limit) score -inf
  auto apply_mask = [&](f32x16& sc, int it) __attribute__((always_inline)) {
    const int t0 = t_begin + it * kTileT;
    const int lim = min(t_end - 1, vis_own);  // last token this row may see
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int tok = t0 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
      sc[v] = tok > lim ? -INFINITY : sc[v];
    }
  };
  // micro-steps: 0..8 row max and reference, 9..24 one probability each (a pair is
  // packed as soon as its second value exists), 25 the row sum
  constexpr int kSoftSteps = 26;
  auto soft_step = [&](int k, const f32x16& sc, SoftState& st, bool allow_restart) __attribute__((always_inline)) {
    if (k < 5) {
      st.mxa[k] = fmaxf(fmaxf(sc[3 * k], sc[3 * k + 1]), sc[3 * k + 2]);
    } else if (k == 5) {
      st.t0 = fmaxf(fmaxf(st.mxa[0], st.mxa[1]), sc[15]);
    } else if (k == 6) {
      st.t1 = fmaxf(fmaxf(st.mxa[2], st.mxa[3]), st.mxa[4]);
    } else if (k == 7) {
      st.mx = half_max(fmaxf(st.t0, st.t1));
    } else if (k == 8) {
      m_seen = fmaxf(m_seen, st.mx);
      // first visible tile of the row: nothing accumulated yet, so set the reference
      if (m_ref == -INFINITY) m_ref = st.mx;
      st.r.overrun = allow_restart && st.mx > m_ref + kHeadroom;
      st.mref = m_ref == -INFINITY ? 0.f : m_ref;
    } else if (k < 25) {
      const int v = k - 9, q = v >> 1;
      const float pv = fast_exp2(sc[v] - st.mref);
      if ((v & 1) == 0) {
        st.pa = pv;
      } else {
        st.r.p[q >> 2][q & 3] = pack_bf16x2(st.pa, pv);
        st.ps[q & 3] = (q < 4 ? 0.f : st.ps[q & 3]) + (st.pa + pv);
      }
    } else {
      l_run += half_sum((st.ps[0] + st.ps[1]) + (st.ps[2] + st.ps[3]));
    }
  };

  // ---- values for this wave's CBW column blocks and every row block:
  //      Oᵀ[c][r] += Σ_t Cᵀ[c][t] · Pᵀ[t][r]; P of all rows comes from LDS one
  //      k-step at a time, the 2*CBW transposed cache fragments stream through a
  //      four-deep window
  // `mstep(j)` runs after value MFMA j (of 2*CBW*RB); with `pinned`, each MFMA and
  // its mstep stay together in issue order (VALU work issued while the MFMA runs)
  auto pv = [&](const char* tile, const char* pbuf, auto hook, auto mstep, auto pinned) __attribute__((always_inline)) {
    auto load = [&](int f) __attribute__((always_inline)) {
      const int kk = f / CBW, cb = CBW * w + f % CBW;
      lds_char* tb = lds_ptr(tile) + kk * 16 * 128 + (cb >> 1) * 4096;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tb + va_off[0][cb & 1]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tb + va_off[1][cb & 1]));
      const i16x8 af = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return af;
    };
    constexpr int NF = 2 * CBW;
    constexpr int WIN = NF < 4 ? NF : 4;
    i16x8 frag[WIN];
#pragma unroll
    for (int f = 0; f < WIN; ++f) frag[f] = load(f);
    u32x4 pb[RB];  // P fragments of the current k-step, one per row block
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int kk = f / CBW, cbl = f % CBW;
      if (cbl == 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) pb[rb] = *(lds_u32x4*)(lds_ptr(pbuf) + (rb * 2 + kk) * 1024 + l * 16);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        acc[cbl * RB + rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, frag[f % WIN]), as_bf16x8(pb[rb]), acc[cbl * RB + rb], 0, 0, 0);
        if (rb == RB - 1 && f + WIN < NF) frag[f % WIN] = load(f + WIN);  // after its last use
        if (rb == 0) hook(f);
        mstep(f * RB + rb);
        if constexpr (decltype(pinned)::value != 0) __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  auto tile_ptr = [&](auto kc) __attribute__((always_inline)) -> char* {
    constexpr int K = decltype(kc)::value;
    if constexpr (K == 0) return s_tile0;
    else if constexpr (K == 1) return s_tile1;
    else if constexpr (K == 2) return s_tile2;
    else return s_tile3;
  };

  // Tiles from `first_masked` on hold tokens some row must not see (past the end of
  // the range, or past a row's causal limit); the tiles before it need no mask.
  const int bound = min(t_end - 1, kv - a.n_q);
  const int first_masked = bound - t_begin - (kTileT - 1) >= 0 ? (bound - t_begin - (kTileT - 1)) / kTileT + 1 : 0;

  // Wait until at most `ahead` tiles (ahead = 0, 1, 2) of this wave's loads are in flight.
  auto wait_tiles = [&](int ahead) __attribute__((always_inline)) {
    if (ahead >= 2) wait_vm<2 * C::LOADS>();
    else if (ahead == 1) wait_vm<C::LOADS>();
    else wait_vm<0>();
  };

  // Four tile buffers, pipelined on the value side. Step i computes tile i's scores,
  // then runs tile i's softmax interleaved with the value MFMAs of tile i - 1 (whose P
  // was published at the end of step i - 1), and publishes P of tile i into the other
  // P buffer. One barrier per step: tiles i and i - 1 are in use, tile i + 1 is in
  // flight, tile i + 2 goes into the buffer of tile i - 2, and P of tile i - 2 (the
  // buffer P of tile i overwrites) was last read in step i - 1. `first` is step 0,
  // which has no previous tile. A score past the headroom only marks the wave's
  // `ovr`; the range is restarted after it (the flags are exchanged once there).
  uint64_t ovr = 0;
  auto vstep = [&](auto kc, auto first, int i, bool allow_restart) __attribute__((always_inline)) {
    constexpr int K = decltype(kc)::value;
    constexpr bool FIRST = decltype(first)::value != 0;
    wait_tiles(i + 1 < n_tiles ? 1 : 0);  // tile i has landed
    lds_barrier();  // tile i and P of tile i - 1 everywhere; tile i - 2 is free
    // tile i + 2 into the buffer of tile i - 2, as one burst ahead of the score
    // chain: measured cheaper than loads spread through the MFMAs, and far cheaper
    // than loads among the value phase's transposed LDS reads
    if (i + 2 < n_tiles) {
      char* nxt = tile_ptr(Ic<(K + 2) % 4>{});
      const u32x4 rs = tile_rsrc(i + 2);
#pragma unroll
      for (int n = 0; n < C::LOADS; ++n) issue_load(rs, nxt, n);
    }
    f32x16 sc = scores(tile_ptr(kc), [](int) {});
    if (i >= first_masked) apply_mask(sc, i);  // uniform
    SoftState st;
    if constexpr (FIRST) {
#pragma unroll
      for (int k = 0; k < kSoftSteps; ++k) soft_step(k, sc, st, allow_restart);
    } else {
      pv(tile_ptr(Ic<(K + 3) % 4>{}), s_p + ((K + 1) & 1) * PBUF, [](int) {}, [&](int j) __attribute__((always_inline)) {
        if (j < kSoftSteps) soft_step(j, sc, st, allow_restart);
      }, Ic<1>{});
    }
    ovr |= __builtin_amdgcn_ballot_w64(st.r.overrun);
    *(lds_u32x4*)(lds_ptr(s_p + (K & 1) * PBUF) + (w * 2 + 0) * 1024 + l * 16) = st.r.p[0];
    *(lds_u32x4*)(lds_ptr(s_p + (K & 1) * PBUF) + (w * 2 + 1) * 1024 + l * 16) = st.r.p[1];
  };


  auto prologue = [&]() __attribute__((always_inline)) {
    if (paged) pg_next = page_id(0);
    constexpr int AHEAD = 2;  // tiles issued before the first step
#pragma unroll
    for (int k = 0; k < AHEAD; ++k)
      if (k < n_tiles) issue_tile(k, k == 0 ? s_tile0 : s_tile1);
  };
  prologue();

  // ---- Q_cat fragments (B operand of the score MFMA): k = 16ks + 8(l/32) + e,
  //      loaded while the first tiles are in flight; the wait covers both, so no
  //      later wait for these loads lands inside the tile loop
  {
    // Q_cat is stored in this kernel's fragment order: one 1 KiB wave load per k-step
    const u32x4* qp = reinterpret_cast<const u32x4*>(a.q_cat) +
                      ((static_cast<int64_t>(b) * hgroups + hg) * NW + w) * C::KS * 64 + l;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = qp[ks * 64];
  }
  wait_vm<0>();

  for (int pass = 0;; ++pass) {
    const bool allow_restart = pass < kMaxRestarts;  // the last pass keeps every score
#pragma unroll
    for (int k = 0; k < CBW * RB; ++k) acc[k] = f32x16{};
    l_run = 0.f;
    ovr = 0;
    if (pass > 0) prologue();
    vstep(Ic<0>{}, Ic<1>{}, 0, allow_restart);
    for (int i = 1; i < n_tiles; i += 4) {
#define MLA_VSTEP(KK, D) \
  if (i + D < n_tiles) vstep(Ic<KK>{}, Ic<0>{}, i + D, allow_restart);
      MLA_VSTEP(1, 0)
      MLA_VSTEP(2, 1)
      MLA_VSTEP(3, 2)
      MLA_VSTEP(0, 3)
#undef MLA_VSTEP
    }
    // restart flags, in tile buffer (n_tiles + 1) % 4: its tile (n_tiles - 3) was last
    // read in step n_tiles - 2, which every wave has left, or it was never used; no
    // load targets it. (The P buffers may still be read by a slower wave's last step.)
    const int kf = (n_tiles + 1) & 3;
    int* s_flag = reinterpret_cast<int*>(kf == 0 ? s_tile0 : kf == 1 ? s_tile1 : kf == 2 ? s_tile2 : s_tile3);
    if (l == 0) s_flag[w] = ovr != 0;
    lds_barrier();  // P of the last tile and every wave's flag
    bool restart = false;
#pragma unroll
    for (int k = 0; k < NW; ++k) restart |= s_flag[k] != 0;  // uniform
    if (!restart) {
      // the value MFMAs of the last tile, from buffer (n_tiles - 1) % 4 (one copy of
      // the code: a branch per buffer would split the accumulators' registers)
      const int kl = (n_tiles - 1) & 3;
      const char* lt = kl == 0 ? s_tile0 : kl == 1 ? s_tile1 : kl == 2 ? s_tile2 : s_tile3;
      pv(lt, s_p + ((n_tiles - 1) & 1) * PBUF, [](int) {}, [](int) {}, Ic<0>{});
      break;
    }
    // restart the range with the largest score seen as every row's reference; the
    // barrier orders every wave's flag reads before the next pass writes P
    wait_vm<0>();
    lds_barrier();
    m_ref = m_seen;
  }

  // ---- epilogue: normalised partial O/l as bf16 rows. 1/l of each row comes from
  //      its score wave; each wave stages its 32*CBW columns of all R rows in its
  //      own tile buffer ([R rows][4*CBW chunks], chunk ^ (row & 15)) and writes
  //      them out as contiguous row segments.
  // 1 / l per row, in the P buffer the last tile did not use (free since the barrier
  // after the last step; the staging below starts after the next barrier)
  float* s_inv = reinterpret_cast<float*>(s_p + (n_tiles & 1) * PBUF + 16);
  if (l < 32) s_inv[r_own] = l_run > 0.f ? 1.f / l_run : 0.f;
  lds_barrier();  // every wave is past the last tile; s_inv complete
  constexpr int CPR = 4 * CBW;  // 16-byte chunks per staged row
  constexpr int RSB = 16 * CPR;  // staged row bytes
  char* stg = w == 0 ? s_tile0 : w == 1 ? s_tile1 : w == 2 ? s_tile2 : s_tile3;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = 32 * rb + (l & 31);
    const float inv = s_inv[row];
#pragma unroll
    for (int cbl = 0; cbl < CBW; ++cbl)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const f32x16& o = acc[cbl * RB + rb];
        const int chunk = (4 * cbl + v4) ^ (row & 15);
        const u32x2 v2 = {pack_bf16x2(o[4 * v4] * inv, o[4 * v4 + 1] * inv),
                          pack_bf16x2(o[4 * v4 + 2] * inv, o[4 * v4 + 3] * inv)};
        *(lds_u32x2*)(lds_ptr(stg) + row * RSB + chunk * 16 + (l >> 5) * 8) = v2;
      }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging writes are done
  __builtin_amdgcn_wave_barrier();
  const int64_t part_row0 = (static_cast<int64_t>(b) * a.n_splits + s) * a.n_q;
  constexpr int RPI = 64 / CPR;  // rows per wave instruction
#pragma unroll 4
  for (int q = 0; q < C::R / RPI; ++q) {
    const int row = RPI * q + l / CPR, ch = l % CPR;
    const int j = row / HG, head = hg * HG + row % HG;
    const u32x4 v = *(lds_u32x4*)(lds_ptr(stg) + row * RSB + ((ch ^ (row & 15)) << 4));
    *reinterpret_cast<u32x4*>(a.o_part + ((part_row0 + j) * a.h + head) * 512 + 32 * CBW * w + ch * 8) = v;
  }
  if (l < 32) {
    float* ml = a.ml_part + ((part_row0 + j_own) * a.h + head_own) * 2;
    ml[0] = m_ref;
    ml[1] = l_run;
  }
}

// Role-split form for 64 query rows per workgroup (a (sequence, token range, head
// group) unit of 64 rows). Waves 0-1 own the scores and the softmax of rows
// 32w .. 32w + 31 (their Q_cat fragments in VGPRs, the same fragment order as the
// 64-row workgroups above). Waves 2-3 own the value contraction for latent columns
// 256 v .. 256 v + 255 (v = w - 2) of all 64 rows (Oᵀ: 16 blocks of 32x32 fp32 in
// AGPRs) and issue every tile load. Both pairs run about 1.1k MFMA cycles per tile,
// so the matrix cores of all four SIMDs stay busy, while a unit holds half the rows
// of the 128-row form: a sequence needs half as many token ranges for the same
// number of workgroups, which halves the split partials the combine reads back.
//
// Step i (one barrier): the value waves wait for their share of tile i, everyone
// passes the barrier; the value waves issue tile i + 2 into the buffer of tile
// i - 2 and run the value MFMAs of tile i - 1 (P from buffer (i - 1) % 2); the score
// waves run tile i's score chain and softmax and publish P into buffer i % 2. P
// buffer i % 2 held tile i - 2's P, which the value waves finished reading in step
// i - 1. Restarts, masking and the output are as in the 128-row form.
template <int DR>
__global__ __launch_bounds__(256) void decode_roles_kernel(DecodeArgs a) {
  constexpr int ROW = 512 + DR, ROWB = ROW * 2, CH = ROW / 8, KS = ROW / 16;
  constexpr int R = 64;                           // query rows per workgroup
  constexpr int TILE_BYTES = kTileT * ROWB;
  constexpr int LOADS = (kTileT * CH) / 128;      // 16-byte loads per value-wave lane per tile
  constexpr int CBW = 8;                          // value column blocks per value wave
  constexpr int RB = 2;                           // row blocks of 32 query rows
  static_assert((kTileT * CH) % 128 == 0, "tile loads per value wave");
  static_assert(R * 256 * 2 <= TILE_BYTES, "a value wave's staged rows fit a tile buffer");
  __shared__ __attribute__((aligned(1024))) char s_tile0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char s_tile1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char s_tile2[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char s_tile3[TILE_BYTES];
  constexpr int PBUF = RB * 2 * 1024;  // P fragments [row block][k-step][lane]
  __shared__ __attribute__((aligned(16))) char s_p[2 * PBUF];
  static_assert(4 * TILE_BYTES + 2 * PBUF <= 160 * 1024, "LDS");
  static_assert(16 + 4 * R <= PBUF, "1 / l fits a P buffer");

  const int tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);  // wave index, uniform
  const bool scorer = w < 2;
  const int vw = w - 2;  // value wave index (value waves only)
  const int hgroups = (a.h * a.n_q) / R;
  const int units = a.batch * a.n_splits * hgroups;
  int u = blockIdx.x;
  if ((units & 7) == 0) u = (blockIdx.x & 7) * (units >> 3) + (blockIdx.x >> 3);
  const int hg = u % hgroups;
  const int s = (u / hgroups) % a.n_splits;
  const int b = u / (hgroups * a.n_splits);

  const int kv = min(a.kv_lens[b], a.max_kv_len);
  const int t_begin = s * a.chunk;
  const int t_end = min(t_begin + a.chunk, kv);
  if (t_begin >= t_end || kv < a.n_q) return;  // empty split: the combine skips it
  const int n_tiles = (t_end - t_begin + kTileT - 1) / kTileT;

  const int HG = R / a.n_q;  // heads per workgroup
  const int r_own = 32 * (w & 1) + (l & 31);  // score waves: this lane's row
  const int j_own = r_own / HG;
  const int head_own = hg * HG + r_own % HG;
  const int vis_own = kv - a.n_q + j_own;

  // ---- tile loads (value waves): wave load n' = 2n + v fills LDS [n'*1024, +1024) =
  //      column group n'/4, rows 8(n'%4) + l/8, chunk position l%8
  uint32_t ld_lane[2];
#pragma unroll
  for (int odd = 0; odd < 2; ++odd) {
    const int t = 8 * odd + (l >> 3);
    ld_lane[odd] = static_cast<uint32_t>(t * ROWB + (((l & 7) ^ swz(t)) << 4));
  }
  const char* cache = static_cast<const char*>(a.cache.data);
  const bool paged = a.cache.block_table != nullptr;
  const __attribute__((address_space(4))) int32_t* table =
      (const __attribute__((address_space(4))) int32_t*)(a.cache.block_table);
  auto page_id = [&](int it) __attribute__((always_inline)) -> int {
    const int blk = (t_begin + it * kTileT) / a.cache.block_size;
    const int id = table[static_cast<int64_t>(b) * a.cache.max_blocks + blk];
    return (id < 0 || id >= a.cache.n_blocks) ? 0 : id;
  };
  // ---- per-lane LDS read offsets (as in the 128-row form)
  int sa_off[4];
  {
    const int t = l & 31, sw = swz(t);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) sa_off[kk] = t * 128 + (((2 * kk + (l >> 5)) ^ sw) << 4);
  }
  int va_off[2][2];
  {
    const int g = l >> 4, i = l & 15;
#pragma unroll
    for (int sec = 0; sec < 2; ++sec) {
      const int t = 4 * (g >> 1) + (i >> 2) + 8 * sec;
      const int sw = swz(t);
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const int low = 2 * (g & 1) + ((i & 3) >> 1);
        va_off[sec][par] = t * 128 + (((4 * par + low) ^ sw) << 4) + ((i & 1) << 3);
      }
    }
  }

  const int bound = min(t_end - 1, kv - a.n_q);
  const int first_masked = bound - t_begin - (kTileT - 1) >= 0 ? (bound - t_begin - (kTileT - 1)) / kTileT + 1 : 0;
  auto tile_ptr = [&](auto kc) __attribute__((always_inline)) -> char* {
    constexpr int K = decltype(kc)::value;
    if constexpr (K == 0) return s_tile0;
    else if constexpr (K == 1) return s_tile1;
    else if constexpr (K == 2) return s_tile2;
    else return s_tile3;
  };
  const int64_t part_row0 = (static_cast<int64_t>(b) * a.n_splits + s) * a.n_q;

  // The two roles run as separate copies of the loop (the branch is taken once, so
  // the score waves' Q fragments and the value waves' accumulators never share a
  // live range); both copies pass the same barriers in the same order.
  auto run = [&](auto role) __attribute__((always_inline)) {
    constexpr bool SC = decltype(role)::value != 0;
    u32x4 qf[SC ? KS : 1];           // score waves: this row's Q_cat fragments
    f32x16 acc[SC ? 1 : CBW * RB];   // value waves: Oᵀ, acc[cbl * RB + rb]
    float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.f;
    uint64_t ovr = 0;
    int pg_next = 0;

    auto tile_rsrc = [&](int it) __attribute__((always_inline)) -> u32x4 {
      const int t0 = t_begin + it * kTileT;
      const char* base;
      if (!paged) {
        base = cache + (static_cast<int64_t>(b) * a.cache.t_max + t0) * ROWB;
      } else {
        base = cache + (static_cast<int64_t>(pg_next) * a.cache.block_size + t0 % a.cache.block_size) * ROWB;
        if (it + 1 < n_tiles) pg_next = page_id(it + 1);
      }
      const uint64_t ba = reinterpret_cast<uint64_t>(base);
      const uint32_t rows = static_cast<uint32_t>(min(kTileT, t_end - t0));
      return u32x4{static_cast<uint32_t>(ba), static_cast<uint32_t>(ba >> 32) & 0xFFFFu,
                   rows * static_cast<uint32_t>(ROWB), 0x00020000u};
    };
    auto issue_tile = [&](int it, char* tile) __attribute__((always_inline)) {
      const u32x4 rsrc = tile_rsrc(it);
#pragma unroll
      for (int n = 0; n < LOADS; ++n) {
        const int np = 2 * n + vw;  // wave-uniform
        const int G = np >> 2, rq = np & 3;
        dma_b128(rsrc, ld_lane[rq & 1], static_cast<uint32_t>(G * 128 + (rq >> 1) * 16 * ROWB),
                 static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_ptr(tile) + np * 1024)));
      }
    };
    constexpr int SDEPTH = 6;
    auto scores = [&](const char* tile) __attribute__((always_inline)) {
      f32x16 sc = {};
      u32x4 fa[SDEPTH];
      auto frag = [&](int ks) __attribute__((always_inline)) {
        return *(lds_u32x4*)(lds_ptr(tile) + sa_off[ks & 3] + (ks >> 2) * 4096);
      };
#pragma unroll
      for (int ks = 0; ks < SDEPTH; ++ks) fa[ks] = frag(ks);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) mfma_v(sc, fa[ks % SDEPTH], qf[ks]);
        else mfma_v_last(sc, fa[ks % SDEPTH], qf[ks]);
        if (ks + SDEPTH < KS) fa[ks % SDEPTH] = frag(ks + SDEPTH);
      }
      return sc;
    };
    auto apply_mask = [&](f32x16& sc, int it) __attribute__((always_inline)) {
      const int t0 = t_begin + it * kTileT;
      const int lim = min(t_end - 1, vis_own);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int tok = t0 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
        sc[v] = tok > lim ? -INFINITY : sc[v];
      }
    };
    // softmax of a tile against the row's fixed reference: P as 8 packed bf16 pairs
    // (values 2k, 2k + 1 of the score accumulator); `overrun` if a score passed it by
    // more than the headroom
    auto softmax = [&](const f32x16& sc, bool allow_restart, u32x4* p) __attribute__((always_inline)) -> bool {
      const float m0 = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      const float m1 = fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7]));
      const float m2 = fmaxf(fmaxf(sc[8], sc[9]), fmaxf(sc[10], sc[11]));
      const float m3 = fmaxf(fmaxf(sc[12], sc[13]), fmaxf(sc[14], sc[15]));
      const float mx = half_max(fmaxf(fmaxf(m0, m1), fmaxf(m2, m3)));
      m_seen = fmaxf(m_seen, mx);
      if (m_ref == -INFINITY) m_ref = mx;  // first tile where the row sees a token
      const bool overrun = allow_restart && mx > m_ref + kHeadroom;
      const float mref = m_ref == -INFINITY ? 0.f : m_ref;
      float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float p0 = fast_exp2(sc[2 * q] - mref), p1 = fast_exp2(sc[2 * q + 1] - mref);
        p[q >> 2][q & 3] = pack_bf16x2(p0, p1);
        ps[q & 3] += p0 + p1;
      }
      l_run += half_sum((ps[0] + ps[1]) + (ps[2] + ps[3]));
      return overrun;
    };
    // value MFMAs of one tile: this value wave's 8 column blocks x both row blocks,
    // P from LDS one k-step at a time, the transposed cache fragments through a
    // four-deep window
    auto pv = [&](const char* tile, const char* pbuf) __attribute__((always_inline)) {
      auto load = [&](int f) __attribute__((always_inline)) {
        const int kk = f / CBW, cb = CBW * vw + f % CBW;
        lds_char* tb = lds_ptr(tile) + kk * 16 * 128 + (cb >> 1) * 4096;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tb + va_off[0][cb & 1]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tb + va_off[1][cb & 1]));
        const i16x8 af = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return af;
      };
      constexpr int NF = 2 * CBW, WIN = 4;
      i16x8 frag[WIN];
#pragma unroll
      for (int f = 0; f < WIN; ++f) frag[f] = load(f);
      u32x4 pb[RB];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int kk = f / CBW, cbl = f % CBW;
        if (cbl == 0) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) pb[rb] = *(lds_u32x4*)(lds_ptr(pbuf) + (rb * 2 + kk) * 1024 + l * 16);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          acc[cbl * RB + rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, frag[f % WIN]), as_bf16x8(pb[rb]), acc[cbl * RB + rb], 0, 0, 0);
          if (rb == RB - 1 && f + WIN < NF) frag[f % WIN] = load(f + WIN);
        }
      }
    };
    auto vstep = [&](auto kc, auto first, int i, bool allow_restart) __attribute__((always_inline)) {
      constexpr int K = decltype(kc)::value;
      constexpr bool FIRST = decltype(first)::value != 0;
      if constexpr (!SC) {
        if (i + 1 < n_tiles) wait_vm<LOADS>();  // tile i has landed (tile i + 1 in flight)
        else wait_vm<0>();
      }
      lds_barrier();  // tile i and P of tile i - 1 everywhere; tile i - 2 is free
      if constexpr (!SC) {
        if (i + 2 < n_tiles) issue_tile(i + 2, tile_ptr(Ic<(K + 2) % 4>{}));
        if constexpr (!FIRST) pv(tile_ptr(Ic<(K + 3) % 4>{}), s_p + ((K + 1) & 1) * PBUF);
      } else {
        f32x16 sc = scores(tile_ptr(kc));
        if (i >= first_masked) apply_mask(sc, i);  // uniform
        u32x4 p[2];
        const bool overrun = softmax(sc, allow_restart, p);
        ovr |= __builtin_amdgcn_ballot_w64(overrun);
        *(lds_u32x4*)(lds_ptr(s_p + (K & 1) * PBUF) + (w * 2 + 0) * 1024 + l * 16) = p[0];
        *(lds_u32x4*)(lds_ptr(s_p + (K & 1) * PBUF) + (w * 2 + 1) * 1024 + l * 16) = p[1];
      }
    };
    auto prologue = [&]() __attribute__((always_inline)) {
      if constexpr (!SC) {
        if (paged) pg_next = page_id(0);
        if (0 < n_tiles) issue_tile(0, s_tile0);
        if (1 < n_tiles) issue_tile(1, s_tile1);
      }
    };

    prologue();
    if constexpr (SC) {
      const u32x4* qp = reinterpret_cast<const u32x4*>(a.q_cat) +
                        ((static_cast<int64_t>(b) * hgroups + hg) * 2 + w) * KS * 64 + l;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = qp[ks * 64];
      wait_vm<0>();
    }
    for (int pass = 0;; ++pass) {
      const bool allow_restart = pass < kMaxRestarts;
      if constexpr (!SC) {
#pragma unroll
        for (int k = 0; k < CBW * RB; ++k) acc[k] = f32x16{};
      }
      l_run = 0.f;
      ovr = 0;
      if (pass > 0) prologue();
      vstep(Ic<0>{}, Ic<1>{}, 0, allow_restart);
      for (int i = 1; i < n_tiles; i += 4) {
#define MLA_RSTEP(KK, D) \
  if (i + D < n_tiles) vstep(Ic<KK>{}, Ic<0>{}, i + D, allow_restart);
        MLA_RSTEP(1, 0)
        MLA_RSTEP(2, 1)
        MLA_RSTEP(3, 2)
        MLA_RSTEP(0, 3)
#undef MLA_RSTEP
      }
      // restart flags in tile buffer (n_tiles + 1) % 4 (its tile was last read in step
      // n_tiles - 2, or never used; no load targets it)
      const int kf = (n_tiles + 1) & 3;
      int* s_flag = reinterpret_cast<int*>(kf == 0 ? s_tile0 : kf == 1 ? s_tile1 : kf == 2 ? s_tile2 : s_tile3);
      if (l == 0) s_flag[w] = ovr != 0;
      lds_barrier();  // P of the last tile and every wave's flag
      const bool restart = (s_flag[0] | s_flag[1]) != 0;  // the score waves' flags; uniform
      if (!restart) {
        if constexpr (!SC) {
          const int kl = (n_tiles - 1) & 3;
          const char* lt = kl == 0 ? s_tile0 : kl == 1 ? s_tile1 : kl == 2 ? s_tile2 : s_tile3;
          pv(lt, s_p + ((n_tiles - 1) & 1) * PBUF);
        }
        break;
      }
      if constexpr (!SC) wait_vm<0>();
      lds_barrier();  // every wave's flag reads are done before the next pass writes P
      m_ref = m_seen;
    }

    // ---- epilogue: 1 / l of each row from the score waves; each value wave stages
    //      its 256 columns of the 64 rows in tile buffer v ([64 rows][32 chunks],
    //      chunk ^ (row & 31)) and writes them out as contiguous 512-byte row segments
    float* s_inv = reinterpret_cast<float*>(s_p + (n_tiles & 1) * PBUF + 16);
    if constexpr (SC) {
      if (l < 32) s_inv[r_own] = l_run > 0.f ? 1.f / l_run : 0.f;
    }
    lds_barrier();  // every wave is past the last tile; s_inv complete
    if constexpr (!SC) {
      constexpr int CPR = 4 * CBW;   // 16-byte chunks per staged row (32)
      constexpr int RSB = 16 * CPR;  // staged row bytes (512)
      char* stg = vw == 0 ? s_tile0 : s_tile1;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int row = 32 * rb + (l & 31);
        const float inv = s_inv[row];
#pragma unroll
        for (int cbl = 0; cbl < CBW; ++cbl)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const f32x16& o = acc[cbl * RB + rb];
            const int chunk = (4 * cbl + v4) ^ (row & 31);
            const u32x2 v2 = {pack_bf16x2(o[4 * v4] * inv, o[4 * v4 + 1] * inv),
                              pack_bf16x2(o[4 * v4 + 2] * inv, o[4 * v4 + 3] * inv)};
            *(lds_u32x2*)(lds_ptr(stg) + row * RSB + chunk * 16 + (l >> 5) * 8) = v2;
          }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging writes are done
      __builtin_amdgcn_wave_barrier();
      constexpr int RPI = 64 / CPR;  // rows per wave instruction (2)
#pragma unroll 4
      for (int q = 0; q < R / RPI; ++q) {
        const int row = RPI * q + l / CPR, ch = l % CPR;
        const int j = row / HG, head = hg * HG + row % HG;
        const u32x4 v = *(lds_u32x4*)(lds_ptr(stg) + row * RSB + ((ch ^ (row & 31)) << 4));
        *reinterpret_cast<u32x4*>(a.o_part + ((part_row0 + j) * a.h + head) * 512 + 256 * vw + ch * 8) = v;
      }
    } else {
      if (l < 32) {
        float* ml = a.ml_part + ((part_row0 + j_own) * a.h + head_own) * 2;
        ml[0] = m_ref;
        ml[1] = l_run;
      }
    }
  };
  if (scorer) run(Ic<1>{});
  else run(Ic<0>{});
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  // hipExtLaunchKernelGGL stamps ev0/ev1 from the dispatch itself, so an event pair
  // brackets exactly this kernel's execution (null events: plain launch).
  const int rows = a.h * a.n_q;
  if (a.role_split) {
    if (rows % 64 != 0) return hipErrorInvalidValue;
    const unsigned units = static_cast<unsigned>(a.batch * a.n_splits * (rows / 64));
    if (a.d_r == 64)
      hipExtLaunchKernelGGL(decode_roles_kernel<64>, dim3(units), dim3(256), 0, s, ev0, ev1, 0, a);
    else if (a.d_r == 0)
      hipExtLaunchKernelGGL(decode_roles_kernel<0>, dim3(units), dim3(256), 0, s, ev0, ev1, 0, a);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (rows % 128 != 0) return hipErrorInvalidValue;
  const unsigned units = static_cast<unsigned>(a.batch * a.n_splits * (rows / 128));
  if (a.d_r == 64)
    hipExtLaunchKernelGGL(decode_kernel<4, 64>, dim3(units), dim3(256), 0, s, ev0, ev1, 0, a);
  else if (a.d_r == 0)
    hipExtLaunchKernelGGL(decode_kernel<4, 0>, dim3(units), dim3(256), 0, s, ev0, ev1, 0, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mla
