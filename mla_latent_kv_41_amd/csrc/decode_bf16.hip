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
// Each wave (one per SIMD) owns 32 query rows end to end: their Q_cat fragments
// stay in VGPRs, their Oᵀ accumulators (512 columns x 32 rows fp32 = 256 registers
// per lane) in AGPRs, and their softmax state in lanes. The value MFMA takes the
// tile's 32 tokens in the order the score MFMA leaves them in its accumulator, so
// P goes from the score accumulator to the value MFMA without leaving registers.
// Waves share only the tile buffers.
//
// Pipelining: 128-row workgroups (one per CU) keep four tile buffers, so the
// direct-to-LDS loads of a tile are issued three tiles before it is consumed;
// 64-row workgroups run two per CU with two tile buffers each.
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
// reference by more than 64 (P > 2^64), the workgroup drains its loads and
// restarts its token range with the largest score seen as the new reference (at
// most 8 times). The decision is workgroup-uniform, through LDS flags read one
// tile later, so every wave takes the same barriers.
//
// Output per (b, split): the normalised partial O/l as bf16 rows of 512 (written
// coalesced through LDS) and (m, l) in fp32; the combine kernel merges splits.
#include "common.hpp"
#include "launch.hpp"

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
  static constexpr int NBUF = NW == 4 ? 4 : 2;             // tile buffers
  static constexpr int ROW = 512 + DR;                     // elements per cache row
  static constexpr int ROWB = ROW * 2;                     // bytes per cache row
  static constexpr int CH = ROW / 8;                       // 16-byte chunks per row
  static constexpr int KS = ROW / 16;                      // score k-steps (K=16 each)
  static constexpr int R = 32 * NW;                        // query rows per workgroup
  static constexpr int TILE_BYTES = kTileT * ROWB;
  static constexpr int LOADS = (kTileT * CH) / (64 * NW);  // 16-B loads per lane per tile
};

template <int V>
struct Ic {
  static constexpr int value = V;
};

// s_waitcnt that bounds only the vector-memory counter (lgkm and exp left free).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace

template <int NW, int DR>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  using C = Cfg<NW, DR>;
  constexpr int NBUF = C::NBUF;
  // Tile buffers as distinct arrays: reads of one are provably independent of the
  // direct-to-LDS loads landing in another, so they need no load wait.
  __shared__ __attribute__((aligned(1024))) char s_tile0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char s_tile1[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char s_tile2[NBUF > 2 ? C::TILE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char s_tile3[NBUF > 3 ? C::TILE_BYTES : 16];
  __shared__ int s_restart[3];  // restart requests of tile i live in slot i % 3

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
  // this lane's row r = 32w + l%32 (lanes l and l^32 hold the same row)
  const int r_own = 32 * w + (l & 31);
  const int j_own = r_own / HG;
  const int head_own = hg * HG + r_own % HG;
  const int vis_own = kv - a.n_q + j_own;  // last visible position of this row

  // ---- Q_cat fragments (B operand of the score MFMA): k = 16ks + 8(l/32) + e
  u32x4 qf[C::KS];
  {
    const int64_t m = static_cast<int64_t>(b) * a.n_q + j_own;
    const u32x4* qp = reinterpret_cast<const u32x4*>(a.q_cat + (m * a.h + head_own) * C::ROW) + (l >> 5);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = qp[2 * ks];
  }

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

  // A 32-token tile never straddles a block (ranges start at multiples of 32 and
  // blocks are multiples of 32 tokens), so one buffer resource covers the tile;
  // its size bound keeps every load of the tile inside it.
  auto issue_tile = [&](int it, char* tile) __attribute__((always_inline)) {
    const int t0 = t_begin + it * kTileT;
    lds_char* dst = lds_ptr(tile);
    const char* base;
    if (!paged) {
      base = cache + (static_cast<int64_t>(b) * a.cache.t_max + t0) * C::ROWB;
    } else {
      const int blk = t0 / a.cache.block_size;
      int id = a.cache.block_table[static_cast<int64_t>(b) * a.cache.max_blocks + blk];
      if (id < 0 || id >= a.cache.n_blocks) id = 0;  // out-of-range entry: stay in bounds
      base = cache + (static_cast<int64_t>(id) * a.cache.block_size + t0 % a.cache.block_size) * C::ROWB;
    }
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, C::TILE_BYTES, 0x00020000);
    const bool full = t0 + kTileT <= t_end;
    const int last = t_end - 1 - t0;  // rows past it re-read row `last` (masked later)
#pragma unroll
    for (int n = 0; n < C::LOADS; ++n) {
      const int np = n * NW + w;  // wave-uniform
      const int G = np >> 2, rq = np & 3;
      // uniform part: group G columns, rows 8*rq (minus the odd-quad base in ld_lane)
      uint32_t soff = static_cast<uint32_t>(G * 128 + (rq >> 1) * 16 * C::ROWB);
      uint32_t voff = ld_lane[rq & 1];
      if (!full) {
        // the LDS slot keeps its chunk position; its source row is clamped to `last`
        const int row = 8 * rq + (l >> 3);
        const uint32_t c16 = voff - static_cast<uint32_t>((8 * (rq & 1) + (l >> 3)) * C::ROWB);
        voff = static_cast<uint32_t>(min(row, last) * C::ROWB) + c16;
        soff = static_cast<uint32_t>(G * 128);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + np * 1024), 16, voff, soff, 0, 0);
    }
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

  f32x16 acc[16];  // Oᵀ: column block cb (32 latent columns) x this wave's 32 rows
  float m_ref = -INFINITY;   // this row's fixed reference max
  float m_seen = -INFINITY;  // largest score this row has seen
  float l_run = 0.f;
  if (tid < 3) s_restart[tid] = 0;

  // ---- scores: Sᵀ[32 tokens][32 rows of this wave], four fragments in flight
  auto scores = [&](const char* tile) __attribute__((always_inline)) {
    f32x16 sc = {};
    u32x4 fa[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) fa[kk] = *(lds_u32x4*)(lds_ptr(tile) + sa_off[kk]);  // group 0
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[ks & 3]), as_bf16x8(qf[ks]), sc, 0, 0, 0);
      if (ks + 4 < C::KS) fa[ks & 3] = *(lds_u32x4*)(lds_ptr(tile) + sa_off[ks & 3] + ((ks + 4) >> 2) * 4096);
    }
    return sc;
  };

  // ---- softmax of tile `it` for row r_own against the fixed reference: returns P
  //      as 8 packed bf16 pairs (values 2k, 2k+1 of the score accumulator) and
  //      whether a score overran the reference by more than the headroom
  struct Soft {
    u32x4 p[2];
    bool overrun;
  };
  auto softmax = [&](f32x16 sc, int it) __attribute__((always_inline)) {
    const int t0 = t_begin + it * kTileT;
    const int lim = min(t_end - 1, vis_own);  // last token this row may see
    if (t0 + kTileT - 1 > min(t_end - 1, kv - a.n_q)) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int tok = t0 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
        if (tok > lim) sc[v] = -INFINITY;
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sc[v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    m_seen = fmaxf(m_seen, mx);
    // first visible tile of the row: nothing accumulated yet, so set the reference
    if (m_ref == -INFINITY) m_ref = mx;
    Soft r;
    r.overrun = mx > m_ref + kHeadroom;
    const float mref = m_ref == -INFINITY ? 0.f : m_ref;
    float psum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const float p0 = fast_exp2(sc[v] - mref), p1 = fast_exp2(sc[v + 1] - mref);
      psum += p0 + p1;
      r.p[v >> 3][(v >> 1) & 3] = pack_bf16x2(p0, p1);
    }
    psum += __shfl_xor(psum, 32);
    l_run += psum;
    return r;
  };

  // ---- values: Oᵀ[c][r] += Σ_t Cᵀ[c][t] · Pᵀ[t][r] for all 512 columns; the 32
  //      (k-step, column block) fragments stream through a four-deep window of
  //      transposed reads so each MFMA finds its operand already loaded
  auto pv = [&](const char* tile, const Soft& sp) __attribute__((always_inline)) {
    auto load = [&](int f) __attribute__((always_inline)) {
      const int kk = f >> 4, cb = f & 15;
      lds_char* tb = lds_ptr(tile) + kk * 16 * 128 + (cb >> 1) * 4096;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tb + va_off[0][cb & 1]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tb + va_off[1][cb & 1]));
      const i16x8 af = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return af;
    };
    i16x8 frag[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) frag[f] = load(f);
#pragma unroll
    for (int f = 0; f < 32; ++f) {
      const int kk = f >> 4, cb = f & 15;
      acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, frag[f & 3]),
                                                       as_bf16x8(sp.p[kk]), acc[cb], 0, 0, 0);
      if (f + 4 < 32) frag[f & 3] = load(f + 4);
    }
  };

  auto tile_ptr = [&](auto kc) __attribute__((always_inline)) -> char* {
    constexpr int K = decltype(kc)::value;
    if constexpr (K == 0) return s_tile0;
    else if constexpr (K == 1) return s_tile1;
    else if constexpr (K == 2) return s_tile2;
    else return s_tile3;
  };

  // step i: tile i in buffer i % NBUF; tiles up to i + NBUF - 2 were issued before.
  // Returns true when a restart was requested at tile i - 1.
  auto step = [&](auto kc, int i) __attribute__((always_inline)) -> bool {
    constexpr int K = decltype(kc)::value;
    const int ahead = min(n_tiles - 1, i + NBUF - 2) - i;  // tiles issued after tile i
    if constexpr (NBUF == 4) {
      if (ahead >= 2) wait_vm<2 * C::LOADS>();
      else if (ahead == 1) wait_vm<C::LOADS>();
      else wait_vm<0>();
    } else {
      wait_vm<0>();
    }
    __syncthreads();  // tile i everywhere; every wave is done with tile i-1
    if (i > 0 && s_restart[(i + 2) % 3]) return true;  // request made at tile i-1
    if (tid == 0) s_restart[(i + 1) % 3] = 0;         // slot of tile i-2, read at tile i-1
    if (i + NBUF - 1 < n_tiles) issue_tile(i + NBUF - 1, tile_ptr(Ic<(K + NBUF - 1) % NBUF>{}));
    const Soft cur = softmax(scores(tile_ptr(kc)), i);
    if (__builtin_amdgcn_ballot_w64(cur.overrun)) s_restart[i % 3] = 1;
    pv(tile_ptr(kc), cur);
    return false;
  };

  for (int restarts = 0;; ++restarts) {
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) acc[cb] = f32x16{};
    l_run = 0.f;
#pragma unroll
    for (int k = 0; k < NBUF - 1; ++k)
      if (k < n_tiles) issue_tile(k, k == 0 ? s_tile0 : k == 1 ? s_tile1 : s_tile2);
    bool restart = false;
    for (int i = 0; i < n_tiles && !restart; i += NBUF) {
      restart = step(Ic<0>{}, i);
      if (!restart && i + 1 < n_tiles) restart = step(Ic<1>{}, i + 1);
      if constexpr (NBUF == 4) {
        if (!restart && i + 2 < n_tiles) restart = step(Ic<2>{}, i + 2);
        if (!restart && i + 3 < n_tiles) restart = step(Ic<3>{}, i + 3);
      }
    }
    wait_vm<0>();
    __syncthreads();
    if (!restart) restart = s_restart[(n_tiles - 1) % 3] != 0;  // request at the last tile
    if (!restart || restarts == kMaxRestarts) break;
    // restart the range with the largest score seen as every row's reference
    __syncthreads();
    if (tid < 3) s_restart[tid] = 0;
    m_ref = m_seen;
    __syncthreads();
  }

  // ---- epilogue: normalised partial O/l as bf16 rows, staged in LDS (wave w uses
  //      tile buffer w) so every global store is a whole 1 KiB row; every wave is
  //      past the last tile (barrier above)
  const int64_t part_row0 = (static_cast<int64_t>(b) * a.n_splits + s) * a.n_q;
  char* stg = w == 0 ? s_tile0 : w == 1 ? s_tile1 : w == 2 ? s_tile2 : s_tile3;  // [32][64 chunks], chunk ^ (row & 15)
  {
    const int rr = l & 31;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int c0 = 32 * cb + 8 * v4;  // this lane holds columns c0 + 4(l/32) .. +3
        const int chunk = (c0 >> 3) ^ (rr & 15);
        u32x2 v2 = {pack_bf16x2(acc[cb][4 * v4] * inv, acc[cb][4 * v4 + 1] * inv),
                    pack_bf16x2(acc[cb][4 * v4 + 2] * inv, acc[cb][4 * v4 + 3] * inv)};
        *(lds_u32x2*)(lds_ptr(stg) + rr * 1024 + chunk * 16 + (l >> 5) * 8) = v2;
      }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging writes are done
  __builtin_amdgcn_wave_barrier();
#pragma unroll 4
  for (int q = 0; q < 32; ++q) {
    const int r = 32 * w + q;
    const int j = r / HG, head = hg * HG + r % HG;
    const u32x4 v = *(lds_u32x4*)(lds_ptr(stg) + q * 1024 + ((l ^ (q & 15)) << 4));
    *reinterpret_cast<u32x4*>(a.o_part + ((part_row0 + j) * a.h + head) * 512 + l * 8) = v;
  }
  if (l < 32) {
    float* ml = a.ml_part + ((part_row0 + j_own) * a.h + head_own) * 2;
    ml[0] = m_ref;
    ml[1] = l_run;
  }
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
  const int rows = a.h * a.n_q;
  if (rows % 128 == 0) {
    const unsigned units = static_cast<unsigned>(a.batch * a.n_splits * (rows / 128));
    if (a.d_r == 64)
      decode_kernel<4, 64><<<units, 256, 0, s>>>(a);
    else
      decode_kernel<4, 0><<<units, 256, 0, s>>>(a);
  } else {
    // 64 query rows per workgroup (e.g. 64 heads, one query): position-free rows only
    if (a.d_r != 0) return hipErrorInvalidValue;
    const unsigned units = static_cast<unsigned>(a.batch * a.n_splits * (rows / 64));
    decode_kernel<2, 0><<<units, 128, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mla
