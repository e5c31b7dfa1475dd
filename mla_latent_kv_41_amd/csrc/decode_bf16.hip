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
// chunk k of the group at position k ^ swz(t), swz(t) = (t >> 1) & 7: rows 2u and
// 2u + 1 (128 bytes apart) share a permutation, and the eight pairs of 16 rows use
// eight different ones. The score operand's column reads are then free of bank
// conflicts both as 32 rows x one chunk per half wave (128-row and role-split forms)
// and as 16 rows x two chunks (eight-wave form): 243-249 B/cycle per CU for
// ds_read_b128, where the eight-wave reads under the earlier pair-interleaved
// permutation ran at 128.
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
// Output per (sequence, token range): the partial O (relative to each row's
// reference m, not yet divided by l) as fp32 rows of 512, stored straight from the
// accumulators, and (m, l) in fp32; the combine kernel merges the ranges.
//
// Work: a launch takes the (sequence, range) pairs of one list the query
// preparation built on the device; workgroup u takes pair u / groups and head
// group u % groups (XCD-aware: each XCD gets a contiguous run of units, so one
// sequence's ranges and head groups share an L2). A workgroup's R rows are R / 32
// consecutive 32-row query blocks of its sequence (block = one query x 32 heads).
#include "common.hpp"
#include "launch.hpp"
#include <hip/hip_ext.h>

namespace mla {

namespace {

constexpr int kTileT = 32;    // tokens per tile
constexpr float kHeadroom = 64.0f;  // largest score - reference allowed (base-2 units)
constexpr int kMaxRestarts = 8;

__device__ __forceinline__ int swz(int t) { return (t >> 1) & 7; }

// LDS of the 128-row and role-split forms: four tile buffers of kTileT rows of 576
// bf16 and the P buffers, 160 KiB in all. Declared once at file scope, so a launch
// that runs either form in its workgroups (decode_mixed_kernel) holds one set. Tile
// buffers as distinct arrays: reads of one are provably independent of the
// direct-to-LDS loads landing in another, so they need no load wait.
constexpr int kLdsTileBytes = kTileT * (512 + 64) * 2;
constexpr int kLdsPBytes = 16 * 1024;
__shared__ __attribute__((aligned(1024))) char lds_tile0[kLdsTileBytes];
__shared__ __attribute__((aligned(1024))) char lds_tile1[kLdsTileBytes];
__shared__ __attribute__((aligned(1024))) char lds_tile2[kLdsTileBytes];
__shared__ __attribute__((aligned(1024))) char lds_tile3[kLdsTileBytes];
__shared__ __attribute__((aligned(16))) char lds_p[kLdsPBytes];
static_assert(4 * kLdsTileBytes + kLdsPBytes <= 160 * 1024, "LDS");

// Tokens [t_begin, t_end) of range s of a kv-token sequence that the plan splits into
// ns = ceil(kv / chunk) ranges. The sequence's nt = ceil(kv / kTileT) tiles are dealt
// out evenly, range s taking tiles floor(s nt / ns) .. floor((s + 1) nt / ns) - 1:
// the ranges of a sequence differ by at most one tile, none exceeds chunk tokens
// (chunk is a multiple of kTileT, so nt <= ns chunk / kTileT), each holds at least
// one tile (chunk >= kTileT, so ns <= nt), and the last ends at kv. With ranges of
// chunk tokens and a remainder instead, 4097 tokens in four ranges would take 33,
// 33, 33 and 30 tiles; dealt out they take 32, 32, 32 and 33, the last tile holding
// one token.
__device__ __forceinline__ void range_tokens(int s, int kv, int chunk, int& t_begin, int& t_end) {
  const int ns = max(1, (kv + chunk - 1) / chunk);  // kv >= 1 for every listed pair
  const int nt = max(1, (kv + kTileT - 1) / kTileT);
  t_begin = kTileT * static_cast<int>(static_cast<int64_t>(s) * nt / ns);
  t_end = min(kTileT * static_cast<int>(static_cast<int64_t>(s + 1) * nt / ns), kv);
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
};

template <int V>
struct Ic {
  static constexpr int value = V;
};

// Phase stamps (instrumented builds only, compiled with -DMLA_STAMPS): each wave of
// a workgroup whose unit is below kStampUnits reads the shader clock (s_memtime) at
// entry, right after every step's barrier (where the wave has no LDS operation
// outstanding, so a read costs one scalar round trip and no other wait), after its
// last value pass and after its epilogue's stores have completed, and writes
//   [0] entry, [1] first step's barrier, [2] last step's barrier, [3] barriers
//   passed, [4] sum of the intervals between consecutive barriers, [5] shortest,
//   [6] longest, [7] after the last value pass, [8] stores complete, [9], [10] sums
//   of the cycles from each step's barrier to the kernel's marks 0 and 1 ([11]: mark 2)
// to stamp_buf[unit][wave][kStampSlots]. Product builds compile none of it.
#ifdef MLA_STAMPS
constexpr bool kStamps = true;
#else
constexpr bool kStamps = false;
#endif
constexpr int kStampUnits = 64, kStampSlots = 16;
constexpr int kStampWaves = 8;  // records per unit (one per wave)
struct StampRec {
  uint64_t v[kStampSlots];
  __device__ __forceinline__ void begin() {
    v[0] = __builtin_amdgcn_s_memtime();
    for (int k = 1; k < kStampSlots; ++k) v[k] = 0;
    v[5] = ~0ull;
  }
  __device__ __forceinline__ void step() {  // right after a barrier
    const uint64_t t = __builtin_amdgcn_s_memtime();
    if (v[3] == 0) {
      v[1] = t;
    } else {
      const uint64_t d = t - v[2];
      v[4] += d;
      v[5] = d < v[5] ? d : v[5];
      v[6] = d > v[6] ? d : v[6];
    }
    v[2] = t;
    ++v[3];
  }
  __device__ __forceinline__ void loop_end() { v[7] = __builtin_amdgcn_s_memtime(); }
  // [9 + k] sums, over the steps, the cycles from the step's barrier to mark k
  __device__ __forceinline__ void mark(int k) {
    if (v[3] != 0) v[9 + k] += __builtin_amdgcn_s_memtime() - v[2];
  }
  __device__ __forceinline__ void end(uint64_t* buf, int unit, int wave, int lane) {
    wait_vm<0>();
    v[8] = __builtin_amdgcn_s_memtime();
    if (unit < kStampUnits && lane == 0)
      for (int k = 0; k < kStampSlots; ++k) buf[(static_cast<int64_t>(unit) * kStampWaves + wave) * kStampSlots + k] = v[k];
  }
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

// v_mfma_f32_16x16x32_bf16 (4 passes) in VGPR form, for the eight-wave form's score
// chains: as an opaque statement it keeps the chain's LDS fragment window as written
// (the compiler shortens the window of the builtin form to two reads in flight).
// The first of a chain takes a zero accumulator, the last waits out the result
// latency (7 wait states for a 4-pass MFMA before VALU reads its result; 11 here).
__device__ __forceinline__ void mfma16_first(f32x4& c, const u32x4& a, const u32x4& b) {
  asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16(f32x4& c, const u32x4& a, const u32x4& b) {
  asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_last(f32x4& c, const u32x4& a, const u32x4& b) {
  asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 2" : "+v"(c) : "v"(a), "v"(b));
}

// The same with the B operand in AGPRs (the precise form's low query halves).
__device__ __forceinline__ void mfma_va(f32x16& c, const u32x4& a, const u32x4& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_va_last(f32x16& c, const u32x4& a, const u32x4& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 4"
      : "+v"(c) : "v"(a), "a"(b));
}

}  // namespace

// The 128-row form's work for workgroup bid of its launch.
template <int NW, int DR>
__device__ __forceinline__ void decode_128(const DecodeArgs& a, const int bid) {
  using C = Cfg<NW, DR>;
  constexpr int NBUF = C::NBUF, CBW = C::CBW, RB = C::RB;
  char* const s_tile0 = lds_tile0;
  char* const s_tile1 = lds_tile1;
  char* const s_tile2 = lds_tile2;
  char* const s_tile3 = lds_tile3;
  // P fragments [parity][row block][k-step][lane]: P of tile i goes into buffer i % 2,
  // so publishing it never waits for readers of tile i - 1's P.
  constexpr int PBUF = RB * 2 * 1024;
  char* const s_p = lds_p;
  static_assert(C::TILE_BYTES <= kLdsTileBytes && 2 * PBUF <= kLdsPBytes, "LDS");

  const int tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);  // wave index, uniform
  const int hgroups = (a.h * a.n_q) / C::R;
  const int HB = a.h / 32;  // 32-head blocks per query

  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous
  // range of units so one sequence's splits (and head groups) share an L2.
  int u = bid;
  if ((a.units & 7) == 0) u = (bid & 7) * (a.units >> 3) + (bid >> 3);
  StampRec stamp;
  if constexpr (kStamps) stamp.begin();
  const int pair = u / hgroups, hg = u - pair * hgroups;
  const WorkItem item = a.list[pair];
  if (item.b < 0) return;  // uniform: past the pairs of this launch
  const int b = item.b, kv = item.kv;
  int t_begin, t_end;
  range_tokens(item.s, kv, a.chunk, t_begin, t_end);
  if (t_begin >= t_end || kv < a.n_q) return;  // not listed by the plan
  const int n_tiles = (t_end - t_begin + kTileT - 1) / kTileT;

  // wave w's score rows: query block qb_own = RB hg + w of the sequence, i.e. query
  // j_own and heads 32 (qb_own % HB) + l%32 (lanes l and l^32 hold the same row)
  const int qb_own = RB * hg + w;
  const int j_own = qb_own / HB;
  const int head_own = 32 * (qb_own - j_own * HB) + (l & 31);
  const int vis_own = kv - a.n_q + j_own;  // last visible position of this row

  // ---- tile loads: LDS block n = 4G + q (1 KiB) holds column group G, rows 8q + l/8,
  //      chunk position l%8; its source is row t = 8q + l/8, logical chunk
  //      8G + ((l%8) ^ swz(t)). Wave w loads groups w and w + 4 whole (runs of four
  //      blocks, one M0 write each) and, with the RoPE key, block q = w of group 8.
  //      ld_adj[q] is the per-lane offset of quarter q, less the 1024 q that the
  //      run's instruction offset adds.
  uint32_t ld_adj[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = 8 * q + (l >> 3);
    ld_adj[q] = static_cast<uint32_t>(t * C::ROWB + (((l & 7) ^ swz(t)) << 4) - 1024 * q);
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
  // This wave's share of a tile (C::LOADS blocks). The whole byte offset is per lane
  // (soffset 0), so the size bound applies to all of it.
  static_assert(NW == 4 && C::LOADS == 8 + (DR == 64 ? 1 : 0), "load runs");
  auto issue_loads = [&](const u32x4& rsrc, char* tile) __attribute__((always_inline)) {
    const uint32_t base = lds_addr(tile);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int G = w + 4 * r;
      dma_run<4>(rsrc, ld_adj, static_cast<uint32_t>(G * 128), base + G * 4096);
    }
    if constexpr (DR == 64)
      dma_run<1>(rsrc, ld_adj + w, static_cast<uint32_t>(8 * 128 + 1024 * w), base + 8 * 4096 + 1024 * w);
  };
  auto issue_tile = [&](int it, char* tile) __attribute__((always_inline)) { issue_loads(tile_rsrc(it), tile); };

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
    if constexpr (kStamps) stamp.step();
    // tile i + 2 into the buffer of tile i - 2, as one burst ahead of the score
    // chain: measured cheaper than loads spread through the MFMAs, and far cheaper
    // than loads among the value phase's transposed LDS reads
    if (i + 2 < n_tiles) issue_tile(i + 2, tile_ptr(Ic<(K + 2) % 4>{}));
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
                      (static_cast<int64_t>(b) * a.n_q * HB + qb_own) * C::KS * 64 + l;
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
      if constexpr (kStamps) stamp.loop_end();
      break;
    }
    // restart the range with the largest score seen as every row's reference; the
    // barrier orders every wave's flag reads before the next pass writes P
    wait_vm<0>();
    lds_barrier();
    m_ref = m_seen;
  }

  // ---- epilogue: the partial O of this wave's columns for every row block, fp32,
  //      straight from the accumulators: lane l holds row l%32 of a block and 4
  //      adjacent columns per 4 values, so a store writes 32 bytes of each of 32 rows
  //      and four of them complete the rows' 128-byte column block. (m, l) of each
  //      row comes from its score lane.
  const int64_t prow0 = static_cast<int64_t>(item.p) * a.n_q;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int qb = RB * hg + rb, j = qb / HB;
    const int head = 32 * (qb - j * HB) + (l & 31);
    float* dst = a.o_part + ((prow0 + j) * a.h + head) * 512 + 32 * CBW * w + 4 * (l >> 5);
#pragma unroll
    for (int cbl = 0; cbl < CBW; ++cbl)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const f32x16& o = acc[cbl * RB + rb];
        *reinterpret_cast<f32x4*>(dst + 32 * cbl + 8 * v4) = f32x4{o[4 * v4], o[4 * v4 + 1], o[4 * v4 + 2], o[4 * v4 + 3]};
      }
  }
  if (l < 32) {
    float* ml = a.ml_part + ((prow0 + j_own) * a.h + head_own) * 2;
    ml[0] = m_ref;
    ml[1] = l_run;
  }
  if constexpr (kStamps) stamp.end(a.stamps, u, w, l);
}

template <int NW, int DR>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  decode_128<NW, DR>(a, blockIdx.x);
}

// Role-split form for 64 query rows per workgroup (a (sequence, token range, head
// group) unit of two 32-row query blocks). Waves 0-1 own the scores and the softmax
// of block w (its Q_cat fragments in VGPRs). Waves 2-3 own the value contraction for
// latent columns 256 v .. 256 v + 255 (v = w - 2) of all 64 rows (Oᵀ: 16 blocks of
// 32x32 fp32 in AGPRs) and issue every tile load. Both pairs run about 1.1k MFMA
// cycles per tile, so the matrix cores of all four SIMDs stay busy, while a unit
// holds half the rows of the 128-row form: a sequence needs half as many token
// ranges for the same number of workgroups, which halves the split partials.
//
// Step i (one barrier): the value waves wait for their share of tile i, everyone
// passes the barrier; the value waves issue tile i + 2 into the buffer of tile
// i - 2 and run the value MFMAs of tile i - 1 (P from buffer (i - 1) % 2); the score
// waves run tile i's score chain and softmax and publish P into buffer i % 2. P
// buffer i % 2 held tile i - 2's P, which the value waves finished reading in step
// i - 1. Restarts, masking and the output are as in the 128-row form.
//
// PRECISE: the query and the probabilities each enter the matrix cores as a pair of
// bf16 values, hi = bf16(x) and lo = bf16(x - hi), so both contractions see about 16
// significant bits of them (the cache is bf16 already). The score waves keep the
// low query halves in their AGPRs, which the role split leaves free on those waves,
// and run two MFMAs per fragment of the tile (it is read once); the value waves
// read a low P buffer beside the high one and run two MFMAs per cache fragment.
// This form serves the sequences too short for bf16 rounding of the query and of
// P to average out (the host plan sends them here).
template <int DR, bool PRECISE>
__device__ __forceinline__ void decode_roles(const DecodeArgs& a, const int bid) {
  constexpr int ROW = 512 + DR, ROWB = ROW * 2, CH = ROW / 8, KS = ROW / 16;
  constexpr int R = 64;                           // query rows per workgroup
  constexpr int TILE_BYTES = kTileT * ROWB;
  constexpr int LOADS = (kTileT * CH) / 128;      // 16-byte loads per value-wave lane per tile
  constexpr int CBW = 8;                          // value column blocks per value wave
  constexpr int RB = 2;                           // row blocks of 32 query rows
  static_assert((kTileT * CH) % 128 == 0, "tile loads per value wave");
  char* const s_tile0 = lds_tile0;
  char* const s_tile1 = lds_tile1;
  char* const s_tile2 = lds_tile2;
  char* const s_tile3 = lds_tile3;
  constexpr int PBUF = RB * 2 * 1024;  // P fragments [row block][k-step][lane]
  // [parity] high P, then (PRECISE) [parity] low P
  char* const s_p = lds_p;
  static_assert(TILE_BYTES <= kLdsTileBytes && (PRECISE ? 4 : 2) * PBUF <= kLdsPBytes, "LDS");

  const int tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);  // wave index, uniform
  const bool scorer = w < 2;
  const int vw = w - 2;  // value wave index (value waves only)
  const int hgroups = (a.h * a.n_q) / R;
  const int HB = a.h / 32;
  int u = bid;
  if ((a.units & 7) == 0) u = (bid & 7) * (a.units >> 3) + (bid >> 3);
  StampRec stamp;
  if constexpr (kStamps) stamp.begin();
  const int pair = u / hgroups, hg = u - pair * hgroups;
  const WorkItem item = a.list[pair];
  if (item.b < 0) return;  // uniform: past the pairs of this launch
  const int b = item.b, kv = item.kv;
  int t_begin, t_end;
  range_tokens(item.s, kv, a.chunk, t_begin, t_end);
  if (t_begin >= t_end || kv < a.n_q) return;  // not listed by the plan
  const int n_tiles = (t_end - t_begin + kTileT - 1) / kTileT;

  // score wave w: query block qb_own = 2 hg + w of the sequence (query j_own, heads
  // 32 (qb_own % HB) + l%32)
  const int qb_own = RB * hg + (w & 1);
  const int j_own = qb_own / HB;
  const int head_own = 32 * (qb_own - j_own * HB) + (l & 31);
  const int vis_own = kv - a.n_q + j_own;

  // ---- tile loads (value waves), in the LDS block layout of the 128-row form: value
  //      wave v loads groups v, v + 2, v + 4, v + 6 whole (runs of four blocks) and,
  //      with the RoPE key, blocks 2v and 2v + 1 of group 8 (a run of two)
  uint32_t ld_adj[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = 8 * q + (l >> 3);
    ld_adj[q] = static_cast<uint32_t>(t * ROWB + (((l & 7) ^ swz(t)) << 4) - 1024 * q);
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
  const int64_t prow0 = static_cast<int64_t>(item.p) * a.n_q;

  // The two roles run as separate copies of the loop (the branch is taken once, so
  // the score waves' Q fragments and the value waves' accumulators never share a
  // live range); both copies pass the same barriers in the same order.
  auto run = [&](auto role) __attribute__((always_inline)) {
    constexpr bool SC = decltype(role)::value != 0;
    u32x4 qf[SC ? KS : 1];                  // score waves: this row's Q_cat fragments
    u32x4 ql[SC && PRECISE ? KS : 1];       // score waves, PRECISE: low halves (AGPRs)
    f32x16 acc[SC ? 1 : CBW * RB];          // value waves: Oᵀ, acc[cbl * RB + rb]
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
    static_assert(LOADS == 16 + (DR == 64 ? 2 : 0), "load runs");
    auto issue_tile = [&](int it, char* tile) __attribute__((always_inline)) {
      const u32x4 rsrc = tile_rsrc(it);
      const uint32_t base = lds_addr(tile);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int G = vw + 2 * r;
        dma_run<4>(rsrc, ld_adj, static_cast<uint32_t>(G * 128), base + G * 4096);
      }
      if constexpr (DR == 64)
        dma_run<2>(rsrc, ld_adj + 2 * vw, static_cast<uint32_t>(8 * 128 + 2048 * vw), base + 8 * 4096 + 2048 * vw);
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
        if constexpr (PRECISE) {
          mfma_v(sc, fa[ks % SDEPTH], qf[ks]);
          if (ks + 1 < KS) mfma_va(sc, fa[ks % SDEPTH], ql[ks]);
          else mfma_va_last(sc, fa[ks % SDEPTH], ql[ks]);
        } else {
          if (ks + 1 < KS) mfma_v(sc, fa[ks % SDEPTH], qf[ks]);
          else mfma_v_last(sc, fa[ks % SDEPTH], qf[ks]);
        }
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
    // (values 2k, 2k + 1 of the score accumulator), and (PRECISE) the low halves in
    // p_lo; `overrun` if a score passed the reference by more than the headroom
    auto softmax = [&](const f32x16& sc, bool allow_restart, u32x4* p, u32x4* p_lo) __attribute__((always_inline)) -> bool {
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
        const uint32_t hi = pack_bf16x2(p0, p1);
        p[q >> 2][q & 3] = hi;
        if constexpr (PRECISE)
          p_lo[q >> 2][q & 3] = pack_bf16x2(p0 - __uint_as_float(hi << 16), p1 - __uint_as_float(hi & 0xFFFF0000u));
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
      u32x4 pb[RB], pbl[PRECISE ? RB : 1];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int kk = f / CBW, cbl = f % CBW;
        if (cbl == 0) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            pb[rb] = *(lds_u32x4*)(lds_ptr(pbuf) + (rb * 2 + kk) * 1024 + l * 16);
            if constexpr (PRECISE) pbl[rb] = *(lds_u32x4*)(lds_ptr(pbuf) + 2 * PBUF + (rb * 2 + kk) * 1024 + l * 16);
          }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          acc[cbl * RB + rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, frag[f % WIN]), as_bf16x8(pb[rb]), acc[cbl * RB + rb], 0, 0, 0);
          if constexpr (PRECISE)
            acc[cbl * RB + rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, frag[f % WIN]), as_bf16x8(pbl[rb]), acc[cbl * RB + rb], 0, 0, 0);
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
        if constexpr (kStamps) stamp.mark(2);
      }
      lds_barrier();  // tile i and P of tile i - 1 everywhere; tile i - 2 is free
      if constexpr (kStamps) stamp.step();
      if constexpr (!SC) {
        if (i + 2 < n_tiles) issue_tile(i + 2, tile_ptr(Ic<(K + 2) % 4>{}));
        if constexpr (!FIRST) pv(tile_ptr(Ic<(K + 3) % 4>{}), s_p + ((K + 1) & 1) * PBUF);
      } else {
        f32x16 sc = scores(tile_ptr(kc));
        if (i >= first_masked) apply_mask(sc, i);  // uniform
        u32x4 p[2], p_lo[2];
        const bool overrun = softmax(sc, allow_restart, p, p_lo);
        ovr |= __builtin_amdgcn_ballot_w64(overrun);
        char* pd = s_p + (K & 1) * PBUF;
        *(lds_u32x4*)(lds_ptr(pd) + (w * 2 + 0) * 1024 + l * 16) = p[0];
        *(lds_u32x4*)(lds_ptr(pd) + (w * 2 + 1) * 1024 + l * 16) = p[1];
        if constexpr (PRECISE) {
          *(lds_u32x4*)(lds_ptr(pd) + 2 * PBUF + (w * 2 + 0) * 1024 + l * 16) = p_lo[0];
          *(lds_u32x4*)(lds_ptr(pd) + 2 * PBUF + (w * 2 + 1) * 1024 + l * 16) = p_lo[1];
        }
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
      const int64_t qoff = (static_cast<int64_t>(b) * a.n_q * HB + qb_own) * KS * 64 + l;
      const u32x4* qp = reinterpret_cast<const u32x4*>(a.q_cat) + qoff;
      const u32x4* qlp = reinterpret_cast<const u32x4*>(PRECISE ? a.q_lo : a.q_cat) + qoff;
      // No wait here: the compiler's own wait before each fragment's first use lets
      // the first score chain start while the later fragments are still arriving.
      // Score waves issue no other vector loads, so those waits cost nothing later.
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qf[ks] = qp[ks * 64];
        if constexpr (PRECISE) ql[ks] = qlp[ks * 64];
      }
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
        if constexpr (kStamps) stamp.loop_end();
        break;
      }
      if constexpr (!SC) wait_vm<0>();
      lds_barrier();  // every wave's flag reads are done before the next pass writes P
      m_ref = m_seen;
    }

    // ---- epilogue: value waves store the partial O of their 256 columns for both
    //      row blocks (fp32, straight from the accumulators, as in the 128-row
    //      form); score waves store (m, l) of their rows
    if constexpr (!SC) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int qb = RB * hg + rb, j = qb / HB;
        const int head = 32 * (qb - j * HB) + (l & 31);
        float* dst = a.o_part + ((prow0 + j) * a.h + head) * 512 + 256 * vw + 4 * (l >> 5);
#pragma unroll
        for (int cbl = 0; cbl < CBW; ++cbl)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const f32x16& o = acc[cbl * RB + rb];
            *reinterpret_cast<f32x4*>(dst + 32 * cbl + 8 * v4) =
                f32x4{o[4 * v4], o[4 * v4 + 1], o[4 * v4 + 2], o[4 * v4 + 3]};
          }
      }
    } else {
      if (l < 32) {
        float* ml = a.ml_part + ((prow0 + j_own) * a.h + head_own) * 2;
        ml[0] = m_ref;
        ml[1] = l_run;
      }
    }
  };
  if (scorer) run(Ic<1>{});
  else run(Ic<0>{});
  if constexpr (kStamps) stamp.end(a.stamps, u, w, l);
}

template <int DR, bool PRECISE>
__global__ __launch_bounds__(256) void decode_roles_kernel(DecodeArgs a) {
  decode_roles<DR, PRECISE>(a, blockIdx.x);
}

// The fast and the precise launch of one decode call as one grid: workgroups below
// fast.units take the 128-row form's units, the rest the precise form's. Workgroups
// are dispatched in order, so every fast unit is placed first and each precise one
// starts on the first CU a fast unit leaves, filling the idle end of a launch whose
// ranges differ in length (ragged batches). fast.units is a multiple of 8, so each
// part keeps its own XCD-contiguous order. Both forms take the whole of a CU's LDS.
// The precise part differs from the fast one only in its list, range length and
// unit count.
template <int DR>
__global__ __launch_bounds__(256) void decode_mixed_kernel(DecodeArgs fast, const WorkItem* prec_list,
                                                           int prec_chunk, int prec_units) {
  const int bid = blockIdx.x;
  if (bid < fast.units) {
    decode_128<4, DR>(fast, bid);
  } else {
    DecodeArgs prec = fast;
    prec.list = prec_list;
    prec.chunk = prec_chunk;
    prec.units = prec_units;
    prec.form = kFormPrecise;
    decode_roles<DR, true>(prec, bid - fast.units);
  }
}

// Eight-wave form for 64 query rows per workgroup (the unit of the role-split form:
// sequence, token range, two 32-row query blocks). Each SIMD hosts one score wave
// and one value wave, so the matrix cores of a SIMD take one wave's MFMAs while the
// other wave runs its softmax, its LDS traffic or waits for its tile loads to be
// taken: overlap the four-wave forms could only get by interleaving code within
// one wave.
//
// Score waves 0-3: wave s takes row block rb = s / 2 (32 rows: one query, 32 heads)
// and token half th = s % 2 of every tile, as two 16-row sub-blocks on
// v_mfma_f32_16x16x32_bf16 (A = 16 tokens x 32 columns of the tile, read from LDS
// once and used by both sub-blocks; B = the rows' Q_cat, held in registers). Its
// accumulators hold, in lane l, rows 16 sb + l % 16 and tokens 16 th + 4 (l / 16) +
// 0..3. The two waves of a row block share each row's reference max: they exchange
// their maxima of the range's first tile through LDS (the range's first tile is
// where a row sees its first token, if it sees any), and their row sums at the end.
// Each writes its half of P into the value MFMA's B-operand order.
//
// Value waves 4-7: wave 4 + v owns latent columns 128 v .. 128 v + 127 of all 64
// rows (Oᵀ: 4 column blocks x 2 row blocks of 32x32 fp32) on v_mfma_f32_32x32x16_bf16,
// with K = 16 tokens per k-step in their natural order, and issues a quarter of
// every tile's loads at the start of the step.
//
// The pipeline, the restart rule, the masking and the output are those of the
// role-split form: step i waits for tile i, passes the one barrier, issues tile i + 2
// into the buffer of tile i - 2, scores tile i and publishes its P into buffer i % 2,
// while the value waves run tile i - 1 from P buffer (i - 1) % 2.
template <int DR>
__global__ __launch_bounds__(512) void decode_pp_kernel(DecodeArgs a) {
  constexpr int ROW = 512 + DR, ROWB = ROW * 2;
  constexpr int KS = ROW / 32;                    // score k-steps (K = 32 each)
  constexpr int KS16 = ROW / 16;                  // k-steps of the Q_cat block order
  constexpr int TILE_BYTES = kTileT * ROWB;
  constexpr int LOADS = 8 + (DR == 64 ? 1 : 0);   // 1 KiB loads per value wave per tile
  constexpr int PBUF = 2 * 2 * 1024;              // P fragments [row block][k-step][lane]
  __shared__ __attribute__((aligned(1024))) char s_tile0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char s_tile1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char s_tile2[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char s_tile3[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char s_p[2 * PBUF];
  __shared__ float s_x[2][2][32];   // [row block][token half][row]: the first tile's row maxima
  __shared__ float s_ms[2][2][32];  // ... the range's largest scores (restart references)
  __shared__ float s_l[2][32];      // [row block][row]: row sums of token half 1
  __shared__ int s_flag[4];
  static_assert(4 * TILE_BYTES + 2 * PBUF + 2 * 4 * 32 * 4 + 2 * 32 * 4 + 16 <= 160 * 1024, "LDS");

  const int tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);  // wave index, uniform
  const bool scorer = w < 4;
  const int hgroups = (a.h * a.n_q) / 64;
  const int HB = a.h / 32;
  int u = blockIdx.x;
  if ((a.units & 7) == 0) u = (blockIdx.x & 7) * (a.units >> 3) + (blockIdx.x >> 3);
  StampRec stamp;
  if constexpr (kStamps) stamp.begin();
  const int pair = u / hgroups, hg = u - pair * hgroups;
  const WorkItem item = a.list[pair];
  if (item.b < 0) return;  // uniform: past the pairs of this launch
  const int b = item.b, kv = item.kv;
  int t_begin, t_end;
  range_tokens(item.s, kv, a.chunk, t_begin, t_end);
  if (t_begin >= t_end || kv < a.n_q) return;  // not listed by the plan
  const int n_tiles = (t_end - t_begin + kTileT - 1) / kTileT;
  const int bound = min(t_end - 1, kv - a.n_q);
  const int first_masked = bound - t_begin - (kTileT - 1) >= 0 ? (bound - t_begin - (kTileT - 1)) / kTileT + 1 : 0;
  const int64_t prow0 = static_cast<int64_t>(item.p) * a.n_q;
  auto tile_ptr = [&](auto kc) __attribute__((always_inline)) -> char* {
    constexpr int K = decltype(kc)::value;
    if constexpr (K == 0) return s_tile0;
    else if constexpr (K == 1) return s_tile1;
    else if constexpr (K == 2) return s_tile2;
    else return s_tile3;
  };

  auto run = [&](auto role) __attribute__((always_inline)) {
    constexpr bool SC = decltype(role)::value != 0;
    // ---------------- score-wave state
    const int rb = (w >> 1) & 1, th = w & 1;
    const int qb_own = 2 * hg + rb;
    const int j_own = qb_own / HB;
    const int vis_own = kv - a.n_q + j_own;
    u32x4 qf[SC ? 2 : 1][SC ? KS : 1];  // Q_cat of sub-blocks 0, 1 (B operand, K = 32)
    float m_ref[2] = {-INFINITY, -INFINITY}, m_seen[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
    uint64_t ovr = 0;
    // score A operand: token 16 th + l % 16, chunk 4 (ks % 2) + l / 16 of group ks / 2
    int sa_off[2];
    {
      const int t = 16 * th + (l & 15), sw = swz(t);
#pragma unroll
      for (int par = 0; par < 2; ++par) sa_off[par] = t * 128 + (((4 * par + (l >> 4)) ^ sw) << 4);
    }
    // ---------------- value-wave state
    const int vw = w & 3;
    f32x16 acc[SC ? 1 : 8];  // Oᵀ: acc[cb * 2 + rb], column block 4 vw + cb
    int pg_next = 0;
    uint32_t ld_adj[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = 8 * q + (l >> 3);
      ld_adj[q] = static_cast<uint32_t>(t * ROWB + (((l & 7) ^ swz(t)) << 4) - 1024 * q);
    }
    // value A operand (transposed reads), tokens in natural order: K index 8 h + e
    // (h = l / 32) of value k-step kk is token 16 kk + 8 h + e. 16-lane group g, lane i
    // reads row 8 (g / 2) + 4 sec + i / 4 and columns 16 (g % 2) + 4 (i % 4) of a
    // 32-column block (sec 0: e = 0..3, sec 1: e = 4..7).
    int va_off[2][2];
    {
      const int g = l >> 4, i = l & 15;
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) {
        const int t = 8 * (g >> 1) + 4 * sec + (i >> 2);
        const int sw = swz(t);
#pragma unroll
        for (int par = 0; par < 2; ++par) {
          const int low = 2 * (g & 1) + ((i & 3) >> 1);
          va_off[sec][par] = t * 128 + (((4 * par + low) ^ sw) << 4) + ((i & 1) << 3);
        }
      }
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
    // value wave vw loads column groups vw and vw + 4 whole (runs of four 1 KiB
    // blocks) and, with the RoPE key, block vw of group 8
    auto issue_tile = [&](int it, char* tile) __attribute__((always_inline)) {
      const u32x4 rsrc = tile_rsrc(it);
      const uint32_t base = lds_addr(tile);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int G = vw + 4 * r;
        dma_run<4>(rsrc, ld_adj, static_cast<uint32_t>(G * 128), base + G * 4096);
      }
      if constexpr (DR == 64)
        dma_run<1>(rsrc, ld_adj + vw, static_cast<uint32_t>(8 * 128 + 1024 * vw), base + 8 * 4096 + 1024 * vw);
    };

    constexpr int SDEPTH = 6;
    auto scores = [&](const char* tile, f32x4 (&sc)[2]) __attribute__((always_inline)) {
      u32x4 fa[SDEPTH];
      auto frag = [&](int ks) __attribute__((always_inline)) {
        return *(lds_u32x4*)(lds_ptr(tile) + sa_off[ks & 1] + (ks >> 1) * 4096);
      };
#pragma unroll
      for (int ks = 0; ks < SDEPTH; ++ks) fa[ks] = frag(ks);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          if (ks == 0) mfma16_first(sc[sb], fa[0], qf[sb][0]);
          else if (ks + 1 < KS) mfma16(sc[sb], fa[ks % SDEPTH], qf[sb][ks]);
          else mfma16_last(sc[sb], fa[ks % SDEPTH], qf[sb][ks]);
        }
        if (ks + SDEPTH < KS) fa[ks % SDEPTH] = frag(ks + SDEPTH);
      }
    };
    // rows of this lane: 16 sb + l % 16; reduce over the four lanes holding a row
    auto row_max = [&](float x) __attribute__((always_inline)) {
      x = fmaxf(x, __shfl_xor(x, 16));
      return fmaxf(x, __shfl_xor(x, 32));
    };
    auto row_sum = [&](float x) __attribute__((always_inline)) {
      x += __shfl_xor(x, 16);
      return x + __shfl_xor(x, 32);
    };
    auto pv = [&](const char* tile, const char* pbuf) __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 pb[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) pb[r] = *(lds_u32x4*)(lds_ptr(pbuf) + (r * 2 + kk) * 1024 + l * 16);
        i16x8 fr[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int gcb = 4 * vw + cb;
          lds_char* tb = lds_ptr(tile) + kk * 16 * 128 + (gcb >> 1) * 4096;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tb + va_off[0][gcb & 1]));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tb + va_off[1][gcb & 1]));
          fr[cb] = i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int r = 0; r < 2; ++r)
            acc[cb * 2 + r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fr[cb]), as_bf16x8(pb[r]),
                                                                      acc[cb * 2 + r], 0, 0, 0);
      }
    };
    auto vstep = [&](auto kc, auto first, int i, bool allow_restart) __attribute__((always_inline)) {
      constexpr int K = decltype(kc)::value;
      constexpr bool FIRST = decltype(first)::value != 0;
      if constexpr (!SC) {
        if (i + 1 < n_tiles) wait_vm<LOADS>();  // tile i has landed (tile i + 1 in flight)
        else wait_vm<0>();
        if constexpr (kStamps) stamp.mark(2);
      }
      lds_barrier();  // tile i and P of tile i - 1 everywhere; tile i - 2 is free
      if constexpr (kStamps) stamp.step();
      if constexpr (!SC) {
        if (i + 2 < n_tiles) issue_tile(i + 2, tile_ptr(Ic<(K + 2) % 4>{}));
        if constexpr (kStamps) stamp.mark(0);
        if constexpr (FIRST) {
          lds_barrier();  // the score waves' exchange of row maxima
        } else {
          pv(tile_ptr(Ic<(K + 3) % 4>{}), s_p + ((K + 1) & 1) * PBUF);
          if constexpr (kStamps) stamp.mark(1);
        }
      } else {
        f32x4 sc[2];
        scores(tile_ptr(kc), sc);
        if (i >= first_masked) {  // uniform
          const int lim = min(t_end - 1, vis_own);
          const int t0 = t_begin + i * kTileT + 16 * th + 4 * (l >> 4);
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) sc[sb][e] = t0 + e > lim ? -INFINITY : sc[sb][e];
        }
        float mx[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          mx[sb] = fmaxf(fmaxf(sc[sb][0], sc[sb][1]), fmaxf(sc[sb][2], sc[sb][3]));
          m_seen[sb] = fmaxf(m_seen[sb], mx[sb]);
        }
        if constexpr (kStamps) stamp.mark(0);
        if constexpr (FIRST) {
          // the row maxima of the range's first tile, over both token halves
          float rm[2];
#pragma unroll
          for (int sb = 0; sb < 2; ++sb) rm[sb] = row_max(mx[sb]);
          if (l < 16) {
            s_x[rb][th][l] = rm[0];
            s_x[rb][th][16 + l] = rm[1];
          }
          lds_barrier();
#pragma unroll
          for (int sb = 0; sb < 2; ++sb) {
            const float other = s_x[rb][th ^ 1][16 * sb + (l & 15)];
            if (m_ref[sb] == -INFINITY) m_ref[sb] = fmaxf(rm[sb], other);
          }
        }
        bool overrun = false;
        u32x2 pk[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          overrun |= allow_restart && mx[sb] > m_ref[sb] + kHeadroom;
          const float mref = m_ref[sb] == -INFINITY ? 0.f : m_ref[sb];
          const float p0 = fast_exp2(sc[sb][0] - mref), p1 = fast_exp2(sc[sb][1] - mref);
          const float p2 = fast_exp2(sc[sb][2] - mref), p3 = fast_exp2(sc[sb][3] - mref);
          pk[sb] = u32x2{pack_bf16x2(p0, p1), pack_bf16x2(p2, p3)};
          l_run[sb] += (p0 + p1) + (p2 + p3);
        }
        ovr |= __builtin_amdgcn_ballot_w64(overrun);
        // P[rb][k-step th][lane 16 sb + l % 16 + 32 (l / 32)][4 ((l / 16) % 2) + e]
        char* pd = s_p + (K & 1) * PBUF + (rb * 2 + th) * 1024 + ((l >> 5) * 32 + (l & 15)) * 16 + ((l >> 4) & 1) * 8;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) *(lds_u32x2*)(lds_ptr(pd) + sb * 16 * 16) = pk[sb];
        if constexpr (kStamps) stamp.mark(1);
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
      // Q_cat block order: column c of head-in-block hi at k-step c / 16, lane
      // hi + 32 ((c / 8) % 2), element c % 8; this lane's fragment of k-step ks,
      // sub-block sb: head-in-block 16 sb + l % 16, columns 32 ks + 8 (l / 16) + 0..7.
      // The compiler's wait before each fragment's first use lets the first score
      // chain start while later fragments still arrive.
      const u32x4* qp = reinterpret_cast<const u32x4*>(a.q_cat) +
                        (static_cast<int64_t>(b) * a.n_q * HB + qb_own) * KS16 * 64 + (l >> 5) * 64 + (l & 15) +
                        32 * ((l >> 4) & 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) qf[sb][ks] = qp[ks * 128 + 16 * sb];
    }
    for (int pass = 0;; ++pass) {
      const bool allow_restart = pass < kMaxRestarts;
      if constexpr (!SC) {
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = f32x16{};
      }
      l_run[0] = l_run[1] = 0.f;
      ovr = 0;
      if (pass > 0) prologue();
      vstep(Ic<0>{}, Ic<1>{}, 0, allow_restart);
      for (int i = 1; i < n_tiles; i += 4) {
#define MLA_PSTEP(KK, D) \
  if (i + D < n_tiles) vstep(Ic<KK>{}, Ic<0>{}, i + D, allow_restart);
        MLA_PSTEP(1, 0)
        MLA_PSTEP(2, 1)
        MLA_PSTEP(3, 2)
        MLA_PSTEP(0, 3)
#undef MLA_PSTEP
      }
      float ms[2] = {0.f, 0.f};
      if constexpr (SC) {
        if (l == 0) s_flag[w] = ovr != 0;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) ms[sb] = row_max(m_seen[sb]);
        if (l < 16) {
          s_ms[rb][th][l] = ms[0];
          s_ms[rb][th][16 + l] = ms[1];
        }
      }
      lds_barrier();  // P of the last tile, every flag and the score waves' m_seen
      const bool restart = (s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3]) != 0;  // uniform
      if (!restart) {
        if constexpr (!SC) {
          const int kl = (n_tiles - 1) & 3;
          const char* lt = kl == 0 ? s_tile0 : kl == 1 ? s_tile1 : kl == 2 ? s_tile2 : s_tile3;
          pv(lt, s_p + ((n_tiles - 1) & 1) * PBUF);
        }
        if constexpr (kStamps) stamp.loop_end();
        break;
      }
      // restart the range with the largest score of each row as its reference
      if constexpr (SC) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          m_ref[sb] = fmaxf(ms[sb], s_ms[rb][th ^ 1][16 * sb + (l & 15)]);
          m_seen[sb] = -INFINITY;
        }
      } else {
        wait_vm<0>();
      }
      lds_barrier();  // every wave's reads of the flags and maxima are done
    }

    // ---- epilogue: value waves store their columns of the partial O (fp32, straight
    //      from the accumulators); the score waves of token half 1 hand their row sums
    //      to those of half 0, which store (m, l)
    float ls[2] = {0.f, 0.f};
    if constexpr (SC) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) ls[sb] = row_sum(l_run[sb]);
      if (th == 1 && l < 16) {
        s_l[rb][l] = ls[0];
        s_l[rb][16 + l] = ls[1];
      }
    }
    lds_barrier();
    if constexpr (!SC) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int qb = 2 * hg + r, j = qb / HB;
        const int head = 32 * (qb - j * HB) + (l & 31);
        float* dst = a.o_part + ((prow0 + j) * a.h + head) * 512 + 128 * vw + 4 * (l >> 5);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const f32x16& o = acc[cb * 2 + r];
            *reinterpret_cast<f32x4*>(dst + 32 * cb + 8 * v4) = f32x4{o[4 * v4], o[4 * v4 + 1], o[4 * v4 + 2], o[4 * v4 + 3]};
          }
      }
    } else {
      if (th == 0 && l < 16) {
        const int hb = qb_own - j_own * HB;
        float* ml = a.ml_part + ((prow0 + j_own) * a.h + 32 * hb + l) * 2;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          ml[32 * sb + 0] = m_ref[sb];
          ml[32 * sb + 1] = ls[sb] + s_l[rb][16 * sb + l];
        }
      }
    }
  };
  if (scorer) run(Ic<1>{});
  else run(Ic<0>{});
  if constexpr (kStamps) stamp.end(a.stamps, u, w, l);
}

#ifdef MLA_STAMPS
__device__ uint64_t stamp_buf[kStampUnits * kStampWaves * kStampSlots];
#endif

hipError_t launch_decode_bf16(const DecodeArgs& a_in, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  DecodeArgs a = a_in;
#ifdef MLA_STAMPS
  if (hipGetSymbolAddress(reinterpret_cast<void**>(&a.stamps), HIP_SYMBOL(stamp_buf)) != hipSuccess)
    return hipErrorInvalidSymbol;
#endif
  // hipExtLaunchKernelGGL stamps ev0/ev1 from the dispatch itself, so an event pair
  // brackets exactly this kernel's execution (null events: plain launch).
  const int rows = a.h * a.n_q;
  const int R = a.form == kForm128 ? 128 : 64;
  if (rows % R != 0 || a.h % 32 != 0 || a.units <= 0) return hipErrorInvalidValue;
  if (a.form == kFormPrecise && a.q_lo == nullptr) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(a.units));
#define MLA_LAUNCH(K) hipExtLaunchKernelGGL(K, grid, dim3(256), 0, s, ev0, ev1, 0, a)
  if (a.form == kForm128) {
    if (a.d_r == 64) MLA_LAUNCH((decode_kernel<4, 64>));
    else if (a.d_r == 0) MLA_LAUNCH((decode_kernel<4, 0>));
    else return hipErrorInvalidValue;
  } else if (a.form == kFormRoles) {
    if (a.d_r == 64) MLA_LAUNCH((decode_roles_kernel<64, false>));
    else if (a.d_r == 0) MLA_LAUNCH((decode_roles_kernel<0, false>));
    else return hipErrorInvalidValue;
  } else if (a.form == kFormPingPong) {
    if (a.d_r == 64) hipExtLaunchKernelGGL((decode_pp_kernel<64>), grid, dim3(512), 0, s, ev0, ev1, 0, a);
    else if (a.d_r == 0) hipExtLaunchKernelGGL((decode_pp_kernel<0>), grid, dim3(512), 0, s, ev0, ev1, 0, a);
    else return hipErrorInvalidValue;
  } else if (a.form == kFormPrecise) {
    if (a.d_r == 64) MLA_LAUNCH((decode_roles_kernel<64, true>));
    else if (a.d_r == 0) MLA_LAUNCH((decode_roles_kernel<0, true>));
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
#undef MLA_LAUNCH
  return hipGetLastError();
}

hipError_t launch_decode_mixed_bf16(const DecodeArgs& fast, const WorkItem* prec_list, int prec_chunk,
                                    int prec_units, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if (fast.form != kForm128 || fast.q_lo == nullptr || prec_list == nullptr) return hipErrorInvalidValue;
  if ((fast.h * fast.n_q) % 128 != 0 || fast.h % 32 != 0) return hipErrorInvalidValue;
  if (fast.units <= 0 || fast.units % 8 != 0 || prec_units <= 0 || prec_chunk <= 0 ||
      static_cast<int64_t>(fast.units) + prec_units > INT32_MAX)
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(fast.units + prec_units));
#define MLA_LAUNCH(K) hipExtLaunchKernelGGL(K, grid, dim3(256), 0, s, ev0, ev1, 0, fast, prec_list, prec_chunk, prec_units)
  if (fast.d_r == 64) MLA_LAUNCH(decode_mixed_kernel<64>);
  else if (fast.d_r == 0) MLA_LAUNCH(decode_mixed_kernel<0>);
  else return hipErrorInvalidValue;
#undef MLA_LAUNCH
  return hipGetLastError();
}

}  // namespace mla

#ifdef MLA_STAMPS
// Instrumented builds only: the device address and size of the stamp buffer (see
// StampRec). Returns 0, or -1 if the address cannot be looked up.
extern "C" int32_t mla_stamps_buffer(void** ptr, size_t* bytes) {
  if (!ptr || !bytes) return -1;
  *bytes = sizeof(mla::stamp_buf);
  return hipGetSymbolAddress(ptr, HIP_SYMBOL(mla::stamp_buf)) == hipSuccess ? 0 : -1;
}
#endif
