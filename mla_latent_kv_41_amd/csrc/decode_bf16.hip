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
// Work split inside the workgroup (NW waves, one per SIMD):
//   scores: wave w owns rows [32w, 32w+32): its Q_cat fragments stay in VGPRs.
//   values: wave w owns latent columns [w*512/NW, (w+1)*512/NW) for all R rows, so
//           the Oᵀ accumulators (512 x R fp32 / NW waves = 256 registers per lane)
//           never need a cross-wave reduction; P goes through LDS.
// Tiles are double-buffered: the next tile's direct-to-LDS loads are in flight
// while the current one is consumed.
//
// LDS tile layout: the 576 (or 512) columns are cut into groups of 64 (128 bytes,
// eight 16-byte chunks); group G holds all 32 rows, row t at G*4096 + t*128, and
// chunk k of the group at position k ^ swz(t), swz(t) = ((u & 1) << 2) | (u >> 1)
// with u = (t >> 1) & 7. The 16-row column reads of the score operand and the
// 4-row transposed reads of the value operand are then free of bank conflicts,
// and each 1 KiB wave load (8 rows x one group) has a per-lane offset that takes
// only two values.
//
// Softmax state is kept in base-2 units (Q_cat carries scale * log2 e). The
// running max is raised only when a score exceeds it by more than TAU = 8, so the
// accumulators are rescaled rarely (exact either way: P <= 2^8 stays in range).
//
// Output per (b, split): Oᵀ (unnormalised) and (m, l) in fp32; the combine kernel
// merges splits.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int kTileT = 32;        // tokens per tile
constexpr float kTau = 8.0f;      // lazy-rescale threshold (base-2 units)
constexpr int kPStride = 80;      // bytes per P row in LDS: 32 bf16 + 16 B pad

__device__ __forceinline__ int swz(int t) {
  const int u = (t >> 1) & 7;
  return ((u & 1) << 2) | (u >> 1);
}

template <int NW, int DR>
struct Cfg {
  static constexpr int ROW = 512 + DR;                  // elements per cache row
  static constexpr int ROWB = ROW * 2;                  // bytes per cache row
  static constexpr int CH = ROW / 8;                    // 16-byte chunks per row
  static constexpr int KS = ROW / 16;                   // score k-steps (K=16 each)
  static constexpr int R = 32 * NW;                     // query rows per workgroup
  static constexpr int CB = 512 / (32 * NW);            // value column blocks per wave
  static constexpr int TILE_BYTES = kTileT * ROWB;
  static constexpr int GROUPS = CH / 8;                 // 128-byte column groups
  static constexpr int LOADS = (kTileT * CH) / (64 * NW);  // 16-B loads per lane per tile
  static constexpr int P_BYTES = R * kPStride;
};

}  // namespace

// Multiply one accumulator element in place, keeping it in its AGPR (a VALU op
// on the accumulators would otherwise pull the whole array into VGPRs).
__device__ __forceinline__ float scale_acc(float x, float s) {
  float tmp;
  asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
               : "+a"(x), "=&v"(tmp)
               : "v"(s));
  return x;
}

template <int V>
struct Ic {
  static constexpr int value = V;
};

template <int NW, int DR>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  using C = Cfg<NW, DR>;
  // Two tile buffers as distinct arrays: reads of one are provably independent of
  // the direct-to-LDS loads landing in the other, so they need no load wait.
  __shared__ __attribute__((aligned(1024))) char s_tile0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char s_tile1[C::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char s_p[C::P_BYTES];
  __shared__ float s_alpha[C::R];
  __shared__ int s_flag[2];

  const int tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);  // wave index, uniform
  const int hgroups = (a.h * a.n_q) / C::R;
  const int units = a.batch * a.n_splits * hgroups;

  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous
  // range of units so one sequence's splits share an L2.
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
  // this lane's score row (Q_cat / softmax state), r = 32w + l%32
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
  auto issue_tile = [&](int it, char* tile) {
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
  // value A operand (transposed reads): 16-lane group g, lane i; rows
  // 8(g/2) + i/4 (+4), columns 16(g%2) + 4(i%4) of a 32-column block, i.e. chunk
  // 4(blk%2) + 2(g%2) + (i%4)/2 of group blk/2, half (i%2)
  int va_off[2][2];
  {
    const int g = l >> 4, i = l & 15;
#pragma unroll
    for (int sec = 0; sec < 2; ++sec) {
      const int t = 8 * (g >> 1) + (i >> 2) + 4 * sec;
      const int sw = swz(t);
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const int low = 2 * (g & 1) + ((i & 3) >> 1);  // chunk within the 4-chunk half group
        va_off[sec][par] = t * 128 + (((4 * par + low) ^ sw) << 4) + ((i & 1) << 3);
      }
    }
  }
  const int colw = w * (512 / NW);  // this wave's first latent column
  // P reads (B operand of the value MFMA): row 32rb + l%32, tokens 16kk + 8(l/32)
  const int pb_off = (l & 31) * kPStride + ((l >> 5) << 4);

  f32x16 acc[C::CB][NW];
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
    for (int rb = 0; rb < NW; ++rb) acc[cb][rb] = f32x16{};

  float m_run = -INFINITY, l_run = 0.f;
  if (tid < 2) s_flag[tid] = 0;

  auto step = [&](auto bufc, int it) {
    constexpr int BUF = decltype(bufc)::value;
    char* tile = BUF == 0 ? s_tile0 : s_tile1;
    char* other = BUF == 0 ? s_tile1 : s_tile0;
    const int t0 = t_begin + it * kTileT;
    __builtin_amdgcn_s_waitcnt(0);  // this lane's loads of this tile have landed
    __syncthreads();                // everyone's have; PV(it-1) finished everywhere
    if (it + 1 < n_tiles) issue_tile(it + 1, other);
    if (tid == 0) s_flag[(it + 1) & 1] = 0;

    // ---- scores: Sᵀ[32 tokens][32 rows of this wave], four fragments in flight
    f32x16 sc = {};
    {
      u32x4 fa[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) fa[kk] = *(lds_u32x4*)(lds_ptr(tile) + sa_off[kk]);  // group 0
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[ks & 3]), as_bf16x8(qf[ks]), sc, 0, 0, 0);
        if (ks + 4 < C::KS) fa[ks & 3] = *(lds_u32x4*)(lds_ptr(tile) + sa_off[ks & 3] + ((ks + 4) >> 2) * 4096);
      }
    }

    // ---- mask tokens past the range or (for multi-token decode) in this row's future
    const int lim = min(t_end - 1, vis_own);  // last token this row may see
    if (t0 + kTileT - 1 > min(t_end - 1, kv - a.n_q)) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int tok = t0 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
        if (tok > lim) sc[v] = -INFINITY;
      }
    }

    // ---- online softmax for row r_own (lanes l and l^32 hold the same row)
    float mx = sc[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sc[v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float alpha = 1.f;
    int need = 0;
    if (mx > m_run + kTau) {
      alpha = fast_exp2(m_run - mx);  // 0 when m_run = -inf
      need = m_run > -INFINITY;
      m_run = mx;
    }
    const float mref = m_run == -INFINITY ? 0.f : m_run;
    float psum = 0.f;
    uint32_t pk[8];
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const float p0 = fast_exp2(sc[v] - mref), p1 = fast_exp2(sc[v + 1] - mref);
      psum += p0 + p1;
      pk[v / 2] = pack_bf16x2(p0, p1);
    }
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;

    // P[r][t] in LDS: lane holds tokens 8i + 4(l/32) + 0..3 for i = 0..3
    {
      lds_char* prow = lds_ptr(s_p) + r_own * kPStride + (l >> 5) * 8;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        u32x2 v2 = {pk[2 * i4], pk[2 * i4 + 1]};
        *(lds_u32x2*)(prow + i4 * 16) = v2;
      }
    }
    if (l < 32) s_alpha[r_own] = alpha;
    if (need) s_flag[it & 1] = 1;
    __syncthreads();

    // ---- rescale the accumulators if any row raised its max (rare)
    if (s_flag[it & 1]) {
#pragma unroll
      for (int rb = 0; rb < NW; ++rb) {
        const float al = s_alpha[32 * rb + (l & 31)];
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[cb][rb][v] = scale_acc(acc[cb][rb][v], al);
      }
    }

    // ---- values: Oᵀ[c][r] += Σ_t Cᵀ[c][t] · Pᵀ[t][r]
    lds_char* pbase = lds_ptr(s_p) + pb_off;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 bfr[NW];
#pragma unroll
      for (int rb = 0; rb < NW; ++rb) bfr[rb] = *(lds_u32x4*)(pbase + rb * 32 * kPStride + kk * 32);
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb) {
        const int cblk = (colw >> 5) + cb;  // 32-column block index within the row
        lds_char* tb = lds_ptr(tile) + kk * 16 * 128 + (cblk >> 1) * 4096;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tb + va_off[0][cblk & 1]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tb + va_off[1][cblk & 1]));
        const i16x8 af = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int rb = 0; rb < NW; ++rb)
          acc[cb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af),
                                                               as_bf16x8(bfr[rb]), acc[cb][rb], 0, 0, 0);
      }
    }
  };

  issue_tile(0, s_tile0);
  for (int it = 0; it < n_tiles; it += 2) {
    step(Ic<0>{}, it);
    if (it + 1 < n_tiles) step(Ic<1>{}, it + 1);
  }

  // ---- write partials: Oᵀ block (cb, rb): lane col r = 32rb + l%32,
  //      rows c = colw + 32cb + 8(v/4) + 4(l/32) + v%4
  const int64_t part_row0 = (static_cast<int64_t>(b) * a.n_splits + s) * a.n_q;
#pragma unroll
  for (int rb = 0; rb < NW; ++rb) {
    const int r = 32 * rb + (l & 31);
    const int j = r / HG, head = hg * HG + r % HG;
    float* orow = a.o_part + ((part_row0 + j) * a.h + head) * 512 + colw + 4 * (l >> 5);
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        f32x4 o = {acc[cb][rb][4 * v4], acc[cb][rb][4 * v4 + 1], acc[cb][rb][4 * v4 + 2], acc[cb][rb][4 * v4 + 3]};
        *reinterpret_cast<f32x4*>(orow + 32 * cb + 8 * v4) = o;
      }
  }
  if (l < 32) {
    float* ml = a.ml_part + ((part_row0 + j_own) * a.h + head_own) * 2;
    ml[0] = m_run;
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
