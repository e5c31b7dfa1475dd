// Per-CU rates of the gfx950 units the attention kernels lean on, measured with the
// shader clock (s_memtime) inside each wave over 256 workgroups (one per CU):
//
//   lds      ds_read_b128, each wave reading contiguous 1 KiB blocks of a 64 KiB LDS array
//   mfma16   v_mfma_f32_16x16x32_bf16, four independent accumulators per wave
//   mfma32   v_mfma_f32_32x32x16_bf16, four independent accumulators per wave
//   vload    global_load_dwordx4 into VGPRs (1 KiB per wave instruction) from a
//            64 KiB buffer that stays in L2 after the first pass, 8 loads in flight
//   dmaload  buffer_load_dwordx4 ... lds (direct-to-LDS, 1 KiB per wave instruction)
//            from the same kind of buffer into 16 KiB of LDS per wave: the cycles a
//            wave spends issuing them, and until all have landed
//   score    ds_read_b128 of the attention kernels' score operand from a cache tile
//            in their LDS layout (32 rows of 128-byte column groups, 16-byte chunk k
//            of row t at position k ^ ((t >> 1) & 7)): 32 rows x one chunk per half
//            wave (128-row and role-split forms), 16 rows x two chunks (eight-wave
//            form), and the eight-wave reads under the pair-interleaved permutation
//            p(u) = ((u & 1) << 2) | (u >> 1), u = (t >> 1) & 7, for comparison
//   stream   chip-wide HBM read rate of direct-to-LDS loads shaped like the tile
//            loads (8 rows x 128 bytes at a 1152-byte row stride), four waves per
//            workgroup each keeping W loads in flight, over 2 GiB
//   sched    the eight-wave attention kernel's load schedule on the DeepSeek shape
//            without its compute: 256 workgroups; units 2p and 2p + 1 (one XCD) read
//            the same 32 tiles of 36 KiB (as the two 64-row head groups of one
//            sequence range do), or distinct ones; four waves issue a tile's 36
//            loads at each step, spin C cycles, wait for the previous tile, then a
//            barrier. Launches rotate over three copies of the data (as the
//            benchmark rotates caches), so the Infinity Cache does not hold them.
//            Variants: the odd unit of each pair reads the shared tiles in an order
//            rotated by `rot` tiles (so the two do not fetch the same lines at the
//            same time), and D = 3 issues three tiles ahead instead of two.
//
// Rates are bytes or FLOPs per cycle per CU, taken from the slowest wave of each
// launch. Every kernel holds at least 96 KiB of LDS, so no CU runs two of the 256
// workgroups. Every access stays inside its array or buffer (offsets are masked to
// the sizes below); the buffer loads carry a 64 KiB size bound as well.
//
//   hipcc --offload-arch=gfx950 -O3 rates.hip -o rates && ./rates   (./rates s: the sched lines only)
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <algorithm>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

#define CHECK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                 \
      exit(1);                                                                \
    }                                                                         \
  } while (0)

constexpr int kBlocks = 256;
constexpr int kPadLds = 96 * 1024;  // LDS held by the kernels that need less

// keeps a kernel's LDS reservation (the store never runs: iters is positive)
#define HOLD_LDS()                                         \
  __shared__ char hold_[kPadLds];                          \
  if (iters < 0) hold_[threadIdx.x] = static_cast<char>(iters)

template <int S>
__device__ __forceinline__ int tile_perm(int t) {
  const int u = (t >> 1) & 7;
  return S == 0 ? u : (((u & 1) << 2) | (u >> 1));
}

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void lds_read(uint64_t* cyc, u32x4* sink, int iters) {
  __shared__ u32x4 buf[6144];  // 96 KiB, the first 64 read
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  for (int k = tid; k < 4096; k += WAVES * 64) buf[k] = u32x4{(uint32_t)k, 1u, 2u, 3u};
  __syncthreads();
  u32x4 acc = {0u, 0u, 0u, 0u};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) acc ^= buf[((it * 8 + r + w * 5) & 63) * 64 + l];
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  if (l == 0) cyc[blockIdx.x * WAVES + w] = t1 - t0;
  sink[blockIdx.x * WAVES * 64 + tid] = acc;
}

template <int WAVES, int KIND>
__global__ __launch_bounds__(WAVES * 64) void mfma_rate(uint64_t* cyc, float* sink, int iters) {
  HOLD_LDS();
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const u32x4 a = {(uint32_t)tid, 2u, 3u, 4u}, b = {5u, (uint32_t)l, 7u, 8u};
  const bf16x8 av = __builtin_bit_cast(bf16x8, a), bv = __builtin_bit_cast(bf16x8, b);
  float out;
  asm volatile("s_nop 4" ::: "memory");  // operands written by VALU settle before the first MFMA
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  // issued from asm so that the loop is the four MFMAs and its counter alone (left to
  // itself, the compiler copies accumulators between iterations); each accumulator is
  // read again three MFMAs after it was written
  if constexpr (KIND == 0) {
    f32x4 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
      asm volatile(
          "v_mfma_f32_16x16x32_bf16 %0, %4, %5, %0\n\t"
          "v_mfma_f32_16x16x32_bf16 %1, %4, %5, %1\n\t"
          "v_mfma_f32_16x16x32_bf16 %2, %4, %5, %2\n\t"
          "v_mfma_f32_16x16x32_bf16 %3, %4, %5, %3"
          : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3)
          : "v"(av), "v"(bv));
    }
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");  // results settle before VALU reads
    out = c0[0] + c1[1] + c2[2] + c3[3];
  } else {
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
      asm volatile(
          "v_mfma_f32_32x32x16_bf16 %0, %4, %5, %0\n\t"
          "v_mfma_f32_32x32x16_bf16 %1, %4, %5, %1\n\t"
          "v_mfma_f32_32x32x16_bf16 %2, %4, %5, %2\n\t"
          "v_mfma_f32_32x32x16_bf16 %3, %4, %5, %3"
          : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3)
          : "v"(av), "v"(bv));
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    out = c0[0] + c1[5] + c2[9] + c3[13];
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  if (l == 0) cyc[blockIdx.x * WAVES + w] = t1 - t0;
  sink[blockIdx.x * WAVES * 64 + tid] = out;
}

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void vload_rate(uint64_t* cyc, const u32x4* src, int iters) {
  HOLD_LDS();
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  u32x4 acc = {0u, 0u, 0u, 0u};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; it += 8) {
    u32x4 v[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] = __builtin_nontemporal_load(src + ((((it + r) * 7 + w * 3) & 63) * 64 + l));
#pragma unroll
    for (int r = 0; r < 8; ++r) acc ^= v[r];
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  if (l == 0) cyc[blockIdx.x * WAVES + w] = t1 - t0;
  if (acc[0] == 0x12345678u && acc[1] == 0x9abcdef0u) cyc[0] = 0;  // keeps the loads
}

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void dma_rate(uint64_t* cyc, const u32x4* src, int iters) {
  __shared__ u32x4 buf[WAVES < 6 ? 6144 : WAVES * 1024];  // 16 KiB per wave, at least 96 KiB
  const int tid = threadIdx.x, l = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint64_t ba = reinterpret_cast<uint64_t>(src);
  const u32x4 rsrc = {static_cast<uint32_t>(ba), static_cast<uint32_t>(ba >> 32) & 0xFFFFu, 65536u, 0x00020000u};
  const uint32_t lbase =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)(buf + w * 1024)));
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    uint32_t m = lbase + (it & 15) * 1024;  // lane l's 16 bytes land at m + 16 l
    const uint32_t voff = l * 16 + ((it * 7 + w * 3) & 63) * 1024;
    asm volatile("" : "+s"(m));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m), "v"(voff), "s"(rsrc)
                 : "m0");
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const uint64_t t2 = __builtin_amdgcn_s_memtime();
  if (l == 0) {
    cyc[(blockIdx.x * WAVES + w) * 2] = t1 - t0;
    cyc[(blockIdx.x * WAVES + w) * 2 + 1] = t2 - t0;
  }
}

// score-operand reads: KIND 0 = 32 rows x one chunk per half wave, 1 = 16 rows x two
// chunks per half wave (wave w takes rows 16 (w % 2) ..); S selects the permutation
template <int KIND, int S>
__global__ __launch_bounds__(512) void score_read(uint64_t* cyc, u32x4* sink, int iters) {
  __shared__ __attribute__((aligned(1024))) char tile[kPadLds];  // groups of 4 KiB
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  for (int k = tid; k < kPadLds / 16; k += 512) reinterpret_cast<u32x4*>(tile)[k] = u32x4{(uint32_t)k, 1u, 2u, 3u};
  __syncthreads();
  int off[4];
  if constexpr (KIND == 0) {
    const int t = l & 31;
#pragma unroll
    for (int q = 0; q < 4; ++q) off[q] = t * 128 + (((2 * q + (l >> 5)) ^ tile_perm<S>(t)) << 4);
  } else {
    const int t = 16 * (w & 1) + (l & 15);
#pragma unroll
    for (int q = 0; q < 4; ++q) off[q] = t * 128 + (((4 * (q & 1) + (l >> 4)) ^ tile_perm<S>(t)) << 4);
  }
  u32x4 acc = {0u, 0u, 0u, 0u};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    asm volatile("" : "+v"(off[0]), "+v"(off[1]), "+v"(off[2]), "+v"(off[3]));  // no hoisting
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const u32x4 v = *(lds_u32x4*)((lds_char*)tile + (r >> 2) * 8192 + off[r & 3]);
      acc[r & 3] += v[0] ^ v[3];
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  if (l == 0) cyc[blockIdx.x * 8 + w] = t1 - t0;
  sink[blockIdx.x * 512 + tid] = acc;
}

// direct-to-LDS load of 1 KiB: lane l's 16 bytes at buffer offset voff land at M0 + 16 l
__device__ __forceinline__ void dma_1k(const u32x4& rsrc, uint32_t voff, uint32_t lds) {
  uint32_t m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("" : "+s"(m));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m), "v"(voff), "s"(rsrc)
               : "m0");
}
// buffer offset of lane l in load r (0 .. 35) of tile `tile`: rows 8 (r % 4) + l / 8,
// column group r / 4, chunk l % 8
// a one-dword direct-to-LDS load per lane (64 lines per wave instruction): an L2
// prefetch whose data lands in a sink nothing reads
__device__ __forceinline__ void dma_4b(const u32x4& rsrc, uint32_t voff, uint32_t lds) {
  uint32_t m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("" : "+s"(m));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m), "v"(voff), "s"(rsrc)
               : "m0");
}
__device__ __forceinline__ uint32_t tile_off(int tile, int r, int l) {
  return static_cast<uint32_t>(tile) * 36864u + (8 * (r % 4) + (l >> 3)) * 1152u + (r / 4) * 128u + (l & 7) * 16u;
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

constexpr int64_t kTileBytes = 36864;                       // 32 rows x 1152 bytes
constexpr int64_t kStreamPerWg = (8ll << 20) / kTileBytes * kTileBytes;  // whole tiles in 8 MiB
constexpr int64_t kRangeBytes = 32 * kTileBytes;            // one range: 32 tiles

template <int W>
__global__ __launch_bounds__(256) void stream_rate(const char* src) {
  __shared__ __attribute__((aligned(1024))) char ring[kPadLds];
  const int l = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint64_t ba = reinterpret_cast<uint64_t>(src + blockIdx.x * kStreamPerWg);
  const u32x4 rsrc = {static_cast<uint32_t>(ba), static_cast<uint32_t>(ba >> 32) & 0xFFFFu,
                      static_cast<uint32_t>(kStreamPerWg), 0x00020000u};
  const uint32_t lbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char*)ring)) + w * 16384;
  const int loads = static_cast<int>(kStreamPerWg / 1024 / 4);
  for (int it = 0; it < loads; ++it) {
    const int k = it * 4 + w;
    dma_1k(rsrc, tile_off(k / 36, k % 36, l), lbase + (it & 15) * 1024);
    wait_vm<W>();
  }
  wait_vm<0>();
}

template <int D, int PF>
__global__ __launch_bounds__(512) void sched_rate(const char* src, int C, int share, int rot, uint64_t* rec) {
  __shared__ __attribute__((aligned(1024))) char tiles[4 * kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sink[4 * 256];
  const int l = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int u = (blockIdx.x & 7) * 32 + (blockIdx.x >> 3);  // contiguous units per XCD
  const uint64_t ba = reinterpret_cast<uint64_t>(src + (share ? u / 2 : u) * kRangeBytes);
  const u32x4 rsrc = {static_cast<uint32_t>(ba), static_cast<uint32_t>(ba >> 32) & 0xFFFFu,
                      static_cast<uint32_t>(kRangeBytes), 0x00020000u};
  const bool loader = w >= 4;
  const int lw = w - 4;
  const int r0 = (u & 1) ? rot : 0;  // the odd unit of a pair starts rot tiles in
  auto issue = [&](int it) {
    const uint32_t tb = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char*)tiles)) + (it & 3) * kTileBytes;
    const int pt = (it + r0) & 31;
#pragma unroll
    for (int k = 0; k < 9; ++k) dma_1k(rsrc, tile_off(pt, 9 * lw + k, l), tb + (9 * lw + k) * 1024);
  };
  // PF > 0: with the tile loads of step i, each unit of the pair also touches its half
  // of the lines (rows 16 (u & 1) .. + 15, all nine 128-byte groups) of tile
  // i + D + PF, one dword per line: lane j < 36 of loader wave lw takes line
  // 36 lw + j, the other lanes repeat line 36 lw
  auto prefetch = [&](int it) {
    const int pt = min(it, 31);
    const int q = 36 * lw + (l < 36 ? l : 0);
    const uint32_t off = static_cast<uint32_t>(pt) * 36864u + static_cast<uint32_t>(16 * (u & 1) + q / 9) * 1152u +
                         static_cast<uint32_t>(q % 9) * 128u;
    const uint32_t sb = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char*)sink)) + lw * 256;
    dma_4b(rsrc, off, sb);
  };
  // D tiles ahead: at step i the loads of tile i + D go into the buffer of tile
  // i + D - 4 (the kernel's form is D = 2; D = 3 keeps a third tile in flight)
  if (loader) {
    for (int k = 0; k < D; ++k) issue(k);
    wait_vm<9 * (D - 1)>();
  }
  __syncthreads();
  uint64_t steps = 0, issued = 0;
  for (int i = 0; i < 32; ++i) {
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    if (loader) {
      if (i + D < 32) {
        issue(i + D);
        if constexpr (PF > 0) prefetch(i + D + PF);
      }
      const uint64_t t1 = __builtin_amdgcn_s_memtime();
      issued += t1 - t0;
      while (__builtin_amdgcn_s_memtime() - t1 < static_cast<uint64_t>(C)) {
      }
      // loads younger than tile i + 1 that may stay in flight (a prefetch follows each
      // tile's loads)
      constexpr int P = PF > 0 ? 1 : 0;
      if (i + D < 32) wait_vm<9 * (D - 1) + P * D>();
      else if (D == 3 && i + 2 < 32) wait_vm<9 + P * 2>();
      else if (i + 1 < 32 && P) wait_vm<P * (D - 1)>();
      else wait_vm<0>();
    }
    __syncthreads();
    steps += __builtin_amdgcn_s_memtime() - t0;
  }
  if (threadIdx.x == 256) {
    rec[blockIdx.x * 2] = steps;
    rec[blockIdx.x * 2 + 1] = issued;
  }
}

// slowest and mean of n per-wave cycle counts (stride apart, from offset off)
static void stats(const uint64_t* h, int n, int stride, int off, double* mx, double* mean) {
  *mx = 0;
  *mean = 0;
  for (int k = 0; k < n; ++k) {
    const double v = static_cast<double>(h[k * stride + off]);
    *mean += v;
    if (v > *mx) *mx = v;
  }
  *mean /= n;
}

template <typename S>
static void run(const char* name, void (*kern)(uint64_t*, S*, int), int waves, int iters, double units_per_iter,
                const char* unit) {
  uint64_t* cyc;
  S* sink;
  CHECK(hipMalloc(&cyc, kBlocks * waves * 8));
  CHECK(hipMalloc(&sink, kBlocks * waves * 64 * sizeof(S)));
  for (int rep = 0; rep < 3; ++rep) kern<<<kBlocks, waves * 64>>>(cyc, sink, iters);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  uint64_t* h = static_cast<uint64_t*>(malloc(kBlocks * waves * 8));
  CHECK(hipMemcpy(h, cyc, kBlocks * waves * 8, hipMemcpyDeviceToHost));
  double mx, mean;
  stats(h, kBlocks * waves, 1, 0, &mx, &mean);
  const double rate = units_per_iter * iters * waves / mx;
  printf("%-8s %2d waves: %.1f %s per cycle per CU (mean %.0f cycles per wave)", name, waves, rate, unit, mean);
  // dense bf16 MFMA peak: 4 SIMDs x 1024 FLOP per cycle
  if (unit[0] == 'F') printf(", %.1f%% of 4096", 100.0 * rate / 4096.0);
  printf("\n");
  free(h);
  CHECK(hipFree(cyc));
  CHECK(hipFree(sink));
}

template <int WAVES>
static void run_vload(int iters) {
  uint64_t* cyc;
  u32x4* src;
  CHECK(hipMalloc(&cyc, kBlocks * WAVES * 8));
  CHECK(hipMalloc(&src, 65536));
  CHECK(hipMemset(src, 1, 65536));
  for (int rep = 0; rep < 3; ++rep) vload_rate<WAVES><<<kBlocks, WAVES * 64>>>(cyc, src, iters);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  uint64_t* h = static_cast<uint64_t*>(malloc(kBlocks * WAVES * 8));
  CHECK(hipMemcpy(h, cyc, kBlocks * WAVES * 8, hipMemcpyDeviceToHost));
  double mx, mean;
  stats(h, kBlocks * WAVES, 1, 0, &mx, &mean);
  printf("vload    %2d waves: %.1f B per cycle per CU (mean %.0f cycles per wave)\n", WAVES, 1024.0 * iters * WAVES / mx,
         mean);
  free(h);
  CHECK(hipFree(cyc));
  CHECK(hipFree(src));
}

template <int WAVES>
static void run_dma(int iters) {
  uint64_t* cyc;
  u32x4* src;
  CHECK(hipMalloc(&cyc, kBlocks * WAVES * 16));
  CHECK(hipMalloc(&src, 65536));
  CHECK(hipMemset(src, 0, 65536));
  for (int rep = 0; rep < 3; ++rep) dma_rate<WAVES><<<kBlocks, WAVES * 64>>>(cyc, src, iters);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  uint64_t* h = static_cast<uint64_t*>(malloc(kBlocks * WAVES * 16));
  CHECK(hipMemcpy(h, cyc, kBlocks * WAVES * 16, hipMemcpyDeviceToHost));
  double mxi, meani, mxd, meand;
  stats(h, kBlocks * WAVES, 2, 0, &mxi, &meani);
  stats(h, kBlocks * WAVES, 2, 1, &mxd, &meand);
  printf("dmaload  %2d waves: %.1f B per cycle per CU landed; issuing took %.1f cycles per load per wave\n", WAVES,
         1024.0 * iters * WAVES / mxd, meani / iters);
  free(h);
  CHECK(hipFree(cyc));
  CHECK(hipFree(src));
}

template <int W>
static void run_stream(const char* src) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  float best = 1e30f;
  for (int rep = 0; rep < 4; ++rep) {
    CHECK(hipEventRecord(e0));
    stream_rate<W><<<kBlocks, 256>>>(src);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    best = ms < best ? ms : best;
  }
  printf("stream   W=%2d loads in flight per wave (%3d KiB per CU): %.2f TB/s\n", W, 4 * W,
         kBlocks * static_cast<double>(kStreamPerWg) / (best * 1e-3) / 1e12);
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
}

static void run_sched(const char* src, int64_t copy, int share, int C, int rot = 0, int D = 2, int PF = 0) {
  uint64_t* rec;
  CHECK(hipMalloc(&rec, kBlocks * 16));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  float tot = 0;
  const int reps = 12;
  for (int rep = 0; rep < reps; ++rep) {
    // shared: one copy (128 ranges) per launch, three in turn; distinct: two copies
    // per launch, two pairs in turn (the buffer holds four)
    const char* base = src + (share ? (rep % 3) * copy : (rep % 2) * 2 * copy);
    CHECK(hipEventRecord(e0));
    if (D == 3) sched_rate<3, 0><<<kBlocks, 512>>>(base, C, share, rot, rec);
    else if (PF == 1) sched_rate<2, 1><<<kBlocks, 512>>>(base, C, share, rot, rec);
    else if (PF == 2) sched_rate<2, 2><<<kBlocks, 512>>>(base, C, share, rot, rec);
    else if (PF == 4) sched_rate<2, 4><<<kBlocks, 512>>>(base, C, share, rot, rec);
    else sched_rate<2, 0><<<kBlocks, 512>>>(base, C, share, rot, rec);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    if (rep >= 3) tot += ms;
  }
  uint64_t h[kBlocks * 2];
  CHECK(hipMemcpy(h, rec, sizeof(h), hipMemcpyDeviceToHost));
  double st = 0, is = 0;
  for (int k = 0; k < kBlocks; ++k) {
    st += static_cast<double>(h[2 * k]);
    is += static_cast<double>(h[2 * k + 1]);
  }
  const double us = tot / (reps - 3) * 1e3, bytes = (share ? 128.0 : 256.0) * kRangeBytes;
  printf("sched    %s ranges, D=%d, PF=%d, C=%4d, rot %2d: %.1f us for %.0f MB (%.2f TB/s), step %.0f cycles, tile issue %.0f\n",
         share ? "shared" : "distinct", D, PF, C, rot, us, bytes / 1e6, bytes / (us * 1e-6) / 1e12, st / (kBlocks * 32.0),
         is / (kBlocks * 32.0));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  CHECK(hipFree(rec));
}

int main(int argc, char** argv) {
  const bool only_sched = argc > 1 && argv[1][0] == 's';
  const int it = 2048;
  if (!only_sched) {
  run("lds", lds_read<8>, 8, it, 8192.0, "B");
  run("mfma16", mfma_rate<4, 0>, 4, it, 4 * 16384.0, "FLOP");
  run("mfma16", mfma_rate<8, 0>, 8, it, 4 * 16384.0, "FLOP");
  run("mfma32", mfma_rate<4, 1>, 4, it / 2, 4 * 32768.0, "FLOP");
  run("mfma32", mfma_rate<8, 1>, 8, it / 2, 4 * 32768.0, "FLOP");
  run_vload<4>(256);
  run_vload<8>(256);
  run_vload<16>(256);
  run_dma<4>(256);
  run_dma<8>(256);
  run("score32", score_read<0, 0>, 8, 1024, 16 * 1024.0, "B");
  run("score16", score_read<1, 0>, 8, 1024, 16 * 1024.0, "B");
  run("score16p", score_read<1, 1>, 8, 1024, 16 * 1024.0, "B");
  }
  // 2 GiB for the stream; four copies of 128 ranges (604 MB) for the schedule
  const int64_t copy = 128 * kRangeBytes;
  const int64_t total = std::max<int64_t>(kBlocks * kStreamPerWg, 4 * copy);
  char* src;
  CHECK(hipMalloc(&src, total));
  CHECK(hipMemset(src, 0, total));
  if (!only_sched) {
    run_stream<1>(src);
    run_stream<2>(src);
    run_stream<4>(src);
    run_stream<9>(src);
    run_stream<18>(src);
  }
  run_sched(src, copy, 1, 0);
  run_sched(src, copy, 1, 800);
  run_sched(src, copy, 0, 800);
  // the odd unit of each pair reads the shared tiles in a rotated order
  for (int rot : {2, 16}) run_sched(src, copy, 1, 0, rot);
  // a third tile in flight
  run_sched(src, copy, 1, 0, 0, 3);
  run_sched(src, copy, 1, 800, 0, 3);
  run_sched(src, copy, 1, 1400, 0, 3);
  run_sched(src, copy, 0, 800, 0, 3);
  // an L2 prefetch of half of tile i + 2 + PF by each unit of the pair
  for (int pf : {1, 2, 4}) {
    run_sched(src, copy, 1, 0, 0, 2, pf);
    run_sched(src, copy, 1, 800, 0, 2, pf);
  }
  CHECK(hipFree(src));
  return 0;
}
