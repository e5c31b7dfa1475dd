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
//
// Rates are bytes or FLOPs per cycle per CU, taken from the slowest wave of each
// launch. Every access stays inside its array or buffer (offsets are masked to the
// sizes below); the buffer loads carry a 64 KiB size bound as well.
//
//   hipcc --offload-arch=gfx950 -O3 rates.hip -o rates && ./rates
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define CHECK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                 \
      exit(1);                                                                \
    }                                                                         \
  } while (0)

constexpr int kBlocks = 256;

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void lds_read(uint64_t* cyc, u32x4* sink, int iters) {
  __shared__ u32x4 buf[4096];  // 64 KiB
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
  __shared__ u32x4 buf[WAVES * 1024];  // 16 KiB per wave
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

int main() {
  const int it = 2048;
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
  return 0;
}
