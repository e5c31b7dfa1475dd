// Device-side helpers shared by the gfx950 kernels of libmla.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) char lds_char;

// Generic -> LDS address-space pointer (the pointee must be __shared__ memory).
__device__ __forceinline__ lds_char* lds_ptr(const void* p) { return (lds_char*)(p); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// fp64 -> bf16 bits, round to nearest even, straight from the fp64 value (no
// intermediate fp32 rounding): keep the top 8 significant bits of the 53.
__device__ __forceinline__ uint16_t f64_to_bf16_bits(double x) {
  uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint16_t sign = static_cast<uint16_t>((u >> 48) & 0x8000u);
  const int e = static_cast<int>((u >> 52) & 0x7FF);
  uint64_t m = u & 0x000FFFFFFFFFFFFFull;
  if (e == 0x7FF) return m ? 0x7FC0 : static_cast<uint16_t>(sign | 0x7F80);
  if (e == 0) return sign;  // fp64 subnormals are far below bf16's range
  const int ue = e - 1023;  // unbiased exponent
  m |= 1ull << 52;          // significand with the implicit bit, 53 bits
  // bf16 keeps 8 significant bits for ue >= -126; below that the spacing is 2^-133.
  int keep = 8;
  if (ue < -126) keep = 8 - (-126 - ue);
  if (keep <= 0) {
    // rounds to 0 or to the smallest subnormal 2^-133
    if (keep == 0 && m > (1ull << 52)) return static_cast<uint16_t>(sign | 1);
    return sign;
  }
  const int drop = 53 - keep;
  const uint64_t half = 1ull << (drop - 1);
  const uint64_t rem = m & ((1ull << drop) - 1);
  uint64_t q = m >> drop;
  if (rem > half || (rem == half && (q & 1))) q += 1;
  // q now has keep (or keep + 1 after a carry) significant bits
  int ebits;
  uint32_t mant;
  if (ue >= -126) {
    int ee = ue;
    if (q >> 8) {  // carry out of 8 bits
      q >>= 1;
      ee += 1;
    }
    if (ee > 127) return static_cast<uint16_t>(sign | 0x7F80);
    ebits = ee + 127;
    mant = static_cast<uint32_t>(q & 0x7F);
  } else {
    // subnormal: value = q * 2^-133
    if (q >> 7) {
      ebits = 1;
      mant = static_cast<uint32_t>(q & 0x7F);
    } else {
      ebits = 0;
      mant = static_cast<uint32_t>(q);
    }
  }
  return static_cast<uint16_t>(sign | (ebits << 7) | mant);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Reductions across the two 32-lane halves of a wave (lanes l and l ^ 32), one
// v_permlane32_swap: both halves receive the bitwise-identical result.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wave-wide reductions without the LDS crossbar (which __shfl uses): butterflies
// inside each 16-lane row by DPP (lanes at distance 1 and 2 by quad permutes, then
// the mirrored half rows and the mirrored rows), then the four row results read
// with v_readlane and combined in a fixed order. The result is wave-uniform.
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, false);
}
template <typename Op>
__device__ __forceinline__ float wave_reduce_f(float x, Op op) {
  x = op(x, __int_as_float(dpp_mov<0xB1>(__float_as_int(x))));   // quad_perm [1,0,3,2]
  x = op(x, __int_as_float(dpp_mov<0x4E>(__float_as_int(x))));   // quad_perm [2,3,0,1]
  x = op(x, __int_as_float(dpp_mov<0x141>(__float_as_int(x))));  // row_half_mirror
  x = op(x, __int_as_float(dpp_mov<0x140>(__float_as_int(x))));  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return op(op(r0, r1), op(r2, r3));
}
__device__ __forceinline__ float wave_max(float x) {
  return wave_reduce_f(x, [](float p, float q) { return fmaxf(p, q); });
}
__device__ __forceinline__ float wave_sum(float x) {
  return wave_reduce_f(x, [](float p, float q) { return p + q; });
}
__device__ __forceinline__ int wave_max_i(int x) {
  x = max(x, dpp_mov<0xB1>(x));
  x = max(x, dpp_mov<0x4E>(x));
  x = max(x, dpp_mov<0x141>(x));
  x = max(x, dpp_mov<0x140>(x));
  return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// Workgroup barrier for LDS traffic between waves: this wave's LDS reads and
// writes are complete before it arrives (lgkmcnt(0) in the same block), but its
// global loads, direct-to-LDS loads included, stay in flight; callers wait for
// those with explicit vmcnt bounds. The memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt that bounds only the vector-memory counter (lgkm and exp left free).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes return zeros.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t ba = reinterpret_cast<uint64_t>(base);
  return u32x4{static_cast<uint32_t>(ba), static_cast<uint32_t>(ba >> 32) & 0xFFFFu, bytes, 0x00020000u};
}
constexpr uint32_t kOobOffset = 0xFFFFFFF0u;  // a lane offset past any size bound

// Direct-to-LDS buffer loads: lane l's 16 (or 4) bytes at buffer offset lane_off +
// off land at LDS address lds + 16 l (4 l). Issued from asm so that the compiler's
// wait insertion does not track them (it would otherwise wait for all such loads
// before unrelated LDS reads, and at loop headers); callers bound them with
// explicit vmcnt waits. The offset is formed inside the block (no per-load offset
// stays live in a VGPR); M0 takes the LDS base and is declared clobbered (the
// v_add gives the one wait state between the M0 write and the load). No memory
// clobber: a buffer being filled is not read before the caller's wait; being
// volatile, the statement keeps its order against other volatile asm (barriers,
// waits).
__device__ __forceinline__ void dma_b128(const u32x4& rsrc, uint32_t lane_off, uint32_t off, uint32_t lds) {
  uint32_t voff;
  asm volatile("" : "+s"(off), "+s"(lds));  // registers, never folded literals
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "v_add_u32 %0, %3, %2\n\t"
      "buffer_load_dwordx4 %0, %4, 0 offen lds"
      : "=&v"(voff)
      : "s"(lds), "v"(lane_off), "s"(off), "s"(rsrc)
      : "m0");
}
// A run of N (1, 2 or 4) such loads into consecutive 1 KiB blocks of LDS with one M0
// write: load k lands at lds + 1024 k + 16 l and reads buffer offset
// adj[k] + s + 1024 k. The instruction offset 1024 k moves the LDS and the buffer
// address together; callers fold -1024 k into adj[k] (which must stay
// non-negative), so the size bound still sees each load's true offset.
template <int N>
__device__ __forceinline__ void dma_run(const u32x4& rsrc, const uint32_t* adj, uint32_t s, uint32_t lds) {
  static_assert(N == 1 || N == 2 || N == 4, "run length");
  asm volatile("" : "+s"(s), "+s"(lds));  // registers, never folded literals
  if constexpr (N == 1) {
    uint32_t v0;
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "v_add_u32 %0, %2, %3\n\t"
        "buffer_load_dwordx4 %0, %4, 0 offen lds"
        : "=&v"(v0)
        : "s"(lds), "v"(adj[0]), "s"(s), "s"(rsrc)
        : "m0");
  } else if constexpr (N == 2) {
    uint32_t v0, v1;
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "v_add_u32 %0, %3, %5\n\t"
        "v_add_u32 %1, %4, %5\n\t"
        "buffer_load_dwordx4 %0, %6, 0 offen lds\n\t"
        "buffer_load_dwordx4 %1, %6, 0 offen offset:1024 lds"
        : "=&v"(v0), "=&v"(v1)
        : "s"(lds), "v"(adj[0]), "v"(adj[1]), "s"(s), "s"(rsrc)
        : "m0");
  } else {
    uint32_t v0, v1, v2, v3;
    asm volatile(
        "s_mov_b32 m0, %4\n\t"
        "v_add_u32 %0, %5, %9\n\t"
        "v_add_u32 %1, %6, %9\n\t"
        "v_add_u32 %2, %7, %9\n\t"
        "v_add_u32 %3, %8, %9\n\t"
        "buffer_load_dwordx4 %0, %10, 0 offen lds\n\t"
        "buffer_load_dwordx4 %1, %10, 0 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %2, %10, 0 offen offset:2048 lds\n\t"
        "buffer_load_dwordx4 %3, %10, 0 offen offset:3072 lds"
        : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
        : "s"(lds), "v"(adj[0]), "v"(adj[1]), "v"(adj[2]), "v"(adj[3]), "s"(s), "s"(rsrc)
        : "m0");
  }
}
__device__ __forceinline__ void dma_b32(const u32x4& rsrc, uint32_t lane_off, uint32_t lds) {
  asm volatile("" : "+s"(lds));
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(lds), "v"(lane_off), "s"(rsrc)
      : "m0");
}
// LDS address of a __shared__ object, as the 32-bit value M0 takes
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_ptr(p)));
}

}  // namespace mla
