// Device helpers shared by the decode kernel (decode.hip) and the narrow kernel
// (narrow_kernel.h): both keep raw fp8 latent rows in LDS, filled by LDS DMA, and convert the
// codes to bf16 as MFMA operands. Internal linkage: every translation unit gets its own copy.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {
namespace dk {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((__vector_size__(2 * sizeof(uint16_t)))) uint16_t u16x2;
typedef __attribute__((address_space(1))) const u32x2 gu32x2;
typedef __attribute__((address_space(1))) const float gf32;
typedef __attribute__((address_space(1))) const int32_t gi32;
typedef __attribute__((address_space(4))) const int32_t ci32;
typedef __attribute__((address_space(3))) u32x4 lu32x4;
typedef __attribute__((address_space(3))) u32x2 lu32x2;
typedef __attribute__((address_space(3))) i32x2 li32x2;

constexpr int kRowB = 512;   // latent bytes of an fp8 row kept in LDS (the V part of d_qk 576)
constexpr int kGroups = 8;   // latent scale groups of 64
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.0f;  // lazy rescale threshold: P <= 2^8

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS slot of 16-byte chunk c of row r is c ^ swz(r): the QK operand reads (16 rows, one
// chunk pair) and the transpose reads of PV (32 rows, one chunk) then hit distinct banks.
__device__ __forceinline__ int swz(int r) { return ((r & 15) << 1) | ((r >> 4) & 1); }

// s_waitcnt with vmcnt <= N and no wait on the LDS/scalar or export counters (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The same with a count known only at run time (0 <= n < 64; larger counts wait for 63).
template <int B>
__device__ __forceinline__ void wait_vmcnt_from(int n) {
  if constexpr (B < 63) {
    if (n == B) {
      wait_vmcnt<B>();
      return;
    }
    wait_vmcnt_from<B + 1>(n);
  } else {
    wait_vmcnt<63>();
  }
}
__device__ __forceinline__ void wait_vmcnt_rt(int n) { wait_vmcnt_from<0>(n); }

// The value of lane l and of lane l ^ 32 (l ^ 16): v_permlane32_swap (v_permlane16_swap) with
// both operands v returns the pair in both lanes, in the same order, so a sum over the pair
// is bit-identical in both lanes.
__device__ __forceinline__ float pair_max32(float v) {
  const uint32_t x = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_max16(float v) {
  const uint32_t x = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float v) {
  const uint32_t x = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_sum16(float v) {
  const uint32_t x = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};  // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// Byte address of p in LDS (p points into a __shared__ variable of the kernel).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}
// x, opaque to the optimiser: addresses derived from it in a loop body are formed there
// (register + constant offset, or one XOR) instead of being hoisted out of the loop as one
// live register per address.
__device__ __forceinline__ uint32_t opaque_u32(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
template <class T>
__device__ __forceinline__ T lds_load(uint32_t a) {
  return *(__attribute__((address_space(3))) const T *)(uintptr_t)a;
}

// 8 e4m3fn codes -> 8 bf16, exactly (scale 1: every e4m3fn value is a bf16 value).
__device__ __forceinline__ bf16x8 codes_to_bf16(u32x2 v) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 16 bytes per lane from global memory into LDS at base + 16 * lane, and 4 bytes per lane
// into base + 4 * lane (the LDS base goes in M0). Inline assembly, so the compiler's
// wait-count bookkeeping does not see these loads; the waves that issue them wait with
// explicit s_waitcnt vmcnt, and every call site issues the instruction with all lanes
// active (unused rows read a static zero row), so each wave's count of them is known.
// M0 is written here only; no compiled code of the kernels uses M0 (clang warns that an M0
// clobber may not be honoured), which the CPU test test_m0_guard checks on the generated
// assembly.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *g, const void *lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(m0)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void *g, const void *lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(g), "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace
}  // namespace dk
}  // namespace smla
