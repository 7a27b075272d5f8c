// Packing kernel for gfx950 (MI355X): bf16 latent rows -> the fp8 paged pool the attention
// kernels read.
//
// The pages name this step without printing it: "fix(sparse-mla-sm120): add topk=256
// prefill-dsv4 dispatch" packs its KV input with quantize_kv_dsv4 (comment thread, the
// compute-mode comparison), and the FlashInfer 4802 merge message (sections Summary and
// Compatibility) places the per-64 fp32 scales inline after the payload or in a page footer.
// Here a group of 64 consecutive elements gets the scale amax / 448, so that its largest
// magnitude lands on e4m3fn's largest finite value; each element becomes the e4m3fn code
// nearest to x * (448 / amax) (ties to even; the multiplier, the product and the stored
// scale are IEEE fp32 operations).
//
// Design. The work is one pass over HBM (read 2 B and write a little over 1 B per element),
// so the kernel is laid out for coalescing and for bytes in flight, not for arithmetic:
// every thread takes the same 8 consecutive elements (one 16-byte load) of 2 consecutive
// rows and issues both loads before using either, 8 neighbouring lanes of a wave hold one
// group and reduce its amax with three lane swaps, and each lane stores its 8 codes as one
// 8-byte write next to its neighbours'. The lane holding a group's first elements stores
// the scale. A row whose slot is outside the pool is skipped by all of its threads. The rows
// are read and the codes written with non-temporal hints (streamed once; measured +9 %);
// the 4-byte scale stores stay ordinary, so the caches merge them with the codes that share
// their line.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int kPackThreads = 256;
constexpr int kRows = 2;  // rows per thread (measured: 2 > 4 > 8)
constexpr float kE4m3Max = 448.f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 values (|v| <= 448) -> two e4m3fn bytes in the low 16 bits, rounded to nearest
// even by the hardware convert.
__device__ __forceinline__ uint32_t to_e4m3x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

__global__ __launch_bounds__(kPackThreads) void smla_pack_kernel(PackParams p) {
  const int cpr = p.d_qk / 8;  // 8-element chunks per row (a multiple of 8: whole groups)
  const int64_t gi = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
  const int64_t quad = gi / cpr;  // this thread's rows: kRows consecutive ones from kRows*quad
  const int c = (int)(gi - quad * cpr);
  // All loads go out before any is used (kRows x 16 bytes in flight per lane); a row past
  // n re-reads the last row and stores nothing, so every lane of a group stays active for
  // the lane swaps.
  u32x4 w[kRows];
  int32_t s[kRows];
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    const int64_t row = min(kRows * quad + k, p.n - 1);
    w[k] = __builtin_nontemporal_load((const u32x4 *)(p.rows + row * p.rows_st + 8 * c));
    s[k] = kRows * quad + k < p.n ? p.slots[row] : -1;
  }
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_lo(w[k][e]);
      x[2 * e + 1] = bf16_hi(w[k][e]);
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 8));
    // the stored scale and the quantising multiplier, each one IEEE division per group (the
    // multiplier stays finite: an all-zero group multiplies its signed zeros by FLT_MAX)
    const float scale = amax / kE4m3Max;
    const float inv = fminf(kE4m3Max / amax, __FLT_MAX__);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = fminf(fmaxf(x[e] * inv, -kE4m3Max), kE4m3Max);
    const u32x2 codes = {to_e4m3x2(v[0], v[1]) | to_e4m3x2(v[2], v[3]) << 16,
                         to_e4m3x2(v[4], v[5]) | to_e4m3x2(v[6], v[7]) << 16};
    // a row whose slot is outside the pool (or past n) is skipped by all of its lanes
    if (s[k] < 0 || (int64_t)s[k] >= p.kv.num_slots) continue;
    const int64_t page = s[k] >> 6, off = s[k] & 63;
    uint8_t *dst = p.kv_data + page * p.kv.page_stride + off * p.kv.row_stride;
    __builtin_nontemporal_store(codes, (u32x2 *)(dst + 8 * c));
    if ((c & 7) == 0) {
      uint8_t *sdst = p.kv_scales + page * p.kv.scale_page_stride + off * p.kv.scale_row_stride;
      *(float *)(sdst + 4 * (c >> 3)) = scale;
    }
  }
}

}  // namespace

hipError_t launch_pack(const PackParams &p, hipStream_t s) {
  const int64_t threads = (p.n + kRows - 1) / kRows * (p.d_qk / 8);
  const int64_t blocks = (threads + kPackThreads - 1) / kPackThreads;
  hipLaunchKernelGGL(smla_pack_kernel, dim3((unsigned)blocks), dim3(kPackThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace smla
