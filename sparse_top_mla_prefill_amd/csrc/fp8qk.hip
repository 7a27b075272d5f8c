// fp8 compute mode for gfx950 (MI355X): QK on fp8 MFMA over the raw pool payload.
//
// The pages fork the kernels on a compute mode: "fix(sparse-mla-sm120): add topk=256
// prefill-dsv4 dispatch" dispatches prefill by (num_heads, compute mode) with an FP8 and a
// BF16 mode, and its comment thread compares the two on the same KV input; the FlashInfer
// 4802 merge message (section "Performance vs main") quantises q into shared memory on the
// fp8 side (quantize_q_to_smem). Here q is quantised per (token, head) to e4m3fn with the
// multiplier 448 / amax and the factor amax / 448 kept for the logits; QK runs on
// v_mfma_f32_16x16x32_fp8_fp8 with the fp8 rows exactly as the pool stores them, one 64-wide
// scale group at a time (a group's fp32 scale differs per key, so each group's partial dot
// products are scaled and added in fp32). P stays bf16 and PV runs on bf16 MFMA with V
// dequantised from the raw tile as it is read.
//
// Design. A workgroup of 4 waves serves one (token, 32-head group) and walks the index list
// in tiles of 32 keys. Raw rows (576 payload bytes) and their 9 scales are staged in LDS:
// 19 KB per tile, so several workgroups share a CU and hide each other's latency. The rows
// of tile i+1 are loaded into registers while tile i is computed, and the slot ids two
// tiles ahead.
//   QK: wave w takes keys 16 (w & 1) .. +16 and heads 16 (w >> 1) .. +16; per group, two
//       MFMAs (K = 32 each) into a zeroed accumulator, then S += scale[key, g] * acc.
//   softmax: per-head tile maxima and sums meet in LDS; every wave keeps the running max of
//       the heads it touches (the same sequence of values), P goes to LDS as bf16 [head][key].
//   PV: wave w owns d columns 128 w .. +128; A = V^T read byte by byte from the raw tile and
//       scaled into bf16 (each V element is read and converted once), B = P^T.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int kFThreads = 256;  // 4 waves
constexpr int kFTile = 32;      // keys per tile
constexpr int kFHeads = 32;     // heads per workgroup
constexpr int kFRS = 576 + 16;  // LDS row stride of a raw fp8 row (bytes)
constexpr int kFGroups = 9;     // scale groups of 64 in d_qk 576
constexpr int kFPS = kFTile + 8;  // P row stride (bf16 elements)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float ninf() { return -__builtin_inff(); }

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// One e4m3fn code -> fp32 (exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8(code, 0);
}

__device__ __forceinline__ uint32_t to_e4m3x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

struct FSmem {
  uint8_t rows[kFTile][kFRS];
  float sc[kFGroups][kFTile];  // scales [group][key]
  int32_t slots[2][kFTile];
  uint32_t vmask[2];
  float tmax[2][kFHeads];  // per key half
  float tsum[2][kFHeads];
  uint16_t P[kFHeads][kFPS];
};

__global__ __launch_bounds__(kFThreads) void smla_fp8qk_kernel(const KParams p) {
  __shared__ __attribute__((aligned(16))) FSmem sm;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int t = (int)blockIdx.x / p.n_hg;
  const int h0 = ((int)blockIdx.x - t * p.n_hg) * kFHeads;
  const int n_tiles = p.n_tiles;

  // slot ids of one tile (wave 0, lanes < 32): raw id, or -1 when not live
  auto tile_slots = [&](int tile) -> int32_t {
    const bool main = tile < p.main_tiles;
    const int pos = (main ? tile : tile - p.main_tiles) * kFTile + (l & 31);
    const int width = main ? p.topk : p.topk_extra;
    const int32_t *row = main ? p.idx + (int64_t)t * p.idx_st : p.eidx + (int64_t)t * p.eidx_st;
    const int32_t *lens = main ? p.len : p.elen;
    const int live = lens ? min(max(lens[t], 0), width) : width;
    const int32_t s = row[min(pos, width - 1)];
    const bool ok = l < kFTile && pos < live && s >= 0 && (int64_t)s < p.kv.num_slots;
    return ok ? s : -1;
  };
  auto commit_slots = [&](int buf, int32_t s) {
    if (l < kFTile) sm.slots[buf][l] = s;
    const uint64_t m = __ballot(s >= 0);
    if (l == 0) sm.vmask[buf] = (uint32_t)m;
  };

  // row staging: thread -> (row r, 8-byte column c of each 64-byte block)
  const int r = tid >> 3, c = tid & 7;
  u32x2 pay[kFGroups];
  float scl[2];
  auto load_rows = [&](int buf) {
    const int32_t s = sm.slots[buf][r];
    const int64_t ss = s < 0 ? 0 : s;  // unused rows read slot 0 (in bounds)
    const uint8_t *base = p.kv.data + (ss >> 6) * p.kv.page_stride + (ss & 63) * p.kv.row_stride;
    const uint8_t *sbase =
        p.kv.scales + (ss >> 6) * p.kv.scale_page_stride + (ss & 63) * p.kv.scale_row_stride;
#pragma unroll
    for (int m = 0; m < kFGroups; ++m) pay[m] = *(const u32x2 *)(base + 64 * m + 8 * c);
    scl[0] = *(const float *)(sbase + 4 * c);
    scl[1] = *(const float *)(sbase + 4 * 8);
  };
  auto store_rows = [&]() {
#pragma unroll
    for (int m = 0; m < kFGroups; ++m) *(u32x2 *)(&sm.rows[r][64 * m + 8 * c]) = pay[m];
    sm.sc[c][r] = scl[0];
    if (c == 0) sm.sc[8][r] = scl[1];
  };

  // q of this lane's QK head, quantised to e4m3fn: chunk (g, ks) holds d = 64 g + 32 ks +
  // 8 (l >> 4) .. +8, the B-operand layout of the fp8 MFMA
  const int kb = w & 1, hb = w >> 1;
  const int hq = 16 * hb + (l & 15);  // QK head within the group
  const int hp = l & 31;              // PV head within the group
  uint64_t q8[kFGroups][2];
  float qs;  // amax / 448 of the head's q row
  {
    const int head = min(h0 + hq, p.h - 1);  // heads past h compute with a live head's q
    const uint16_t *qr = p.q + (int64_t)t * p.q_st + (int64_t)head * p.q_sh + 8 * (l >> 4);
    u32x4 qv[kFGroups][2];
    float amax = 0.f;
#pragma unroll
    for (int g = 0; g < kFGroups; ++g)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        qv[g][ks] = *(const u32x4 *)(qr + 64 * g + 32 * ks);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          amax = fmaxf(amax, fabsf(__uint_as_float(qv[g][ks][e] << 16)));
          amax = fmaxf(amax, fabsf(__uint_as_float(qv[g][ks][e] & 0xffff0000u)));
        }
      }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    qs = amax / 448.f;
    const float inv = fminf(448.f / amax, __FLT_MAX__);
#pragma unroll
    for (int g = 0; g < kFGroups; ++g)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = fminf(fmaxf(__uint_as_float(qv[g][ks][e] << 16) * inv, -448.f), 448.f);
          const float b =
              fminf(fmaxf(__uint_as_float(qv[g][ks][e] & 0xffff0000u) * inv, -448.f), 448.f);
          const uint32_t two = to_e4m3x2(a, b);
          if (e < 2) lo |= two << (16 * e); else hi |= two << (16 * (e - 2));
        }
        q8[g][ks] = (uint64_t)lo | ((uint64_t)hi << 32);
      }
  }
  const float zscale = qs * p.scale_log2;  // acc -> log2-domain logit

  // prologue: slot ids of tiles 0 and 1, rows of tile 0
  if (w == 0) {
    commit_slots(0, tile_slots(0));
    commit_slots(1, n_tiles > 1 ? tile_slots(1) : -1);
  }
  __syncthreads();
  load_rows(0);
  store_rows();
  __syncthreads();

  float m_run = ninf(), l_run = 0.f;  // PV head hp: running max (log2 units) and sum
  float mq_run = ninf();              // QK head hq: the same running max
  f32x16 oacc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[b][e] = 0.f;

  for (int i = 0; i < n_tiles; ++i) {
    const bool more = i + 1 < n_tiles;
    int32_t s2 = -1;
    if (more) load_rows((i + 1) & 1);
    if (w == 0 && i + 2 < n_tiles) s2 = tile_slots(i + 2);
    const uint32_t vm = sm.vmask[i & 1];

    // QK: S for keys 16 kb + 4 (l >> 4) + e, head hq
    float sv[4] = {0.f, 0.f, 0.f, 0.f};
    const uint8_t *arow = &sm.rows[16 * kb + (l & 15)][8 * (l >> 4)];
#pragma unroll
    for (int g = 0; g < kFGroups; ++g) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint64_t a = *(const uint64_t *)(arow + 64 * g + 32 * ks);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)a, (long)q8[g][ks], acc, 0, 0, 0);
      }
      const f32x4 s4 = *(const f32x4 *)(&sm.sc[g][16 * kb + 4 * (l >> 4)]);
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[e] = fmaf(s4[e], acc[e], sv[e]);
    }
    float tmx = ninf();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = 16 * kb + 4 * (l >> 4) + e;
      sv[e] = ((vm >> key) & 1) ? sv[e] * zscale : ninf();
      tmx = fmaxf(tmx, sv[e]);
    }
    tmx = fmaxf(tmx, __shfl_xor(tmx, 16));
    tmx = fmaxf(tmx, __shfl_xor(tmx, 32));
    if (l < 16) sm.tmax[kb][hq] = tmx;
    __syncthreads();

    // softmax: P = 2^(S - m) for the QK head, in bf16
    {
      const float mn = fmaxf(mq_run, fmaxf(sm.tmax[0][hq], sm.tmax[1][hq]));
      mq_run = mn;
      float ps = 0.f;
      uint32_t pw[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float a = mn == ninf() ? 0.f : __builtin_amdgcn_exp2f(sv[2 * e] - mn);
        const float b = mn == ninf() ? 0.f : __builtin_amdgcn_exp2f(sv[2 * e + 1] - mn);
        pw[e] = pk_bf16(a, b);
        ps += a + b;  // the row sum takes P before its bf16 rounding, as in the bf16 mode
      }
      *(u32x2 *)(&sm.P[hq][16 * kb + 4 * (l >> 4)]) = u32x2{pw[0], pw[1]};
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      if (l < 16) sm.tsum[kb][hq] = ps;
    }
    __syncthreads();

    // PV: rescale, then O^T[d][head] += V^T P^T over the tile's 32 keys
    {
      const float mn = fmaxf(m_run, fmaxf(sm.tmax[0][hp], sm.tmax[1][hp]));
      const float f = m_run == ninf() ? 0.f : __builtin_amdgcn_exp2f(m_run - mn);
      m_run = mn;
      l_run = l_run * f + sm.tsum[0][hp] + sm.tsum[1][hp];
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[b][e] *= f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int k0 = 16 * ks + 8 * (l >> 5);  // this lane's 8 keys
        const bf16x8 pb = *(const bf16x8 *)(&sm.P[hp][k0]);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int d = 128 * w + 32 * b + (l & 31);
          const int g = (128 * w + 32 * b) >> 6;
          const f32x4 sa = *(const f32x4 *)(&sm.sc[g][k0]);
          const f32x4 sb = *(const f32x4 *)(&sm.sc[g][k0 + 4]);
          uint32_t v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x0 = e4m3_to_f32(sm.rows[k0 + 2 * e][d]) * (e < 2 ? sa[2 * e] : sb[2 * e - 4]);
            const float x1 =
                e4m3_to_f32(sm.rows[k0 + 2 * e + 1][d]) * (e < 2 ? sa[2 * e + 1] : sb[2 * e - 3]);
            v[e] = pk_bf16(x0, x1);
          }
          const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{v[0], v[1], v[2], v[3]});
          oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[b], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // the tile's rows, scales and P are consumed
    if (more) store_rows();
    if (w == 0 && i + 2 < n_tiles) commit_slots(i & 1, s2);
    __syncthreads();
  }

  // finalize with the sink: o = O 2^(m - m') / (l 2^(m - m') + 2^(sigma - m'))
  const int head = h0 + hp;
  if (head < p.h) {
    const float sig = p.sink ? p.sink[head] * kLog2e : ninf();
    const float mf = fmaxf(m_run, sig);
    float scale = 0.f, lse = ninf();
    if (mf != ninf()) {
      const float fo = m_run == ninf() ? 0.f : __builtin_amdgcn_exp2f(m_run - mf);
      const float fs = sig == ninf() ? 0.f : __builtin_amdgcn_exp2f(sig - mf);
      const float den = l_run * fo + fs;
      scale = fo / den;
      lse = (mf + __log2f(den)) * kLn2;
    }
    if (p.lse && w == 0 && l < 32) p.lse[(int64_t)t * p.lse_st + head] = lse;
    uint16_t *dst = p.out + (int64_t)t * p.out_st + (int64_t)head * p.out_sh;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 128 * w + 32 * b + 8 * j + 4 * (l >> 5);
        const u32x2 o = {pk_bf16(oacc[b][4 * j] * scale, oacc[b][4 * j + 1] * scale),
                         pk_bf16(oacc[b][4 * j + 2] * scale, oacc[b][4 * j + 3] * scale)};
        *(u32x2 *)(dst + d0) = o;
      }
  }
}

}  // namespace

hipError_t launch_fp8qk(const KParams &p, hipStream_t s) {
  hipLaunchKernelGGL(smla_fp8qk_kernel, dim3((unsigned)((int64_t)p.T * p.n_hg)), dim3(kFThreads),
                     0, s, p);
  return hipGetLastError();
}

}  // namespace smla
