// Sparse top-k MLA attention kernels for gfx950 (MI355X).
//
// What is computed. For query token t and head h:
//   o[t,h] = sum_j e^{z_j} v_j / (sum_j e^{z_j} + e^{sink_h}),   z_j = sm_scale * <q[t,h], r_j>,
// where r_j are the latent rows of the token's valid top-k slots and v_j = r_j[0:d_v].
//
// The pages say what the path must serve:
//   - "[SM12x] Drop the 64-head TP pad on the DSv4 MLA prefill path" (section Problem):
//     all heads of a token share one latent KV head, so one gathered row feeds every head.
//   - The FlashInfer 4802 merge message (inside "fix(sm120): explain sparse-MLA decode
//     dispatch misses; add config query API"):
//       . 64-wide index tiles, any head count in [1,128] and any topk % 64 == 0
//         (section "Runtime envelopes");
//       . sinks and an optional out_lse (section Summary);
//       . the decode form's split-K partials and their merge (section "Runner and CUDA
//         graphs").
//
// Design (gfx950, wave64).
//   - One workgroup of 4 waves serves one (token, head group, index chunk). It walks the
//     chunk in tiles of TILE keys:
//       . the slot ids of tile i+2 become row addresses in LDS;
//       . the rows of tile i+1 are gathered (16 B per lane), dequantised to bf16 on load
//         and written to the idle half of a double-buffered LDS tile;
//       . meanwhile every wave computes on tile i.
//   - Each wave owns 16*NB heads (a head slice), or half of a tile's keys for small head
//     counts (NKS = 2). Its q rows live in registers for the whole walk.
//   - QK: S^T = K Q^T on v_mfma_f32_16x16x32_bf16. The A operand is 8 consecutive latent
//     elements of one gathered row (one ds_read_b128). The B operand is the wave's q,
//     already in registers.
//   - Online softmax on S^T, where every lane owns one head column: max and sum need only
//     two cross-lane exchanges. The running max is rescaled lazily, only when it grows by
//     more than 2^8, and the choice is made per head, so heads stay independent.
//   - PV: O^T = V^T P^T. The A operand comes straight from the row-major tile through
//     ds_read_b64_tr_b16 (the LDS transpose read), so no second, transposed copy is
//     stored. The B operand is P, rounded to bf16, in exactly the register layout that
//     S^T left it in.
//   - fp8 rows are dequantised once per workgroup on the way into LDS (e4m3fn code ->
//     fp32, times the per-64 fp32 scale, rounded to bf16), not once per wave.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "smla_internal.h"

namespace smla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.0f;  // lazy rescale threshold: P <= 2^8
constexpr int kThreads = 256;
constexpr int kStageRounds = 3;

template <int D_QK>
struct Geo;
template <>
struct Geo<576> {
  static constexpr int D_V = 512, TILE = 64;
};
template <>
struct Geo<1088> {
  static constexpr int D_V = 1024, TILE = 32;
};

struct RowAddr {
  const uint8_t *data;   // nullptr: the slot is unused
  const uint8_t *scale;  // fp8 scales of the row
};

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};  // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// Two e4m3fn bytes (the low or high 16 bits of w) times an fp32 scale -> two packed bf16.
// The scaled convert instructions of gfx950 apply only the exponent of their scale operand
// (power-of-two block scales), so the codes are converted exactly with scale 1, multiplied
// by the full fp32 scale, and rounded once to bf16.
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, float s, bool hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
  const f32x2 f = hi ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true)
                     : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
  return pack_bf16(f[0] * s, f[1] * s);
}

__device__ __forceinline__ float wave_xor_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float wave_xor_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Staging: the 256 threads split a tile as TPR = 256 / TILE threads per row. Thread
// (row r = tid / TPR, q = tid % TPR) moves the row's 16-byte source chunks k = q + TPR*j.
// So one thread reads one row address per tile, and every load, scale read and LDS store
// is that row's base plus an immediate offset. The chunks of a thread are split into
// kStageRounds rounds so that only one round's registers are live at a time.
template <int D_QK>
struct Tiling {
  static constexpr int TILE = Geo<D_QK>::TILE;
  static constexpr int RS = D_QK + 8;         // LDS row stride (bf16 elements), +16 B pad
  static constexpr int TPR = kThreads / TILE;  // threads per row
  static constexpr int CPR8 = D_QK / 16;      // 16-byte source chunks per fp8 row
  static constexpr int CPR16 = D_QK / 8;      // 16-byte source chunks per bf16 row
  static constexpr int J8 = (CPR8 + TPR - 1) / TPR;    // chunks per thread, fp8
  static constexpr int J16 = (CPR16 + TPR - 1) / TPR;  // chunks per thread, bf16
  static constexpr int NPR8 = (J8 + kStageRounds - 1) / kStageRounds;
  static constexpr int NPR16 = (J16 + kStageRounds - 1) / kStageRounds;
};

typedef __attribute__((address_space(1))) const u32x4 gu32x4;
typedef __attribute__((address_space(1))) const float gf32;
typedef __attribute__((address_space(3))) u32x4 lu32x4;

struct Stage {
  u32x4 v[6];
  float sc[3];
};

template <int D_QK>
__device__ __forceinline__ void stage_issue(Stage &st, int round, bool fp8, const RowAddr &a,
                                            int q) {
  using TL = Tiling<D_QK>;
  if (fp8) {
#pragma unroll
    for (int i = 0; i < TL::NPR8; ++i) {
      const int k = q + TL::TPR * (round * TL::NPR8 + i);
      st.v[i] = u32x4{0, 0, 0, 0};
      st.sc[i] = 0.0f;
      if (a.data && k < TL::CPR8) {
        st.v[i] = *(gu32x4 *)(a.data + 16 * k);
        st.sc[i] = *(gf32 *)(a.scale + 4 * (k >> 2));
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TL::NPR16; ++i) {
      const int k = q + TL::TPR * (round * TL::NPR16 + i);
      st.v[i] = u32x4{0, 0, 0, 0};
      if (a.data && k < TL::CPR16) st.v[i] = *(gu32x4 *)(a.data + 16 * k);
    }
  }
}

template <int D_QK>
__device__ __forceinline__ void stage_commit(const Stage &st, int round, bool fp8, uint16_t *row,
                                             int q) {
  using TL = Tiling<D_QK>;
  if (fp8) {
#pragma unroll
    for (int i = 0; i < TL::NPR8; ++i) {
      const int k = q + TL::TPR * (round * TL::NPR8 + i);
      if (k < TL::CPR8) {
        const float s = st.sc[i];
        u32x4 lo, hi;
        lo[0] = fp8x2_to_bf16x2(st.v[i][0], s, false);
        lo[1] = fp8x2_to_bf16x2(st.v[i][0], s, true);
        lo[2] = fp8x2_to_bf16x2(st.v[i][1], s, false);
        lo[3] = fp8x2_to_bf16x2(st.v[i][1], s, true);
        hi[0] = fp8x2_to_bf16x2(st.v[i][2], s, false);
        hi[1] = fp8x2_to_bf16x2(st.v[i][2], s, true);
        hi[2] = fp8x2_to_bf16x2(st.v[i][3], s, false);
        hi[3] = fp8x2_to_bf16x2(st.v[i][3], s, true);
        lu32x4 *dst = (lu32x4 *)(row + 16 * k);
        dst[0] = lo;
        dst[1] = hi;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TL::NPR16; ++i) {
      const int k = q + TL::TPR * (round * TL::NPR16 + i);
      if (k < TL::CPR16) *(lu32x4 *)(row + 8 * k) = st.v[i];
    }
  }
}

// Map a tile number to its pool and index pointer.
struct TileSrc {
  const PoolArgs *pool;
  const int32_t *idx;
};

template <int TILE>
__device__ __forceinline__ TileSrc tile_source(const KParams &p, int t, int tile) {
  const int n_main = p.topk / TILE;
  if (tile < n_main) return {&p.kv, p.idx + t * p.idx_st + tile * TILE};
  return {&p.ex, p.eidx + t * p.eidx_st + (tile - n_main) * TILE};
}

// Wave 0 turns a tile's slot ids into row addresses and a validity mask.
template <int TILE>
__device__ __forceinline__ void fill_rows(const KParams &p, int t, int tile, RowAddr *ra,
                                          uint64_t *vmask, int lane) {
  const TileSrc src = tile_source<TILE>(p, t, tile);
  bool valid = false;
  if (lane < TILE) {
    const int64_t s = src.idx[lane];
    const PoolArgs &pl = *src.pool;
    valid = s >= 0 && s < pl.num_slots;
    RowAddr a = {nullptr, nullptr};
    if (valid) {
      const int64_t page = s >> 6, off = s & 63;
      a.data = pl.data + page * pl.page_stride + off * pl.row_stride;
      a.scale = pl.scales ? pl.scales + page * pl.scale_page_stride + off * pl.scale_row_stride
                          : nullptr;
    }
    ra[lane] = a;
  }
  const uint64_t m = __ballot(valid);
  if (lane == 0) *vmask = m;
}

template <int TILE>
__device__ __forceinline__ bool tile_is_fp8(const KParams &p, int tile) {
  return tile < p.topk / TILE ? p.kv.fp8 != 0 : p.ex.fp8 != 0;
}

template <int D_QK, int NB, int NKS>
__global__ __launch_bounds__(kThreads, 1) void smla_attn_kernel(const KParams p) {
  constexpr int D_V = Geo<D_QK>::D_V;
  constexpr int TILE = Geo<D_QK>::TILE;
  constexpr int RS = Tiling<D_QK>::RS;
  constexpr int KPW = TILE / NKS;  // keys of a tile handled by one wave
  constexpr int NKB = KPW / 16;    // S^T key blocks per wave
  constexpr int NKK = KPW / 32;    // PV k-steps per wave
  constexpr int NHS = 4 / NKS;     // head slices per workgroup
  constexpr int HG = NHS * 16 * NB;
  constexpr int QS = D_QK / 32;    // QK k-steps
  constexpr int DB = D_V / 16;     // O^T row blocks
  static_assert(KPW % 32 == 0, "a wave needs whole PV k-steps");

  __shared__ __attribute__((aligned(16))) uint16_t tiles[2][TILE * RS];
  __shared__ RowAddr rows[3][TILE];
  __shared__ uint64_t vmask[3];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int hs = w % NHS, ks = w / NHS;

  int b = blockIdx.x;
  const int chunk = b % p.n_chunks;
  b /= p.n_chunks;
  const int hg = b % p.n_hg;
  const int t = b / p.n_hg;

  const int head0 = hg * HG + hs * 16 * NB;
  const bool active = head0 < p.h;

  const int n_tiles = (p.topk + p.topk_extra) / TILE;
  const int tile_begin = chunk * p.tiles_per_chunk;
  const int tile_end = min(n_tiles, tile_begin + p.tiles_per_chunk);

  // q of this wave's heads, as QK B operands: lane (g, li) holds q[head li][32s + 8g .. +7].
  // Heads past h read head 0's row (always in bounds) and are zeroed.
  bf16x8 qop[NB][QS];
#pragma unroll
  for (int hb = 0; hb < NB; ++hb) {
    const int head = head0 + 16 * hb + li;
    const bool ok = active && head < p.h;
    const uint16_t *qrow = p.q + (int64_t)t * p.q_st + (int64_t)(ok ? head : 0) * p.q_sh + 8 * g;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      u32x4 v = *reinterpret_cast<const u32x4 *>(qrow + 32 * s);
      if (!ok) v = u32x4{0, 0, 0, 0};
      qop[hb][s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 oacc[NB][DB];
#pragma unroll
  for (int hb = 0; hb < NB; ++hb)
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[hb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref[NB], l_part[NB];
#pragma unroll
  for (int hb = 0; hb < NB; ++hb) {
    m_ref[hb] = neg_inf();
    l_part[hb] = 0.f;
  }

  Stage st;
  const int srow = tid / Tiling<D_QK>::TPR, sq = tid % Tiling<D_QK>::TPR;
  if (tile_begin < tile_end) {
    // Prologue: rows of the first tile into buffer 0, addresses of the second.
    if (w == 0) fill_rows<TILE>(p, t, tile_begin, rows[0], &vmask[0], lane);
    __syncthreads();
    const bool f8 = tile_is_fp8<TILE>(p, tile_begin);
    const RowAddr a0 = rows[0][srow];
#pragma unroll
    for (int r = 0; r < kStageRounds; ++r) {
      stage_issue<D_QK>(st, r, f8, a0, sq);
      stage_commit<D_QK>(st, r, f8, tiles[0] + srow * RS, sq);
    }
    if (w == 0 && tile_begin + 1 < tile_end)
      fill_rows<TILE>(p, t, tile_begin + 1, rows[1], &vmask[1], lane);
    __syncthreads();
  }

  for (int it = tile_begin; it < tile_end; ++it) {
    const int i = it - tile_begin;
    const int cur = i & 1, nxt = cur ^ 1;
    const int a_cur = i % 3, a_nxt = (i + 1) % 3, a_nn = (i + 2) % 3;
    const bool has_next = it + 1 < tile_end;
    const bool f8n = has_next && tile_is_fp8<TILE>(p, it + 1);
    const uint16_t *kt = tiles[cur] + ks * KPW * RS;

    RowAddr an = {nullptr, nullptr};
    if (has_next) {
      an = rows[a_nxt][srow];
      stage_issue<D_QK>(st, 0, f8n, an, sq);
    }
    uint16_t *const srow_dst = tiles[nxt] + srow * RS;

    uint32_t pop[NB][NKK][4];  // P^T as bf16 B operands of PV
    if (active) {
      // ---- S^T = K Q^T over d_qk, two-stage pipeline: operands of step s+1 load while the
      // MFMAs of step s run.
      f32x4 sacc[NB][NKB];
#pragma unroll
      for (int hb = 0; hb < NB; ++hb)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) sacc[hb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t *krow = kt + li * RS + 8 * g;
      bf16x8 abuf[2][NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        abuf[0][kb] = *reinterpret_cast<const bf16x8 *>(krow + 16 * kb * RS);
#pragma unroll
      for (int s = 0; s < QS; ++s) {
        if (s + 1 < QS) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            abuf[(s + 1) & 1][kb] =
                *reinterpret_cast<const bf16x8 *>(krow + 16 * kb * RS + 32 * (s + 1));
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int hb = 0; hb < NB; ++hb)
            sacc[hb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abuf[s & 1][kb], qop[hb][s],
                                                                    sacc[hb][kb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // ---- mask, online softmax (log2 domain)
      const uint64_t vm = vmask[a_cur] >> (ks * KPW);
      float tmax[NB];
#pragma unroll
      for (int hb = 0; hb < NB; ++hb) tmax[hb] = neg_inf();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = (vm >> (16 * kb + 4 * g + e)) & 1;
#pragma unroll
          for (int hb = 0; hb < NB; ++hb) {
            const float x = ok ? sacc[hb][kb][e] * p.scale_log2 : neg_inf();
            sacc[hb][kb][e] = x;
            tmax[hb] = fmaxf(tmax[hb], x);
          }
        }
      bool need_any = false;
      bool need[NB];
      float m_new[NB];
#pragma unroll
      for (int hb = 0; hb < NB; ++hb) {
        tmax[hb] = wave_xor_max(tmax[hb]);
        m_new[hb] = fmaxf(m_ref[hb], tmax[hb]);
        need[hb] = m_new[hb] > m_ref[hb] + kRescaleLog2;
        need_any |= need[hb];
      }
      if (__any(need_any)) {
#pragma unroll
        for (int hb = 0; hb < NB; ++hb) {
          const float f = need[hb] ? fast_exp2(m_ref[hb] - m_new[hb]) : 1.0f;
          m_ref[hb] = need[hb] ? m_new[hb] : m_ref[hb];
          l_part[hb] *= f;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            oacc[hb][db] *= f;
            if ((db & 3) == 3) __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
#pragma unroll
      for (int hb = 0; hb < NB; ++hb) {
        const float mu = m_ref[hb] == neg_inf() ? 0.0f : m_ref[hb];
        float ps[NKB][4];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ps[kb][e] = fast_exp2(sacc[hb][kb][e] - mu);
            l_part[hb] += ps[kb][e];
          }
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          pop[hb][kk][0] = pack_bf16(ps[2 * kk][0], ps[2 * kk][1]);
          pop[hb][kk][1] = pack_bf16(ps[2 * kk][2], ps[2 * kk][3]);
          pop[hb][kk][2] = pack_bf16(ps[2 * kk + 1][0], ps[2 * kk + 1][1]);
          pop[hb][kk][3] = pack_bf16(ps[2 * kk + 1][2], ps[2 * kk + 1][3]);
        }
      }
    }

    if (has_next) {
      stage_commit<D_QK>(st, 0, f8n, srow_dst, sq);
      stage_issue<D_QK>(st, 1, f8n, an, sq);
    }

    // ---- O^T += V^T P^T; V^T operands through the LDS transpose read.
    // Lane (g, li) addresses key row 4g + li/4 (+16 for the second half of the k-step) and
    // elements 4*(li%4)..+3 of a 16-wide d block; it receives d = db*16 + li for 4 keys.
    // Two d blocks per step (independent accumulators), operands one step ahead.
    const uint16_t *vbase = kt + (4 * g + (li >> 2)) * RS + 4 * (li & 3);
    auto load_v = [&](int db, int kk) -> bf16x8 {
      const uint16_t *src = vbase + 32 * kk * RS + 16 * db;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4 *)(src));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4 *)(src + 16 * RS));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      const u32x4 a4 = {l2[0], l2[1], h2[0], h2[1]};
      return __builtin_bit_cast(bf16x8, a4);
    };
    auto pv_range = [&](auto db0_c, auto db1_c) {
      constexpr int db0 = decltype(db0_c)::value, db1 = decltype(db1_c)::value;
      constexpr int NSTEP = (db1 - db0) / 2;
      bf16x8 vbuf[2][2][NKK];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) vbuf[0][j][kk] = load_v(db0 + j, kk);
#pragma unroll
      for (int st2 = 0; st2 < NSTEP; ++st2) {
        const int db = db0 + 2 * st2;
        if (st2 + 1 < NSTEP) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) vbuf[(st2 + 1) & 1][j][kk] = load_v(db + 2 + j, kk);
        }
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int hb = 0; hb < NB; ++hb) {
              const u32x4 b4 = {pop[hb][kk][0], pop[hb][kk][1], pop[hb][kk][2], pop[hb][kk][3]};
              oacc[hb][db + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  vbuf[st2 & 1][j][kk], __builtin_bit_cast(bf16x8, b4), oacc[hb][db + j], 0, 0, 0);
            }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (active) pv_range(std::integral_constant<int, 0>{}, std::integral_constant<int, DB / 2>{});

    if (has_next) {
      stage_commit<D_QK>(st, 1, f8n, srow_dst, sq);
      stage_issue<D_QK>(st, 2, f8n, an, sq);
    }

    if (active) pv_range(std::integral_constant<int, DB / 2>{}, std::integral_constant<int, DB>{});

    if (has_next) stage_commit<D_QK>(st, 2, f8n, srow_dst, sq);
    if (w == 0 && it + 2 < tile_end) fill_rows<TILE>(p, t, it + 2, rows[a_nn], &vmask[a_nn], lane);
    __syncthreads();
  }

  // ---- per-head totals across the four lane groups
  float l_tot[NB];
#pragma unroll
  for (int hb = 0; hb < NB; ++hb) l_tot[hb] = wave_xor_sum(l_part[hb]);

  if constexpr (NKS == 2) {
    // Merge the two key halves of each head slice through LDS (tiles are free now).
    float *xo = reinterpret_cast<float *>(&tiles[0][0]);
    float *xm = xo + NHS * NB * DB * 64 * 4;
    if (ks == 1 && active) {
#pragma unroll
      for (int hb = 0; hb < NB; ++hb) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
          *reinterpret_cast<f32x4 *>(xo + (((hs * NB + hb) * DB + db) * 64 + lane) * 4) =
              oacc[hb][db];
        xm[((hs * NB + hb) * 64 + lane) * 2 + 0] = m_ref[hb];
        xm[((hs * NB + hb) * 64 + lane) * 2 + 1] = l_tot[hb];
      }
    }
    __syncthreads();
    if (ks == 1) return;
    if (active) {
#pragma unroll
      for (int hb = 0; hb < NB; ++hb) {
        const float m1 = xm[((hs * NB + hb) * 64 + lane) * 2 + 0];
        const float l1 = xm[((hs * NB + hb) * 64 + lane) * 2 + 1];
        const float mm = fmaxf(m_ref[hb], m1);
        const float f0 = m_ref[hb] == neg_inf() ? 0.f : fast_exp2(m_ref[hb] - mm);
        const float f1 = m1 == neg_inf() ? 0.f : fast_exp2(m1 - mm);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const f32x4 o1 =
              *reinterpret_cast<const f32x4 *>(xo + (((hs * NB + hb) * DB + db) * 64 + lane) * 4);
          oacc[hb][db] = oacc[hb][db] * f0 + o1 * f1;
        }
        l_tot[hb] = l_tot[hb] * f0 + l1 * f1;
        m_ref[hb] = mm;
      }
    }
  }
  if (!active) return;

#pragma unroll
  for (int hb = 0; hb < NB; ++hb) {
    const int head = head0 + 16 * hb + li;
    if (head >= p.h) continue;
    if (p.n_chunks > 1) {
      // Split-K partial: unnormalised O, running max (log2 units) and sum.
      const int64_t row = ((int64_t)t * p.n_chunks + chunk) * p.h + head;
      float *wo = p.ws_o + row * D_V + 4 * g;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4 *>(wo + 16 * db) = oacc[hb][db];
      if (g == 0) {
        p.ws_ml[row * 2 + 0] = m_ref[hb];
        p.ws_ml[row * 2 + 1] = l_tot[hb];
      }
      continue;
    }
    const float sig = p.sink ? p.sink[head] * kLog2e : neg_inf();
    const float mf = fmaxf(m_ref[hb], sig);
    float scale = 0.f, lse = neg_inf();
    if (mf != neg_inf()) {
      const float fo = m_ref[hb] == neg_inf() ? 0.f : fast_exp2(m_ref[hb] - mf);
      const float fs = sig == neg_inf() ? 0.f : fast_exp2(sig - mf);
      const float den = l_tot[hb] * fo + fs;
      scale = fo / den;
      lse = (mf + __log2f(den)) * kLn2;
    }
    uint16_t *orow = p.out + (int64_t)t * p.out_st + (int64_t)head * p.out_sh + 4 * g;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const f32x4 o = oacc[hb][db] * scale;
      const u32x2 pk = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
      *reinterpret_cast<u32x2 *>(orow + 16 * db) = pk;
    }
    if (p.lse && g == 0) p.lse[(int64_t)t * p.lse_st + head] = lse;
  }
}

// Merge split-K partials of one (token, head) with the sink; 64 threads.
template <int D_V>
__global__ __launch_bounds__(64) void smla_combine_kernel(const KParams p) {
  const int t = blockIdx.x / p.h, head = blockIdx.x % p.h;
  const int lane = threadIdx.x;
  const int64_t base = (int64_t)t * p.n_chunks * p.h + head;
  float mmax = neg_inf();
  for (int c = 0; c < p.n_chunks; ++c) mmax = fmaxf(mmax, p.ws_ml[(base + (int64_t)c * p.h) * 2]);
  const float sig = p.sink ? p.sink[head] * kLog2e : neg_inf();
  const float mf = fmaxf(mmax, sig);
  constexpr int PER = D_V / 64;
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  float den = 0.f, lse = neg_inf();
  if (mf != neg_inf()) {
    for (int c = 0; c < p.n_chunks; ++c) {
      const int64_t row = base + (int64_t)c * p.h;
      const float mc = p.ws_ml[row * 2], lc = p.ws_ml[row * 2 + 1];
      if (mc == neg_inf()) continue;
      const float f = fast_exp2(mc - mf);
      den += lc * f;
      const float *src = p.ws_o + row * D_V + PER * lane;
#pragma unroll
      for (int j = 0; j < PER; j += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(src + j);
        acc[j] += v[0] * f;
        acc[j + 1] += v[1] * f;
        acc[j + 2] += v[2] * f;
        acc[j + 3] += v[3] * f;
      }
    }
    if (sig != neg_inf()) den += fast_exp2(sig - mf);
    lse = (mf + __log2f(den)) * kLn2;
  }
  const float inv = mf != neg_inf() ? 1.0f / den : 0.f;
  uint16_t *orow = p.out + (int64_t)t * p.out_st + (int64_t)head * p.out_sh + PER * lane;
#pragma unroll
  for (int j = 0; j < PER; j += 4) {
    const u32x2 pk = {pack_bf16(acc[j] * inv, acc[j + 1] * inv),
                      pack_bf16(acc[j + 2] * inv, acc[j + 3] * inv)};
    *reinterpret_cast<u32x2 *>(orow + j) = pk;
  }
  if (p.lse && lane == 0) p.lse[(int64_t)t * p.lse_st + head] = lse;
}

template <int D_QK, int NB, int NKS>
hipError_t launch_one(const KParams &p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.T * p.n_hg * p.n_chunks;
  hipLaunchKernelGGL((smla_attn_kernel<D_QK, NB, NKS>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     s, p);
  return hipGetLastError();
}

}  // namespace

Variant choose_variant(int d_qk, int h) {
  // One 16-head block per wave. Small head counts split each tile's keys over two waves.
  if (d_qk == 576) return h > 32 ? Variant{576, 512, 64, 1, 1} : Variant{576, 512, 64, 1, 2};
  return {1088, 1024, 32, 1, 1};
}

hipError_t launch_attention(const Variant &v, const KParams &p, hipStream_t s) {
  if (v.d_qk == 576) {
    if (v.nks == 1) return launch_one<576, 1, 1>(p, s);
    return launch_one<576, 1, 2>(p, s);
  }
  return launch_one<1088, 1, 1>(p, s);
}

hipError_t launch_combine(const Variant &v, const KParams &p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.T * p.h;
  if (v.d_v == 512)
    hipLaunchKernelGGL((smla_combine_kernel<512>), dim3((unsigned)blocks), dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL((smla_combine_kernel<1024>), dim3((unsigned)blocks), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace smla
