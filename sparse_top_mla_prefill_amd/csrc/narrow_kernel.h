// Narrow kernel for gfx950 (MI355X): few heads per token, d_qk 576, d_v 512, fp8 pools.
// Device code of both compute modes; narrow.hip builds the bf16 instance and narrow_fp8.hip
// the fp8 one, each in a translation unit of its own (with both in one, the compiler
// inlines the shared helpers differently and the bf16 instance runs slower).
//
// The same function as the wide kernels (attn.hip). At 32 or fewer heads a gathered row
// feeds few MFMAs, so the per-row costs dominate: the gather, the fp8 conversion and the
// LDS traffic. The pages size the small-head-count case separately ("[SM12x] Drop the
// 64-head TP pad on the DSv4 MLA prefill path", section Problem: prefill cost scales with
// the number of heads, which tensor parallelism divides; FlashInfer 4802 merge message,
// section "swapAB prefill": a kernel shape for small head counts).
//
// Design. One workgroup per CU walks work items (token, group of 16*HB heads) grid apart;
// the tiles of its items form one stream that never drains between items.
//   - Raw rows in LDS. Every fp8 row goes straight into LDS by LDS DMA: the 512 latent bytes
//     (16-byte chunks swizzled per row) and the nine group scales into a ring of four tile
//     slots, the 64 rope bytes into a ring of three. Tile s+2 is requested while tiles s
//     (logits) and s-1 (value product) are computed, into the slots tile s-2 left.
//   - Waves 0..3 compute logits, waves 4..7 the value product (128 of the 512 d columns, all
//     heads), waves 8..11 issue every global-to-LDS transfer; one of each per SIMD. One
//     barrier per tile: the load waves' issue stalls overlap the other waves' work.
//   - QK: logit wave w takes head block w % HB (q in registers, loaded from global memory
//     once per item) and 16 HB keys; S^T = K q^T on v_mfma_f32_16x16x32_bf16, A = 8 codes of
//     a row converted exactly to bf16, each 64-wide scale group accumulated separately and
//     S = sum_g scale[key][g] acc_g.
//   - softmax without a second barrier: each logit wave keeps its own running maximum per
//     head (log2 domain, moved lazily when it grows by more than 2^8) and row sum, and puts
//     P (bf16, in the PV B-operand order) and that maximum into LDS. The value waves keep
//     the running maximum M of the whole tile and bring each wave's P onto it with the
//     factor 2^(m_w - M), folded into the scale they multiply P by anyway; at an item's end
//     the row sum is sum_w 2^(m_w - M) l_w.
//   - PV: O^T += V^T P'^T, A = V^T by ds_read_b64_tr_b8 converted to bf16, B = P' =
//     bf16(P * scale[key][g] * 2^(m_w - M)) for the latent group g of the d block (the V
//     scale is folded into P; with P itself in bf16 that is the same two roundings a
//     dequantised V and a bf16 P make in the wide kernels).
//   - Outputs: the value waves finalise an item (sink, lse) after its last tile's product.
//   - fp8 compute mode (FQ): the pages fork the prefill kernels on an FP8 and a BF16 compute
//     mode ("fix(sparse-mla-sm120): add topk=256 prefill-dsv4 dispatch", sections Description
//     and Change; FlashInfer 4802 merge message, section "Performance vs main", which
//     quantises q in shared memory on the fp8 side). There the logit waves round q to e4m3fn
//     per (token, head) with the multiplier 448 / amax (the KV packing rule) at the first
//     tile of each item, and QK runs on v_mfma_f32_16x16x32_fp8_fp8 straight over the raw
//     codes in LDS: the K side needs no conversion at all, and the logits take back amax /
//     448. PV is unchanged (bf16).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dkern.h"
#include "smla_internal.h"
#include "walk.h"

namespace smla {

// Zero bytes that unused index entries are gathered from (a masked row must hold finite
// codes), and a sink for the stores of padded heads (every lane stores).
static __device__ __align__(256) uint8_t g_nzero[1024];
static __device__ __align__(256) uint16_t g_ndump[64 * 8 * 4];

namespace {

using namespace dk;

constexpr int kNThreads = 768;  // waves 0..3 logits, 4..7 value product, 8..11 loads
constexpr int kNLat = 4;        // latent and scale slots: tiles s-1 .. s+2
constexpr int kNRope = 3;       // rope slots: tiles s .. s+2
constexpr int kNIdx = 4;        // slot-id entries: tiles s .. s+3
constexpr int kNTile = 64;

template <int HB>
struct NSmem {
  uint8_t lat[kNLat][kNTile * kRowB];      // raw latent codes, swizzled chunks
  float sc[kNLat][kGroups][kNTile];        // latent scales [slot][group][row]
  uint8_t rope[kNRope][kNTile * 64];       // raw rope codes, chunk pairs swapped on rows 8..15 mod 16
  float scr[kNRope][kNTile];               // rope scales [slot][row]
  u32x4 pf[2][HB][2][64];                  // P (bf16) by tile parity: [head block][PV k-step][lane]
  int32_t sl[kNIdx][kNTile];               // checked slot ids (-1: unused)
  float mw[2][16 * HB][4 / HB];            // each logit wave's running max at the tile [head][wave]
  float lw[2][16 * HB][4 / HB];            // each logit wave's row sum at an item's last tile
  float sink[2][16 * HB];                  // sink logits (log2 units) of alternate items
};

static_assert(sizeof(NSmem<2>) <= 160 * 1024, "LDS of a CU");

// Row addresses from the 32-bit strides (page stride < 2^32, row stride < 2^24, checked by
// the host): one 32 x 32 -> 64-bit multiply-add and one 24-bit multiply.
__device__ __forceinline__ const uint8_t *nrow_data(const PoolArgs &pl, int32_t s) {
  const uint32_t ss = s < 0 ? 0u : (uint32_t)s;
  const uint8_t *a =
      pl.data + (uint64_t)(ss >> 6) * pl.page_stride32 + __umul24(ss & 63u, pl.row_stride32);
  return s < 0 ? g_nzero : a;
}
__device__ __forceinline__ const uint8_t *nrow_scales(const PoolArgs &pl, int32_t s) {
  const uint32_t ss = s < 0 ? 0u : (uint32_t)s;
  const uint8_t *a = pl.scales + (uint64_t)(ss >> 6) * pl.scale_page_stride32 +
                     __umul24(ss & 63u, pl.scale_row_stride32);
  return s < 0 ? g_nzero : a;
}

// Logit waves. Wave w takes head block qb = w % HB (16 heads, their q in registers) and the
// HB key blocks of 16 keys from block HB (w / HB) on; it also loads and checks the slot ids
// of index entries 16w .. 16w+15, its share of every tile's 64, three tiles ahead.
template <int HB, bool FQ>
__device__ __forceinline__ void nqk_role(const KParams &p, NSmem<HB> &sm, int w, int lane,
                                         int G) {
  const int hl = lane & 15, kq = lane >> 4;
  const int qb = w % HB, kb0 = HB * (w / HB);
  const int irow = 16 * w + hl;  // the index entry this lane loads
  // q of the item: head 16 qb + hl (a padded head reads the group's first), 8 dims 32k + 8kq
  // .. per k-step, as bf16 (qop); in the fp8 mode the bf16 rows as loaded (qraw) and their
  // e4m3fn codes (q8), with zsc = (amax / 448) * scale_log2 taking the logits back
  u32x4 qop[18];
  u32x2 q8[FQ ? 18 : 1];
  float zsc = 0.f;
  // (live false: past the last item, token 0's q is read instead, so that the registers are
  // written on every path)
  auto load_q = [&](const NCur &c, bool live) __attribute__((always_inline)) {
    const int head = (live ? c.hg : 0) * 16 * HB + 16 * qb + hl;
    const uint16_t *src = p.q + (int64_t)(live ? c.t : 0) * p.q_st +
                          (int64_t)(head < p.h ? head : 0) * p.q_sh + 8 * kq;
#pragma unroll
    for (int k = 0; k < 18; ++k) qop[k] = *(const u32x4 *)(src + 32 * k);
  };
  // fp8 mode: amax of the head's row over the four lanes that hold it, then every value
  // times fl32(448 / amax) (FLT_MAX for a zero row), clamped to +-448 and rounded to the
  // nearest e4m3fn code, ties to even
  // (amax is taken on the packed bits: the 15 magnitude bits of a finite bf16 order as its
  // absolute value does, so a 16-bit integer max of them is the max of |q|, and no value is
  // unpacked twice)
  auto quantize_q = [&]() __attribute__((always_inline)) {
    u16x2 mb = {0, 0};
#pragma unroll
    for (int k = 0; k < 18; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        mb = __builtin_elementwise_max(mb, __builtin_bit_cast(u16x2, qop[k][e] & 0x7fff7fffu));
    float amax = __uint_as_float((uint32_t)(mb[0] > mb[1] ? mb[0] : mb[1]) << 16);
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    zsc = (amax / 448.f) * p.scale_log2;
    const float inv = fminf(448.f / amax, __FLT_MAX__);
#pragma unroll
    for (int k = 0; k < 18; ++k) {
      uint32_t two[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = fminf(fmaxf(__uint_as_float(qop[k][e] << 16) * inv, -448.f), 448.f);
        const float b = fminf(fmaxf(__uint_as_float(qop[k][e] & 0xffff0000u) * inv, -448.f), 448.f);
        two[e] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
      }
      q8[FQ ? k : 0] = u32x2{two[0] | (two[1] << 16), two[2] | (two[3] << 16)};
    }
  };
  // ---- prologue: slot ids of tiles 0..2 (this wave's 16 entries), the slot-id load of
  //      tile 3, the sink load of tile 0's item and its q
  NCur cs = ncur_at(p, 0);
  NCur c3 = cs;
  {
    NCur c = cs;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int32_t v = nslot_check(p, c, irow, i < G, nslot_load(p, c, irow, i < G));
      if (kq == 0) sm.sl[i][irow] = v;
      ncur_next(p, c);
    }
    c3 = c;
  }
  NCur c4 = c3;
  ncur_next(p, c4);
  // loads one tile ahead: the raw slot id of tile s+3 and the sink of tile s's item, by parity
  // of the tile (or, in the item-wise walk, in one register each: each value is used before
  // its successor is requested)
  int32_t idxv[2];
  float snk[2];
  auto sink_load = [&](const NCur &c, bool live) -> float {
    const int hd = c.hg * 16 * HB + lane;
    return *(gf32 *)(p.sink && lane < 16 * HB && hd < p.h && live ? p.sink + hd
                                                                   : (const float *)g_nzero);
  };
  idxv[0] = nslot_load(p, c3, irow, 3 < G);
  snk[0] = sink_load(cs, 0 < G);
  load_q(cs, true);
  __syncthreads();  // (P) slot ids of tiles 0..2

  float m = neg_inf(), l_part = 0.f;

  // Tile s of the stream. rc: s mod 2, or -1 in the item-wise walk; lc: 1 for the last tile of
  // its item, 0 for another, -1 when known only at run time.
  auto body = [&](int s, auto rc, auto lc) __attribute__((always_inline)) {
    constexpr int r = decltype(rc)::value;
    constexpr int rn = r < 0 ? 0 : r ^ 1, rc0 = r < 0 ? 0 : r;
    constexpr int L = decltype(lc)::value;
    const bool last = L < 0 ? cs.j == p.n_tiles - 1 : L == 1;
    const int par = s & 1;
    __syncthreads();  // (B_s) tile s has landed; P of tile s-1 is in LDS
    // slot ids of tile s+3 (loaded in iteration s-1), then the next loads: the slot ids of
    // tile s+4 and the sink of tile s+1's item
    {
      const int32_t sid = nslot_check(p, c3, irow, s + 3 < G, idxv[rc0]);
      if (kq == 0) sm.sl[(s + 3) % kNIdx][irow] = sid;
      idxv[rn] = nslot_load(p, c4, irow, s + 4 < G);
    }
    if (lane < 16 * HB) sm.sink[cs.k & 1][lane] = snk[rc0] * kLog2e;
    NCur cn = cs;
    ncur_next(p, cn);
    snk[rn] = sink_load(cn, s + 1 < G);
    if (cs.j == 0) {
      m = neg_inf();
      l_part = 0.f;
    }
    // S^T for keys 16 (kb0 + kb) + 4kq + e, heads 16qb + hl
    const int slot = (int)opaque_u32(s % kNLat);
    const int rslot = (int)opaque_u32(s % kNRope);
    // This lane's 8 codes of k-step 0 in key block kb, as offsets in the latent and rope
    // arrays. Chunk 2k + (kq >> 1) of a row sits at chunk (2k + (kq >> 1)) ^ swz(row), i.e.
    // at byte 32 (k ^ (sw >> 1)) + 16 ((kq >> 1) ^ (sw & 1)) of the row: k-step k is the
    // k-step-0 offset with 32k XORed in (bits 5..8; the slot and row bits lie above, the rest
    // below). The rope rows swap their chunk pairs on rows 8..15 mod 16 in the same way.
    uint32_t la[HB], ra[HB];
#pragma unroll
    for (int kb = 0; kb < HB; ++kb) {
      const int row = 16 * (kb0 + kb) + hl;
      const int sw = swz(row);
      la[kb] = opaque_u32(slot * (kNTile * kRowB) + row * kRowB + 32 * (sw >> 1) +
                          16 * ((kq >> 1) ^ (sw & 1)) + 8 * (kq & 1));
      ra[kb] = opaque_u32(rslot * (kNTile * 64) + row * 64 + 32 * ((row >> 3) & 1) +
                          16 * (kq >> 1) + 8 * (kq & 1));
    }
    const uint32_t lat0 = lds_addr(sm.lat), rope0 = lds_addr(sm.rope);
    // Group g's products are scaled into S two groups later, in group order: the MFMAs of
    // three groups are in flight at once, and S is forced complete through group g - 2 at
    // each step (without that the compiler defers every scaling to the end and keeps all
    // nine accumulators live).
    constexpr int kLag = 2;
    f32x4 S[HB], acc[kGroups + 1][HB];
#pragma unroll
    for (int kb = 0; kb < HB; ++kb) S[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto scale_in = [&](int g) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < HB; ++kb) {
        const int key = 16 * (kb0 + kb) + 4 * kq;
        const f32x4 sv = g < kGroups ? *(f32x4 *)&sm.sc[slot][g][key]
                                     : *(f32x4 *)&sm.scr[rslot][key];
#pragma unroll
        for (int e = 0; e < 4; ++e) S[kb][e] += sv[e] * acc[g][kb][e];
        asm volatile("" : "+v"(S[kb]));
      }
    };
#pragma unroll
    for (int g = 0; g <= kGroups; ++g) {
#pragma unroll
      for (int kb = 0; kb < HB; ++kb) acc[g][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int k = 2 * g + s2;
#pragma unroll
        for (int kb = 0; kb < HB; ++kb) {
          const u32x2 raw = g < kGroups ? lds_load<u32x2>(lat0 + (la[kb] ^ (32 * k)))
                                        : lds_load<u32x2>(rope0 + (ra[kb] ^ (32 * s2)));
          if constexpr (FQ)
            acc[g][kb] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(
                __builtin_bit_cast(long, raw), __builtin_bit_cast(long, q8[FQ ? k : 0]),
                acc[g][kb], 0, 0, 0);
          else
            acc[g][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                codes_to_bf16(raw), __builtin_bit_cast(bf16x8, qop[k]), acc[g][kb], 0, 0, 0);
        }
      }
      if (g >= kLag) scale_in(g - kLag);
    }
#pragma unroll
    for (int g = kGroups + 1 - kLag; g <= kGroups; ++g) scale_in(g);
    // q of the next tile's item, when it starts one: requested as soon as the last MFMA of
    // this tile has read q, so that it lands behind this tile's softmax and the barrier
    if constexpr (L < 0) {
      if (s + 1 < G && cn.j == 0) load_q(cn, true);
    } else if (last) {
      load_q(cn, s + 1 < G);
    }

    // this wave's softmax: running max per head over its keys, P relative to it
    f32x4 z[HB];
    float mx = neg_inf();
#pragma unroll
    for (int kb = 0; kb < HB; ++kb) {
      const int4 sl4 = *(int4 *)&sm.sl[s % kNIdx][16 * (kb0 + kb) + 4 * kq];
      const int slv[4] = {sl4.x, sl4.y, sl4.z, sl4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        z[kb][e] = slv[e] >= 0 ? S[kb][e] * (FQ ? zsc : p.scale_log2) : neg_inf();
        mx = fmaxf(mx, z[kb][e]);
      }
    }
    mx = pair_max32(pair_max16(mx));
    const bool need = mx > m + kRescaleLog2;
    const float mnew = need ? mx : m;
    if (need) l_part *= fast_exp2(m - mnew);  // 0 while m is -inf
    m = mnew;
#pragma unroll
    for (int kb = 0; kb < HB; ++kb) {
      float pr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pr[e] = z[kb][e] != neg_inf() ? fast_exp2(z[kb][e] - m) : 0.f;
        l_part += pr[e];
      }
      // PV k-step b/2 takes key blocks b & ~1 and b | 1 as the two 8-byte halves of each
      // lane's entry, lane for lane
      const int b = kb0 + kb;
      *(lu32x2 *)((uint8_t *)&sm.pf[par][qb][b >> 1][lane] + 8 * (b & 1)) =
          u32x2{pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3])};
    }
    if (kq == 0) sm.mw[par][16 * qb + hl][w / HB] = m;
    if (last) {
      const float lw = pair_sum32(pair_sum16(l_part));
      if (kq == 0) sm.lw[par][16 * qb + hl][w / HB] = lw;
    }
    cs = cn;
    ncur_next(p, c3);
    ncur_next(p, c4);
  };
  using IC0 = std::integral_constant<int, 0>;
  using IC1 = std::integral_constant<int, 1>;
  using ICN = std::integral_constant<int, -1>;
  if constexpr (FQ) {
    // Item by item, the last tile apart: the next item's q, loaded during that tile, and this
    // item's codes are then never live together.
    for (int s = 0; s < G;) {
      quantize_q();  // the item's q has been loaded
      for (int j = 1; j < p.n_tiles; ++j) body(s++, ICN{}, IC0{});
      body(s++, ICN{}, IC1{});
    }
  } else {
    int s = 0;
    for (;;) {
      if (s >= G) break;
      body(s++, IC0{}, ICN{});
      if (s >= G) break;
      body(s++, IC1{}, ICN{});
    }
  }
  __syncthreads();  // (B_G) P of the last tile
}

// Value waves: wave 4 + u takes d columns 128u .. 128u+127 of every head of the group.
template <int HB>
__device__ __forceinline__ void npv_role(const KParams &p, NSmem<HB> &sm, int w, int lane,
                                         int G) {
  constexpr int kKW = 4 / HB;  // logit waves per head block
  const int hl = lane & 15, kq = lane >> 4;
  const int u = w - 4;
  __syncthreads();  // (P)

  f32x4 oacc[HB][8];  // O^T for d 128u + 16db + 4kq + e, head 16hb + hl
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[hb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float M[HB];        // running max of the item per head (lazy)
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) M[hb] = neg_inf();
  float f[HB][kKW];   // 2^(m_w - M) of the tile being multiplied, per logit wave
  const int lt = lane & 15, ee = lt >> 1;  // the row this lane supplies to a transpose read

  // Bring the tile's logit-wave maxima onto M: move M (and rescale O) when the tile's max
  // exceeds it by more than 2^8, then the factor of each wave.
  auto tile_factors = [&](int par, bool first) __attribute__((always_inline)) {
    bool need_any = false;
    float fo[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      if (first) M[hb] = neg_inf();
      float mw[kKW];
      float mt = neg_inf();
#pragma unroll
      for (int i = 0; i < kKW; ++i) {
        mw[i] = sm.mw[par][16 * hb + hl][i];
        mt = fmaxf(mt, mw[i]);
      }
      const bool need = mt > M[hb] + kRescaleLog2;
      const float mnew = need ? mt : M[hb];
      fo[hb] = need ? fast_exp2(M[hb] - mnew) : 1.0f;  // 0 while M is -inf
      need_any = need_any || need;
      M[hb] = mnew;
#pragma unroll
      for (int i = 0; i < kKW; ++i) f[hb][i] = mw[i] == neg_inf() ? 0.f : fast_exp2(mw[i] - M[hb]);
    }
    if (__any(need_any)) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int db = 0; db < 8; ++db) oacc[hb][db] *= fo[hb];
    }
  };
  auto pv_tile = [&](int s) __attribute__((always_inline)) {
    const int slot = s % kNLat, par = s & 1;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int key = 32 * ks + (ee < 4 ? 4 * kq + ee : 16 + 4 * kq + ee - 4);
      const uint8_t *vrow = sm.lat[slot] + key * kRowB + 8 * (lt & 1);
      const int sk = swz(key);
      // P of key blocks 2ks (values 0..3) and 2ks+1 (4..7), brought onto M
      float pl[HB][8];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const u32x4 v = sm.pf[par][hb][ks][lane];
        const float f0 = f[hb][(2 * ks) / HB], f1 = f[hb][(2 * ks + 1) / HB];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float fe = e < 2 ? f0 : f1;
          pl[hb][2 * e] = __uint_as_float(v[e] << 16) * fe;
          pl[hb][2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u) * fe;
        }
      }
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        const int g = 2 * u + g2;
        const f32x4 s0 = *(f32x4 *)&sm.sc[slot][g][32 * ks + 4 * kq];
        const f32x4 s1 = *(f32x4 *)&sm.sc[slot][g][32 * ks + 16 + 4 * kq];
        bf16x8 b[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          const u32x4 pk = {pack_bf16(pl[hb][0] * s0[0], pl[hb][1] * s0[1]),
                            pack_bf16(pl[hb][2] * s0[2], pl[hb][3] * s0[3]),
                            pack_bf16(pl[hb][4] * s1[0], pl[hb][5] * s1[1]),
                            pack_bf16(pl[hb][6] * s1[2], pl[hb][7] * s1[3])};
          b[hb] = __builtin_bit_cast(bf16x8, pk);
        }
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4) {
          const int db = 4 * g2 + d4;
          const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (li32x2 *)(vrow + 16 * ((8 * u + db) ^ sk)));
          const bf16x8 a = codes_to_bf16(__builtin_bit_cast(u32x2, raw));
#pragma unroll
          for (int hb = 0; hb < HB; ++hb)
            oacc[hb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[hb], oacc[hb][db], 0, 0, 0);
        }
      }
    }
  };
  // Outputs of the item that ends with the tile just multiplied (parity par): O / l with the
  // sink, the lse, then a fresh O. Every lane stores (padded heads into g_ndump).
  auto finish_item = [&](const NCur &ce, int par) __attribute__((always_inline)) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int head = ce.hg * 16 * HB + 16 * hb + hl;
      const bool ok = head < p.h;
      float l = 0.f;  // row sum on M over the logit waves of the head block, in wave order
#pragma unroll
      for (int i = 0; i < kKW; ++i) l += f[hb][i] * sm.lw[par][16 * hb + hl][i];
      const float sig = p.sink ? sm.sink[ce.k & 1][16 * hb + hl] : neg_inf();
      const float mf = fmaxf(M[hb], sig);
      float scale = 0.f, lse = neg_inf();
      if (mf != neg_inf()) {
        const float fo = M[hb] == neg_inf() ? 0.f : fast_exp2(M[hb] - mf);
        const float fs = sig == neg_inf() ? 0.f : fast_exp2(sig - mf);
        const float den = l * fo + fs;
        scale = fo / den;
        lse = (mf + __log2f(den)) * kLn2;
      }
      uint16_t *orow = ok ? p.out + (int64_t)ce.t * p.out_st + (int64_t)head * p.out_sh + 128 * u + 4 * kq
                          : g_ndump + 8 * lane;
      const int dstep = ok ? 16 : 0;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const u32x2 v = {pack_bf16(oacc[hb][db][0] * scale, oacc[hb][db][1] * scale),
                         pack_bf16(oacc[hb][db][2] * scale, oacc[hb][db][3] * scale)};
        *(u32x2 *)(orow + dstep * db) = v;
        oacc[hb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if (p.lse && u == hb) {
        float *dst = ok && kq == 0 ? p.lse + (int64_t)ce.t * p.lse_st + head
                                   : reinterpret_cast<float *>(g_ndump) + lane;
        *dst = lse;
      }
    }
  };

  NCur cp = ncur_at(p, 0);  // tile s-1
  __syncthreads();  // (B_0)
  for (int s = 1; s <= G; ++s) {
    __syncthreads();  // (B_s) P and maxima of tile s-1 are in LDS
    const int par = (s - 1) & 1;
    tile_factors(par, cp.j == 0);
    pv_tile(s - 1);
    if (cp.j == p.n_tiles - 1) finish_item(cp, par);
    ncur_next(p, cp);
  }
}

// Load waves: every global-to-LDS transfer of the stream. A load wave stalls while the
// memory queue of the CU is full; those stalls overlap the other waves' work.
template <int HB>
__device__ __forceinline__ void nld_role(const KParams &p, NSmem<HB> &sm, int w, int lane,
                                         int G) {
  const int u = w - 8;
  // loads of one tile by this wave: 8 latent row pairs, 2 latent scale groups, 16 rows of
  // rope codes, and (load wave 0) the rope scales
  const int n_tile_loads = 11 + (u == 0 ? 1 : 0);
  auto issue_tile = [&](int s, const NCur &c) __attribute__((always_inline)) {
    const PoolArgs &pl = c.j < p.main_tiles ? p.kv : p.ex;
    const int slot = s % kNLat, rslot = s % kNRope, islot = s % kNIdx;
    int32_t s8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) s8[i] = sm.sl[islot][2 * (u + 4 * i) + (lane >> 5)];
    const int32_t ssc = sm.sl[islot][lane];
    const int rrow = 16 * u + (lane >> 2);  // rope row of this lane
    const int32_t srp = sm.sl[islot][rrow];
    const uint8_t *src[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rr = 2 * (u + 4 * i) + (lane >> 5);
      src[i] = nrow_data(pl, s8[i]) + 16 * ((lane & 31) ^ swz(rr));
    }
    const uint8_t *scs = nrow_scales(pl, ssc);
    const uint8_t *rsrc =
        nrow_data(pl, srp) + kRowB + 16 * ((lane & 3) ^ (2 * ((rrow >> 3) & 1)));
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(src[i], sm.lat[slot] + 1024 * (u + 4 * i));
#pragma unroll
    for (int i = 0; i < 2; ++i) dma4(scs + 4 * (2 * u + i), &sm.sc[slot][2 * u + i][0]);
    dma16(rsrc, sm.rope[rslot] + 1024 * u);
    if (u == 0) dma4(scs + 4 * kGroups, &sm.scr[rslot][0]);
  };

  NCur c1 = ncur_at(p, 0);
  ncur_next(p, c1);  // tile s+1
  NCur c2 = c1;
  ncur_next(p, c2);  // tile s+2
  __syncthreads();  // (P) slot ids of tiles 0..2
  issue_tile(0, ncur_at(p, 0));
  if (1 < G) issue_tile(1, c1);
  wait_vmcnt_rt(1 < G ? n_tile_loads : 0);  // tile 0 has landed
  __syncthreads();  // (B_0)
  for (int s = 0; s < G; ++s) {
    // tile s+2 into the slots tile s-2 left (its slot ids came in iteration s-1)
    if (s + 2 < G) issue_tile(s + 2, c2);
    // tile s+1 has landed: only tile s+2's loads may still be in flight
    wait_vmcnt_rt(s + 2 < G ? n_tile_loads : 0);
    __syncthreads();  // (B_s+1)
    ncur_next(p, c1);
    ncur_next(p, c2);
  }
}

template <int HB, bool FQ>
__global__ __launch_bounds__(kNThreads, 1) void smla_narrow_kernel(const KParams p) {
  __shared__ __attribute__((aligned(16))) NSmem<HB> sm;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int total = p.T * p.n_hg;
  const int n_items = (total - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int G = n_items * p.n_tiles;
  if (w < 4)
    nqk_role<HB, FQ>(p, sm, w, lane, G);
  else if (w < 8)
    npv_role<HB>(p, sm, w, lane, G);
  else
    nld_role<HB>(p, sm, w, lane, G);
}

}  // namespace
}  // namespace smla
