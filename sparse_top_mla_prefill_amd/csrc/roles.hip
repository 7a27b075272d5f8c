// Role-split kernel for gfx950 (MI355X): prefill form, more than 32 heads (64 per work
// item), d_qk 576, d_v 512, fp8 pools, bf16 compute.
//
// The same function as the wide kernels (attn.hip), with the same latent operands: each
// gathered fp8 latent value is dequantised once (code times its fp32 group scale, rounded to
// bf16), q is bf16, and the MFMAs accumulate in fp32. The rope part of a logit is taken on
// the exact codes and multiplied by the row's rope scale in fp32 (one rounding fewer than
// the wide kernels' bf16 rope values). All heads of a token share one latent KV head ("[SM12x] Drop the 64-head TP pad on the DSv4 MLA prefill
// path", section Problem), so one gathered row feeds 64 heads here.
//
// Design. One workgroup per CU walks work items (token, group of 64 heads) grid apart, as one
// stream of 64-key tiles that never drains between items (the item order of walk.h: the two
// head groups of a token run on one XCD and share its L2).
//   - Two wave roles, one wave of each per SIMD, and one barrier per tile.
//     Logit waves 0..3: wave (hh, kh) = (w & 1, w >> 1) computes S^T for heads 32hh..32hh+31
//     and keys 32kh..32kh+31 of tile s on v_mfma_f32_32x32x16_bf16 (A: one key row per lane,
//     read from LDS; B: q of the item, in registers), then its part of the softmax, and puts
//     P (bf16, in the PV B-operand order) and its running maxima into LDS. They also check
//     the slot ids of tile s+3 and store each entry's row data and scale addresses, which
//     the value waves load from.
//     Value waves 4..7: wave u owns d columns 128u..128u+127. It computes O^T += V^T P^T for
//     its 128 d and all 64 heads over tile s-1 (A: V^T by ds_read_b64_tr_b16 from the bf16
//     tile, B: P from LDS), and after each 16-key step of that product writes the same 16
//     rows of its d slice of tile s+1 into the buffer the step has just read (fp8 codes loaded
//     into registers one tile earlier, times their group scale, rounded to bf16), then issues
//     the loads of those rows of tile s+2. Each value wave also moves a quarter of the rope
//     codes (raw) and rope scales.
//   - LDS: two bf16 tiles of 64 rows. A row holds the 512 latent values, then in its padding
//     the 64 raw rope codes: 1104 bytes, 69 units of 16 (69 = 5 mod 32, so the QK operand
//     reads of 32 rows and the rope reads fall in distinct banks, and each quarter of the
//     transpose reads of PV touches four disjoint 64-byte spans). The rope scales, P, the
//     maxima and the entries' row addresses are double-buffered by tile parity, the entries'
//     logit offsets four tiles deep. QK takes the rope (exact codes) and the latent (operands
//     read three k-steps ahead) in accumulators of their own, and adds the rope part times
//     each key's rope scale at the end.
//   - Softmax without a second barrier: each logit wave keeps its own running maximum per
//     head over its 32 keys, an integer in log2 units, moved to the ceiling of the new
//     maximum only when that grows by more than 2^8 (so P <= 2^8). The value waves keep M,
//     the largest of those maxima seen in the item, and bring a wave's P onto M by
//     2^(m_w - M): an exact power of two, applied to the packed bf16 P as a saturating
//     integer subtract from its exponent field. At an item's end the row sum is
//     sum_w 2^(m_w - M) l_w.
//   - The sink and lse as in the wide kernels (FlashInfer 4802 merge message, section
//     Summary); the value waves store the outputs of an item after its last product.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "dkern.h"
#include "smla_internal.h"
#include "walk.h"

namespace smla {

// Zero bytes that unused index entries are gathered from (their rows then hold zeros), and
// a sink for the stores of padded heads (every lane stores).
static __device__ __align__(256) uint8_t g_rzero[1024];
static __device__ __align__(256) uint16_t g_rdump[64 * 8 * 4];

namespace {

using namespace dk;

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((address_space(1))) const u32x4 gu32x4;
typedef __attribute__((address_space(3))) i16x4 li16x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint64_t)))) uint64_t u64x2;

constexpr int kRThreads = 512;         // waves 0..3 logits, 4..7 value product and staging
constexpr int kRStride = 552;          // bf16 elements per LDS row
constexpr int kRRowB = 2 * kRStride;   // 1104 bytes
constexpr int kRRopeB = 1024;          // raw rope codes at this byte of an LDS row
constexpr int kRIdx = 4;               // logit-offset entries: tiles s .. s+3

struct RSmem {
  uint16_t lat[2][64 * kRStride];  // tiles by parity
  u32x4 pf[2][2][4][64];           // P (bf16) by parity: [head block][PV k-step][lane]
  uint64_t rp[2][64][2];           // row data and scale addresses of each entry, by parity
  float kbias[kRIdx][64];          // logit offset of each entry: 0, or -inf when unused
  float mw[2][2][64];              // each logit wave's running max at the tile [key half][head]
  float lw[2][2][64];              // each logit wave's row sum at an item's last tile
  float sink[2][64];               // sink logits (log2 units) of alternate items
  float rsc[2][64];                // rope scales of the rows, by parity
};
static_assert(sizeof(RSmem) <= 160 * 1024, "LDS of a CU");

// Calls f(std::integral_constant<int, k>) for k = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void rfor(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    rfor<B + 1, E>(f);
  }
}

// Row addresses from the 32-bit strides (page stride < 2^32, row stride < 2^24, checked by
// the host): the data and the scales of slot s; an unused entry (s < 0) reads the zero row.
struct RowPtr {
  const uint8_t *data, *scales;
};
__device__ __forceinline__ RowPtr row_ptr(const PoolArgs &pl, int32_t s) {
  const uint32_t ss = s < 0 ? 0u : (uint32_t)s;
  const uint64_t page = ss >> 6;
  const uint32_t off = ss & 63u;
  const uint8_t *d = pl.data + page * pl.page_stride32 + __umul24(off, pl.row_stride32);
  const uint8_t *c = pl.scales + page * pl.scale_page_stride32 + __umul24(off, pl.scale_row_stride32);
  return RowPtr{s < 0 ? g_rzero : d, s < 0 ? g_rzero : c};
}

// Two e4m3fn codes (bytes 0, 1 or 2, 3 of w) times an fp32 scale -> two packed bf16: exact
// conversion, one fp32 product, one rounding to nearest even.
__device__ __forceinline__ uint32_t dq2(uint32_t w, float s, bool hi) {
  const f32x2 f = hi ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true)
                     : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
  return pack_bf16(f[0] * s, f[1] * s);
}

// P (8 packed bf16, all >= 0) times 2^-d, d in 0..255 given as s2 = d << 7 in both halves:
// the exponent field less d, saturating at zero (a value whose exponent does not exceed d
// becomes zero or a subnormal below 2^-126).
// (Written out element by element: with the same expression assigned to r[e] in a loop over
// e, this compiler keeps element 0 only and copies it into all four.)
__device__ __forceinline__ uint32_t psub(uint32_t v, uint32_t s2) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(
                                          __builtin_bit_cast(u16x2, v), __builtin_bit_cast(u16x2, s2)));
}
__device__ __forceinline__ u32x4 pshift(u32x4 v, uint32_t s2) {
  return u32x4{psub(v[0], s2), psub(v[1], s2), psub(v[2], s2), psub(v[3], s2)};
}

// The data and scale addresses of a tile's entry (the zero row for an unused one), written by
// lanes 0..15 of a logit wave for entries 16w .. 16w+15.
__device__ __forceinline__ void put_rows(const KParams &p, RSmem &sm, const NCur &c, int par,
                                         int entry, int32_t sid, int lane) {
  const RowPtr a = row_ptr(c.j < p.main_tiles ? p.kv : p.ex, sid);
  if (lane < 16) {
    sm.rp[par][entry][0] = (uint64_t)(uintptr_t)a.data;
    sm.rp[par][entry][1] = (uint64_t)(uintptr_t)a.scales;
  }
}

// Logit waves. Wave w: head block hh = w & 1, key half kh = w >> 1. Lane (j, kg) = (lane & 31,
// lane >> 5) holds S^T for head 32hh + j and keys 32kh + 8(e/4) + 4kg + e%4, e = 0..15. It
// also loads and checks the slot ids of index entries 16w .. 16w+15 three tiles ahead.
__device__ __forceinline__ void rqk_role(const KParams &p, RSmem &sm, int w, int lane, int G) {
  const int hh = w & 1, kh = w >> 1;
  const int j = lane & 31, kg = lane >> 5;
  const int irow = 16 * w + (lane & 15);  // the index entry this lane loads
  // q of the item: head 32hh + j (a padded head reads the group's first), dims 16k + 8kg ..
  // +7 of k-step k
  u32x4 q[36];
  auto load_q = [&](const NCur &c, bool live) __attribute__((always_inline)) {
    const int head = (live ? c.hg : 0) * 64 + 32 * hh + j;
    const uint16_t *src = p.q + (int64_t)(live ? c.t : 0) * p.q_st +
                          (int64_t)(head < p.h ? head : 0) * p.q_sh + 8 * kg;
#pragma unroll
    for (int k = 0; k < 36; ++k) q[k] = *(gu32x4 *)(src + 16 * k);
  };
  auto sink_load = [&](const NCur &c, bool live) -> float {
    const int hd = c.hg * 64 + lane;
    return *(gf32 *)(p.sink && hd < p.h && live ? p.sink + hd : (const float *)g_rzero);
  };
  // ---- prologue: entries of tiles 0..2 (this wave's 16; the row addresses of tile 2 go
  //      into parity 0 once tile 0's are consumed), the slot-id load of tile 3, the sink of
  //      tile 0's item and its q
  NCur cs = ncur_at(p, 0);
  NCur c3 = cs;
  NCur c2p = cs;
  int32_t sid2 = -1;
  {
    NCur c = cs;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int32_t v = nslot_check(p, c, irow, i < G, nslot_load(p, c, irow, i < G));
      if (lane < 16) sm.kbias[i][irow] = v >= 0 ? 0.f : neg_inf();
      if (i < 2)
        put_rows(p, sm, c, i, irow, v, lane);
      else {
        c2p = c;
        sid2 = v;
      }
      ncur_next(p, c);
    }
    c3 = c;
  }
  NCur c4 = c3;
  ncur_next(p, c4);
  // loads one tile ahead, by parity of the tile: the raw slot id of tile s+3 and the sink of
  // tile s's item
  int32_t idxv[2];
  float snk[2];
  idxv[0] = nslot_load(p, c3, irow, 3 < G);
  snk[0] = sink_load(cs, 0 < G);
  load_q(cs, true);
  __syncthreads();  // (P) entries of tiles 0 and 1
  __syncthreads();  // (B_0) tile 0 is in LDS, tile 0's row addresses consumed
  put_rows(p, sm, c2p, 0, irow, sid2, lane);
  __syncthreads();  // (B_0b) entries of tile 2

  float m = neg_inf(), l_part = 0.f;

  auto body = [&](int s, auto rc) __attribute__((always_inline)) {
    constexpr int r = decltype(rc)::value, rn = r ^ 1;
    const int par = s & 1;
    const bool last = cs.j == p.n_tiles - 1;
    {
      const int32_t sid = nslot_check(p, c3, irow, s + 3 < G, idxv[r]);
      if (lane < 16) sm.kbias[(s + 3) % kRIdx][irow] = sid >= 0 ? 0.f : neg_inf();
      put_rows(p, sm, c3, (s + 3) & 1, irow, sid, lane);
      idxv[rn] = nslot_load(p, c4, irow, s + 4 < G);
    }
    if (w == 0) sm.sink[cs.k & 1][lane] = snk[r] * kLog2e;
    NCur cn = cs;
    ncur_next(p, cn);
    snk[rn] = sink_load(cn, s + 1 < G);
    if (cs.j == 0) {
      m = neg_inf();
      l_part = 0.f;
    }
    // ---- S^T = K q^T over the 64 rope dims (raw codes in the rows' padding) and the 512
    //      latent dims (bf16)
    const uint32_t row = lds_addr(sm.lat[par]) + (uint32_t)(32 * kh + j) * kRRowB;
    const uint32_t abase = row + 16 * kg;
    // rope dims on the exact codes (e4m3fn -> bf16) into an accumulator of their own, scaled
    // by each key's rope scale once the latent products are in (so the latent chain does not
    // wait on the rope products)
    f32x16 S = {}, Sr = {};
    f32x4 r4[4];
    {
      u32x2 rraw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) rraw[i] = lds_load<u32x2>(row + kRRopeB + 16 * i + 8 * kg);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        Sr = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            codes_to_bf16(rraw[k]), __builtin_bit_cast(bf16x8, q[32 + k]), Sr, 0, 0, 0);
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) r4[b4] = *(f32x4 *)&sm.rsc[par][32 * kh + 8 * b4 + 4 * kg];
    }
    constexpr int LA = 3;  // operand reads ahead of their MFMA
    u32x4 ab[LA + 1];
#pragma unroll
    for (int k = 0; k < LA; ++k) ab[k] = lds_load<u32x4>(abase + 32 * k);
    rfor<0, 32>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      if constexpr (k + LA < 32) ab[(k + LA) % (LA + 1)] = lds_load<u32x4>(abase + 32 * (k + LA));
      const bf16x8 a = __builtin_bit_cast(bf16x8, ab[k % (LA + 1)]);
      const bf16x8 b = __builtin_bit_cast(bf16x8, q[k]);
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, S, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int b4 = 0; b4 < 4; ++b4)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[4 * b4 + e] = fmaf(Sr[4 * b4 + e], r4[b4][e], S[4 * b4 + e]);
    // q of the next tile's item, when it starts one: requested once the last MFMA has read q
    if (s + 1 < G && cn.j == 0) load_q(cn, true);

    // ---- this wave's softmax: running max per head over its keys, P relative to it. An
    //      unused entry's logit is -inf (its offset), and so its P is 0: exp2(-inf - mu)
    //      with mu = m, or 0 while no key has been valid.
    float z[16];
    float mx = neg_inf();
#pragma unroll
    for (int b4 = 0; b4 < 4; ++b4) {
      const f32x4 kb4 = *(f32x4 *)&sm.kbias[s % kRIdx][32 * kh + 8 * b4 + 4 * kg];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        z[4 * b4 + e] = fmaf(S[4 * b4 + e], p.scale_log2, kb4[e]);
        mx = fmaxf(mx, z[4 * b4 + e]);
      }
    }
    mx = pair_max32(mx);
    const bool need = mx > m + kRescaleLog2;
    const float mnew = need ? ceilf(mx) : m;
    if (need) l_part *= fast_exp2(m - mnew);  // 0 while m is -inf
    m = mnew;
    const float mu = m == neg_inf() ? 0.f : m;
    float pr[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      pr[e] = fast_exp2(z[e] - mu);
      l_part += pr[e];
    }
    // PV k-step 2kh + b takes this lane's values 8b .. 8b+7, lane for lane
#pragma unroll
    for (int b = 0; b < 2; ++b)
      sm.pf[par][hh][2 * kh + b][lane] =
          u32x4{pack_bf16(pr[8 * b], pr[8 * b + 1]), pack_bf16(pr[8 * b + 2], pr[8 * b + 3]),
                pack_bf16(pr[8 * b + 4], pr[8 * b + 5]), pack_bf16(pr[8 * b + 6], pr[8 * b + 7])};
    if (lane < 32) sm.mw[par][kh][32 * hh + j] = m;
    if (last) {
      const float lw = pair_sum32(l_part);
      if (lane < 32) sm.lw[par][kh][32 * hh + j] = lw;
    }
    cs = cn;
    ncur_next(p, c3);
    ncur_next(p, c4);
    __syncthreads();  // (B_s+1) P of tile s is in LDS; tile s+1 has been written
  };
  using IC0 = std::integral_constant<int, 0>;
  using IC1 = std::integral_constant<int, 1>;
  int s = 0;
  for (;;) {
    if (s >= G) break;
    body(s++, IC0{});
    if (s >= G) break;
    body(s++, IC1{});
  }
}

// Value waves: wave 4 + u owns d columns 128u .. 128u+127 of every head of the group.
__device__ __forceinline__ void rpv_role(const KParams &p, RSmem &sm, int w, int lane, int G) {
  const int u = w - 4;
  const int j = lane & 31, kg = lane >> 5;
  // Staging: block b (the rows of 16-key step b of PV) is rows 16b + (lane >> 2); lane
  // takes the 32 codes at d 128u + 32(lane & 3) of its row (two 16-byte loads, four 16-byte
  // LDS writes; the 16 lanes of one LDS write pass cover 4 consecutive rows, 80 bytes apart
  // modulo 256, so their 64-byte pieces fall in distinct banks) and the group scale of
  // those codes. Rope: rows 16u + (lane >> 4) + 4((lane >> 2) & 3) (again 4 rows 4 apart per
  // write pass), codes 16(lane & 3) .. +15, and the rope scale.
  const int c4 = lane & 3;
  const int brow = lane >> 2;
  const int rrow = 16 * u + (lane >> 4) + 4 * ((lane >> 2) & 3);
  u32x4 cv[4][2];
  float cs[4];
  u32x4 rv;
  float rs;
  auto rows_of = [&](int par, int entry) __attribute__((always_inline)) {
    const u64x2 v = *(const u64x2 *)&sm.rp[par][entry][0];
    return RowPtr{(const uint8_t *)(uintptr_t)v[0], (const uint8_t *)(uintptr_t)v[1]};
  };
  auto issue_block = [&](int b, int par) __attribute__((always_inline)) {
    const RowPtr a = rows_of(par, 16 * b + brow);
    const uint8_t *src = a.data + 128 * u + 32 * c4;
    cv[b][0] = *(gu32x4 *)(src);
    cv[b][1] = *(gu32x4 *)(src + 16);
    cs[b] = *(gf32 *)(a.scales + 4 * (2 * u + (c4 >> 1)));
  };
  auto issue_rope = [&](int par) __attribute__((always_inline)) {
    const RowPtr a = rows_of(par, rrow);
    rv = *(gu32x4 *)(a.data + kRowB + 16 * (lane & 3));
    rs = *(gf32 *)(a.scales + 4 * kGroups);
  };
  auto commit_block = [&](int b, int buf) __attribute__((always_inline)) {
    uint8_t *dst = (uint8_t *)sm.lat[buf] + (16 * b + brow) * kRRowB + 256 * u + 64 * c4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 v = cv[b][h];
      const float sc = cs[b];
      *(lu32x4 *)(dst + 32 * h) = u32x4{dq2(v[0], sc, false), dq2(v[0], sc, true),
                                        dq2(v[1], sc, false), dq2(v[1], sc, true)};
      *(lu32x4 *)(dst + 32 * h + 16) = u32x4{dq2(v[2], sc, false), dq2(v[2], sc, true),
                                             dq2(v[3], sc, false), dq2(v[3], sc, true)};
    }
  };
  auto commit_rope = [&](int buf) __attribute__((always_inline)) {
    uint8_t *dst = (uint8_t *)sm.lat[buf] + rrow * kRRowB;
    *(lu32x4 *)(dst + kRRopeB + 16 * (lane & 3)) = rv;
    if ((lane & 3) == 0) sm.rsc[buf][rrow] = rs;
  };

  f32x16 oacc[4][2];  // O^T [d block][head block]: d 128u + 32db + 8(e/4) + 4kg + e%4, head 32hb + j
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) oacc[db][hb] = f32x16{};
  float M[2] = {neg_inf(), neg_inf()};  // running max of the item per head block (eager)
  uint32_t sh[2][2];                    // P exponent shift (d << 7, both halves) [hb][kh]

  // Bring the tile's logit-wave maxima onto M: M grows to the largest of them (rescaling O),
  // then each wave's shift M - m_w.
  auto tile_factors = [&](int par, bool first) __attribute__((always_inline)) {
    bool need_any = false;
    float fo[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      if (first) M[hb] = neg_inf();
      const float ma = sm.mw[par][0][32 * hb + j], mb = sm.mw[par][1][32 * hb + j];
      const float mt = fmaxf(ma, mb);
      const bool need = mt > M[hb];
      const float mnew = need ? mt : M[hb];
      fo[hb] = need ? fast_exp2(M[hb] - mnew) : 1.0f;  // 0 while M is -inf
      need_any = need_any || need;
      M[hb] = mnew;
      const float mk[2] = {ma, mb};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t d = mk[k] == neg_inf() ? 255u : (uint32_t)fminf(mnew - mk[k], 255.f);
        sh[hb][k] = (d << 7) | (d << 23);
      }
    }
    if (__any(need_any)) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) oacc[db][hb] *= fo[hb];
    }
  };

  // V^T operand of PV: lane (G, lt) = (lane >> 4, lane & 15) reads key rows 4(lane >> 5) +
  // lt / 4 and 8 more of the 16-key step, 4 elements from d 32db + 16(G & 1) + 4(lt & 3) of
  // this wave's slice; the two transposed reads give the 32x32x16 A operand whose k order is
  // keys {0..3, 8..11} (lanes 0..31) and {4..7, 12..15} (lanes 32..63), the order of P.
  const int G4 = lane >> 4, lt = lane & 15;
  const int voff = (4 * kg + (lt >> 2)) * kRStride + 128 * u + 16 * (G4 & 1) + 4 * (lt & 3);
  auto load_v = [&](const uint16_t *tile, int kb, int db) __attribute__((always_inline)) {
    const uint16_t *src = tile + voff + 16 * kb * kRStride + 32 * db;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4 *)(src));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4 *)(src + 8 * kRStride));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    const u32x4 a4 = {l2[0], l2[1], h2[0], h2[1]};
    return __builtin_bit_cast(bf16x8, a4);
  };

  // Outputs of the item that ends with the tile just multiplied (parity par): O / l with the
  // sink, the lse, then a fresh O. Every lane stores (padded heads into g_rdump).
  auto finish_item = [&](const NCur &ce, int par) __attribute__((always_inline)) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int head = ce.hg * 64 + 32 * hb + j;
      const bool ok = head < p.h;
      float l = 0.f;  // row sum on M over the two logit waves of the head block
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float mk = sm.mw[par][k][32 * hb + j];
        l += (mk == neg_inf() ? 0.f : fast_exp2(mk - M[hb])) * sm.lw[par][k][32 * hb + j];
      }
      const float sig = p.sink ? sm.sink[ce.k & 1][32 * hb + j] : neg_inf();
      const float mf = fmaxf(M[hb], sig);
      float scale = 0.f, lse = neg_inf();
      if (mf != neg_inf()) {
        const float fo = M[hb] == neg_inf() ? 0.f : fast_exp2(M[hb] - mf);
        const float fs = sig == neg_inf() ? 0.f : fast_exp2(sig - mf);
        const float den = l * fo + fs;
        scale = fo / den;
        lse = (mf + __log2f(den)) * kLn2;
      }
      uint16_t *orow = ok ? p.out + (int64_t)ce.t * p.out_st + (int64_t)head * p.out_sh +
                                128 * u + 4 * kg
                          : g_rdump + 8 * lane;
      const int dstep = ok ? 1 : 0;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const u32x2 v = {pack_bf16(oacc[db][hb][4 * e4] * scale, oacc[db][hb][4 * e4 + 1] * scale),
                           pack_bf16(oacc[db][hb][4 * e4 + 2] * scale, oacc[db][hb][4 * e4 + 3] * scale)};
          *(u32x2 *)(orow + dstep * (32 * db + 8 * e4)) = v;
        }
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db][hb] = f32x16{};
      if (p.lse && u == hb) {
        float *dst = ok && kg == 0 ? p.lse + (int64_t)ce.t * p.lse_st + head
                                   : reinterpret_cast<float *>(g_rdump) + lane;
        *dst = lse;
      }
    }
  };

  // One iteration s: the product of tile s-1 (when PV), each 16-key step followed by the
  // staging of the same rows of tile s+1 into the buffer it has read and the loads of those
  // rows of tile s+2 (when ST).
  NCur cp = ncur_at(p, 0);  // tile s-1
  auto step = [&](int s, auto pvc, auto stc) __attribute__((always_inline)) {
    constexpr bool PV = decltype(pvc)::value, ST = decltype(stc)::value;
    const int par = (s - 1) & 1, buf = (s + 1) & 1;
    const int ipar = s & 1;  // row addresses of tile s+2
    if constexpr (PV) tile_factors(par, cp.j == 0);
    const uint16_t *tile = sm.lat[par];
    rfor<0, 4>([&](auto kc) __attribute__((always_inline)) {
      constexpr int kb = decltype(kc)::value;
      if constexpr (PV) {
        bf16x8 pb[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          pb[hb] = __builtin_bit_cast(bf16x8, pshift(sm.pf[par][hb][kb][lane], sh[hb][kb >> 1]));
        bf16x8 va[2];
        va[0] = load_v(tile, kb, 0);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          if (db + 1 < 4) va[(db + 1) & 1] = load_v(tile, kb, db + 1);
#pragma unroll
          for (int hb = 0; hb < 2; ++hb)
            oacc[db][hb] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db & 1], pb[hb], oacc[db][hb], 0, 0, 0);
        }
      }
      if constexpr (ST) {
        commit_block(kb, buf);
        issue_block(kb, ipar);
      }
    });
    if constexpr (ST) {
      commit_rope(buf);
      issue_rope(ipar);
    }
    if constexpr (PV) {
      if (cp.j == p.n_tiles - 1) finish_item(cp, par);
      ncur_next(p, cp);
    }
  };

  __syncthreads();  // (P) entries of tiles 0 and 1
  // tile 0 into buffer 0, tile 1's loads in flight
  {
#pragma unroll
    for (int b = 0; b < 4; ++b) issue_block(b, 0);
    issue_rope(0);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      commit_block(b, 0);
      issue_block(b, 1);
    }
    commit_rope(0);
    issue_rope(1);
  }
  __syncthreads();  // (B_0)
  __syncthreads();  // (B_0b) entries of tile 2
  using T_ = std::true_type;
  using F_ = std::false_type;
  step(0, F_{}, T_{});  // tile 1 into buffer 1, tile 2's loads
  __syncthreads();      // (B_1)
  for (int s = 1; s < G; ++s) {
    step(s, T_{}, T_{});
    __syncthreads();  // (B_s+1)
  }
  step(G, T_{}, F_{});
}

__global__ __launch_bounds__(kRThreads, 1) void smla_roles_kernel(const KParams p) {
  __shared__ __attribute__((aligned(16))) RSmem sm;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int total = p.T * p.n_hg;
  const int n_items = (total - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int G = n_items * p.n_tiles;
  if (G <= 0) return;
  if (w < 4) {
    rqk_role(p, sm, w, lane, G);
  } else {
    // The value waves carry the longer chain of a tile (the product, then the staging of
    // each block behind it), and a SIMD runs the MFMAs and the vector work of its two waves
    // largely one after the other: issuing the value wave's instructions first when both
    // are ready shortens the tile (T=8192, h=128, topk=2048: 6.09 -> 5.67 ms; raising the
    // priority only around the staging or only around the product gains nothing).
    __builtin_amdgcn_s_setprio(2);
    rpv_role(p, sm, w, lane, G);
  }
}

}  // namespace

hipError_t launch_roles(const KParams &p, hipStream_t s) {
  if (p.T <= 0 || p.n_tiles <= 0 || p.grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(smla_roles_kernel, dim3(p.grid), dim3(kRThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace smla
