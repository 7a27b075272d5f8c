// Decode kernel for gfx950 (MI355X): few query tokens, d_qk 576, d_v 512, fp8 pools.
//
// What is computed is the same function as the wide kernels (attn.hip): for token t and
// head h, o = sum_j e^{z_j} v_j / (sum_j e^{z_j} + e^{sink_h}) over the token's valid top-k
// rows. The pages frame decode as bound by the KV gather, not by the math ("[SM12x] Drop the
// 64-head TP pad on the DSv4 MLA prefill path", section Problem), and split a decode row's
// index list over workgroups with a merge of the partial results (FlashInfer 4802 merge
// message inside "fix(sm120): explain sparse-MLA decode dispatch misses; add config query
// API", sections "Runner and CUDA graphs" and "Dispatch: cpb model + crossover").
//
// Design. A workgroup of 8 waves serves one work item: 16 heads of one token and a chunk of
// at most 4 index tiles of 64 keys. The whole chunk is resident in LDS, so every gather of
// the item is issued at once, right after its slot ids arrive:
//   - the 512 latent bytes of each fp8 row go straight from global memory into LDS
//     (global_load_lds_dwordx4, 16-byte chunks swizzled per row), raw, not dequantised;
//   - the eight latent scales of each row go into LDS the same way, as [tile][group][row];
//   - the 64 rope bytes and the rope scale of each row go into registers of the wave that
//     computes that row's logits.
// Waves 0..3 compute logits, waves 4..7 the value product; the two kinds pair up on each
// SIMD, so one's vector work runs beside the other's MFMAs.
//   QK (wave w, 16 keys 16w.. of each tile): S^T = K q^T on v_mfma_f32_16x16x32_bf16.
//     A = 8 fp8 codes of one row read from LDS and converted exactly to bf16; B = q in
//     registers. A row's scale differs per 64-wide group of d, so each group's two MFMAs go
//     into a fresh accumulator that is added to S times that group's per-key scale.
//   softmax: log2 domain, running max per head shared by all waves (tile maxima meet in
//     LDS), lazily moved when it grows by more than 2^8. P = 2^(S - m) times the key's
//     scale of latent group g is written, as bf16, for each of the 8 latent groups: the
//     scale of V is folded into P, so V is used as raw codes.
//   PV (wave 4+u, d columns 128u..128u+127 = latent groups 2u, 2u+1): O^T += V^T P'^T on
//     v_mfma_f32_16x16x32_bf16, A = V^T by ds_read_b64_tr_b8 (LDS transpose read of 8 keys
//     x 16 codes) converted to bf16, B = the P' of the block's group.
// A key's index in the PV k dimension is permuted so that each QK lane's four P values are
// one 8-byte half of a PV B-operand entry; the transpose reads of V use the same order.
// Split items: every chunk of a (token, 16 heads) writes O / l in bf16 and (m, l) to the
// workspace and then counts itself in; the chunk that completes the count merges. The merge
// takes every chunk in chunk order and in its stored form, so the result does not depend on
// the order of arrival; the counter is left at zero for the next call.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "dkern.h"
#include "smla_internal.h"

namespace smla {

// Arrival counters of split items, one per (token, head group) of a call; every call takes
// its own range of this pool (handed out round-robin by the host) and leaves it zero.
static __device__ __align__(256) uint32_t g_arrivals[kArrivalSlots];
// Zero bytes that unused index entries are gathered from (a masked row must hold finite
// codes: an e4m3fn NaN code times a zero weight would still be NaN).
static __device__ __align__(256) uint8_t g_zero_row[1024];

hipError_t arrival_region(uint32_t **ptr) {
  static std::mutex mu;
  static void *addr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_arrivals));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = static_cast<uint32_t *>(addr[dev]);
  return hipSuccess;
}

namespace {

using namespace dk;

constexpr int kDThreads = 512;  // 8 waves: 0..3 QK, 4..7 PV
constexpr int kDTile = 64;      // keys per index tile
constexpr int kDHeads = 16;     // heads per workgroup
constexpr int kDRowB = kRowB;
constexpr int kDGroups = kGroups;

struct DSmem {
  // raw latent codes, [tile][row][32 chunks of 16 B]; chunk c of row r sits at slot
  // c ^ swz(r), so the QK reads (16 rows, one chunk pair) and the transpose reads of PV
  // (32 rows, one chunk) hit distinct banks
  uint8_t lat[kDMaxTiles][kDTile * kDRowB];
  float sc[kDMaxTiles][kDGroups][kDTile];  // latent scales [tile][group][row]
  float scr[kDMaxTiles][kDTile];           // rope scales [tile][row]
  union {
    uint16_t q[kDHeads * 576];  // the item's q rows until the QK waves hold them
    struct {
      u32x4 pb[kDGroups][2][64];  // P' per latent group: [group][PV k-step][lane]
      f32x4 tmx[kDHeads];         // tile maxima: [head][QK wave]
      f32x4 lsum[kDHeads];        // row sums: [head][QK wave]
    } x;
  };
  int32_t sl[kDMaxTiles * kDTile];  // slot ids of the chunk (-1: unused)
  int32_t last;                     // this workgroup merges the chunks
};

// Wait until at most 10 k of this wave's LDS-DMA loads are outstanding (k < 5): one tile's
// rows and scales are 10 loads per value wave.
__device__ __forceinline__ void wait_dma_tiles(int k) {
  switch (k) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<10>(); break;
    case 2: wait_vmcnt<20>(); break;
    case 3: wait_vmcnt<30>(); break;
    default: wait_vmcnt<40>(); break;
  }
}

// Pool address of a slot's row (latent codes first) and of its scales, from the 32-bit
// strides (page stride < 2^32, row stride < 2^24, checked by the host); an unused entry
// (s < 0) reads g_zero_row.
__device__ __forceinline__ const uint8_t *row_data(const PoolArgs &pl, int32_t s) {
  const uint32_t ss = s < 0 ? 0u : (uint32_t)s;
  const uint8_t *a =
      pl.data + (uint64_t)(ss >> 6) * pl.page_stride32 + __umul24(ss & 63u, pl.row_stride32);
  return s < 0 ? g_zero_row : a;
}
__device__ __forceinline__ const uint8_t *row_scales(const PoolArgs &pl, int32_t s) {
  const uint32_t ss = s < 0 ? 0u : (uint32_t)s;
  const uint8_t *a = pl.scales + (uint64_t)(ss >> 6) * pl.scale_page_stride32 +
                     __umul24(ss & 63u, pl.scale_row_stride32);
  return s < 0 ? g_zero_row : a;
}

// Stores and loads of the split partials: agent-scope atomic accesses, which gfx950 makes
// coherent across the XCDs (written through to, and read from, the device-coherent level
// past the per-XCD L2s). With the stores acknowledged before a workgroup barrier that
// precedes the count, the chunk that completes the count sees every other chunk's partial;
// agent-scope fences would instead write back or invalidate a whole L2.
__device__ __forceinline__ void st_agent(const void *a, u32x2 v) {
  __hip_atomic_store((uint64_t *)a, __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32x2 ld_agent(const void *a) {
  return __builtin_bit_cast(
      u32x2, __hip_atomic_load((uint64_t *)a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void st_agent16(const void *a, u32x4 v) {
  st_agent(a, u32x2{v[0], v[1]});
  st_agent((const uint8_t *)a + 8, u32x2{v[2], v[3]});
}
__device__ __forceinline__ u32x4 ld_agent16(const void *a) {
  const u32x2 x = ld_agent(a), y = ld_agent((const uint8_t *)a + 8);
  return u32x4{x[0], x[1], y[0], y[1]};
}
__device__ __forceinline__ float ld_agent_f32(const float *a) {
  return __uint_as_float(
      __hip_atomic_load((uint32_t *)a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

struct DItem {
  int t, hg, chunk, head0, tile0, nt;
};

// The two roles run separate code with the same sequence of barriers; the role test is
// uniform, so the compiler's wait counts for one role's loads never land in the other's
// code (the value waves keep several gathers in flight across barriers).

// Logit waves (w < 4): slot ids, rope codes, QK, softmax, P'.
__device__ __forceinline__ void qk_role(const KParams &p, DSmem &sm, const DItem &it, int w,
                                        int lane) {
  const int hl = lane & 15, kq = lane >> 4;
  const int nt = it.nt;
  if (w < nt) {
    const int tile = it.tile0 + w;
    const bool main = tile < p.main_tiles;
    const int base = (main ? tile : tile - p.main_tiles) * kDTile;
    const int width = main ? p.topk : p.topk_extra;
    const int32_t *row =
        main ? p.idx + (int64_t)it.t * p.idx_st : p.eidx + (int64_t)it.t * p.eidx_st;
    const int32_t s32 = *(gi32 *)(row + min(base + lane, width - 1));
    const int32_t *lens = main ? p.len : p.elen;
    const int live = lens ? min(max(*(ci32 *)(lens + it.t), 0), width) : width;
    const int64_t nslots = main ? p.kv.num_slots : p.ex.num_slots;
    const bool ok = base + lane < live && s32 >= 0 && (int64_t)s32 < nslots;
    sm.sl[kDTile * w + lane] = ok ? s32 : -1;
  }
  __syncthreads();  // (1) slot ids

  // rope codes of key 16w + hl of every tile (d 512 + 32 s + 8 kq), and the rope scale of
  // (tile kq, key 16w + hl), which goes to LDS for the lanes that need it
  // (loads are unconditional, absent tiles reading g_zero_row, so that each tile's wait
  // count is fixed and no loaded value is merged with a default before it is used)
  int32_t srow[kDMaxTiles];
#pragma unroll
  for (int j = 0; j < kDMaxTiles; ++j) srow[j] = j < nt ? sm.sl[kDTile * j + 16 * w + hl] : -1;
  const int32_t sown = kq < nt ? sm.sl[kDTile * kq + 16 * w + hl] : -1;
  const float rsc =
      *(gf32 *)(row_scales(it.tile0 + kq < p.main_tiles ? p.kv : p.ex, sown) + 4 * kDGroups);
  u32x2 rope[kDMaxTiles][2];
#pragma unroll
  for (int j = 0; j < kDMaxTiles; ++j) {
    const uint8_t *rd =
        row_data(it.tile0 + j < p.main_tiles ? p.kv : p.ex, srow[j]) + kDRowB + 8 * kq;
    rope[j][0] = *(gu32x2 *)rd;
    rope[j][1] = *(gu32x2 *)(rd + 32);
  }
  __syncthreads();  // (2) q is in LDS
  bf16x8 qop[18];  // q of head hl, d 32 s + 8 kq .. +7
#pragma unroll
  for (int s = 0; s < 18; ++s)
    qop[s] = __builtin_bit_cast(bf16x8, *(lu32x4 *)(sm.q + hl * 576 + 32 * s + 8 * kq));

  float m = neg_inf();  // running max (log2 units) of head hl, the same in every wave
  float l_part = 0.f;   // this lane's share of head hl's row sum
  const int row = 16 * w + hl;
  const int sw = swz(row);
#pragma unroll
  for (int i = 0; i < kDMaxTiles; ++i) {
    if (i >= nt) break;
    __syncthreads();  // (3) tile i has landed; P' of tile i-1 is in LDS
    // the rope scales of tile kq, for the lanes of this wave that read them
    if (i == 0) sm.scr[kq][16 * w + hl] = rsc;
    // S^T for keys 16w + 4kq + r, head hl. The tile's operands are read first (16 latent
    // pieces, the 8 group scales and the rope scales), then each group's two MFMAs go into
    // an accumulator of its own, and S = sum over groups of the keys' group scale times it.
    const uint8_t *lrow = sm.lat[i] + row * kDRowB + 8 * (kq & 1);
    u32x2 araw[2 * kDGroups];
#pragma unroll
    for (int s = 0; s < 2 * kDGroups; ++s)
      araw[s] = *(lu32x2 *)(lrow + 16 * ((2 * s + (kq >> 1)) ^ sw));
    f32x4 scl[kDGroups];
#pragma unroll
    for (int g = 0; g < kDGroups; ++g) scl[g] = *(f32x4 *)&sm.sc[i][g][16 * w + 4 * kq];
    const f32x4 srope = *(f32x4 *)&sm.scr[i][16 * w + 4 * kq];
    f32x4 acc[kDGroups + 1];
#pragma unroll
    for (int g = 0; g <= kDGroups; ++g) {
      acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const u32x2 raw = g < kDGroups ? araw[2 * g + s2] : rope[i][s2];
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(raw), qop[2 * g + s2],
                                                         acc[g], 0, 0, 0);
      }
    }
    f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g <= kDGroups; ++g) {
      const f32x4 sv = g < kDGroups ? scl[g] : srope;
#pragma unroll
      for (int r = 0; r < 4; ++r) S[r] += sv[r] * acc[g][r];
    }
    const int4 sl4 = *(int4 *)&sm.sl[kDTile * i + 16 * w + 4 * kq];
    const int slv[4] = {sl4.x, sl4.y, sl4.z, sl4.w};
    f32x4 z;
    float mx = neg_inf();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[r] = slv[r] >= 0 ? S[r] * p.scale_log2 : neg_inf();
      mx = fmaxf(mx, z[r]);
    }
    mx = pair_max32(pair_max16(mx));
    if (kq == 0) sm.x.tmx[hl][w] = mx;
    __syncthreads();  // (4) tile maxima
    const f32x4 tm4 = sm.x.tmx[hl];
    const float tmax = fmaxf(fmaxf(tm4[0], tm4[1]), fmaxf(tm4[2], tm4[3]));
    const bool need = tmax > m + kRescaleLog2;
    const float mnew = need ? tmax : m;
    if (need) l_part *= fast_exp2(m - mnew);
    m = mnew;
    f32x4 pr;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = z[r] != neg_inf() ? fast_exp2(z[r] - m) : 0.f;
      l_part += pr[r];
    }
    // P' = P times the key's scale of group g, in the PV B-operand layout: PV k-step w/2
    // takes key blocks w & ~1 and w | 1 as the two 8-byte halves of each lane's entry.
#pragma unroll
    for (int g = 0; g < kDGroups; ++g) {
      const u32x2 v = {pack_bf16(pr[0] * scl[g][0], pr[1] * scl[g][1]),
                       pack_bf16(pr[2] * scl[g][2], pr[3] * scl[g][3])};
      *(lu32x2 *)((uint8_t *)&sm.x.pb[g][w >> 1][lane] + 8 * (w & 1)) = v;
    }
  }
  __syncthreads();  // (5) P' of the last tile
  const float lw = pair_sum32(pair_sum16(l_part));
  if (kq == 0) sm.x.lsum[hl][w] = lw;
  __syncthreads();  // (6) row sums
  if (p.n_chunks > 1) __syncthreads();  // (7) partials stored; the logit waves end here
}

// Value waves (w >= 4): q and row gathers into LDS, PV, output or split-K merge.
__device__ __forceinline__ void pv_role(const KParams &p, DSmem &sm, const DItem &it, int w,
                                        int lane) {
  const int hl = lane & 15, kq = lane >> 4;
  const int u = w - 4;
  const int nt = it.nt;
  {
    const uint8_t *qt = reinterpret_cast<const uint8_t *>(p.q + (int64_t)it.t * p.q_st);
    for (int m = u; m < 18; m += 4) {  // 18 KB of q, 1 KB per instruction
      const int o = 1024 * m + 16 * lane;
      const int hd = o / 1152, within = o - hd * 1152;
      const int head = it.head0 + hd < p.h ? it.head0 + hd : 0;  // padded heads: head 0's q
      dma16(qt + (int64_t)head * p.q_sh * 2 + within,
            reinterpret_cast<uint8_t *>(sm.q) + 1024 * m);
    }
  }
  __syncthreads();  // (1) slot ids
  // rows: 8 row pairs and 2 scale groups per tile for this wave (10 loads per tile). Tiles 0
  // and 1 are requested now and tile i + 2 during tile i, so this wave's wait for a tile's
  // rows never waits for more than the next tile's, and a stall on a full memory queue
  // overlaps the logit waves' work instead of holding the first tile back.
  auto issue_tile = [&](int j) __attribute__((always_inline)) {
    const int tile = it.tile0 + j;
    const PoolArgs &pl = tile < p.main_tiles ? p.kv : p.ex;
    int32_t s8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) s8[i] = sm.sl[kDTile * j + 2 * (u + 4 * i) + (lane >> 5)];
    const int32_t ssc = sm.sl[kDTile * j + lane];
    const uint8_t *src[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 2 * (u + 4 * i) + (lane >> 5);
      src[i] = row_data(pl, s8[i]) + 16 * ((lane & 31) ^ swz(r));
    }
    const uint8_t *scs = row_scales(pl, ssc);
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(src[i], sm.lat[j] + 1024 * (u + 4 * i));
#pragma unroll
    for (int i = 0; i < 2; ++i) dma4(scs + 4 * (2 * u + i), &sm.sc[j][2 * u + i][0]);
  };
  issue_tile(0);
  if (nt > 1) issue_tile(1);
  wait_dma_tiles(min(nt, 2));  // q has landed: only the row gathers are outstanding
  __syncthreads();  // (2) q is in LDS

  float m = neg_inf();
  f32x4 oacc[8];  // O^T for d 128u + 16 db + 4 kq + e, head hl
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int lt = lane & 15, ee = lt >> 1;  // the row this lane supplies to a transpose read
  // PV of tile i: 2 k-steps of 32 keys x 8 d blocks
  auto pv_tile = [&](int i) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int key = 32 * ks + (ee < 4 ? 4 * kq + ee : 16 + 4 * kq + ee - 4);
      const uint8_t *vrow = sm.lat[i] + key * kDRowB + 8 * (lt & 1);
      const int sk = swz(key);
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, sm.x.pb[2 * u + g2][ks][lane]);
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4) {
          const int db = 4 * g2 + d4;
          const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (li32x2 *)(vrow + 16 * ((8 * u + db) ^ sk)));
          const bf16x8 a = codes_to_bf16(__builtin_bit_cast(u32x2, raw));
          oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, oacc[db], 0, 0, 0);
        }
      }
    }
  };
#pragma unroll
  for (int i = 0; i < kDMaxTiles; ++i) {
    if (i >= nt) break;
    wait_dma_tiles(i + 1 < nt ? 1 : 0);  // only tile i + 1 may still be in flight
    __syncthreads();  // (3) tile i has landed; P' of tile i-1 is in LDS
    if (i + 2 < nt) issue_tile(i + 2);
    if (i > 0) pv_tile(i - 1);
    __syncthreads();  // (4) tile maxima
    const f32x4 tm4 = sm.x.tmx[hl];
    const float tmax = fmaxf(fmaxf(tm4[0], tm4[1]), fmaxf(tm4[2], tm4[3]));
    const bool need = tmax > m + kRescaleLog2;
    const float mnew = need ? tmax : m;
    if (__any(need)) {
      const float f = need ? fast_exp2(m - mnew) : 1.0f;  // 0 on the first live tile
#pragma unroll
      for (int db = 0; db < 8; ++db) oacc[db] *= f;
    }
    m = mnew;
  }
  __syncthreads();  // (5) P' of the last tile
  pv_tile(nt - 1);
  __syncthreads();  // (6) row sums
  const f32x4 ls4 = sm.x.lsum[hl];
  const float l = (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]);
  const int head = it.head0 + hl;
  const bool head_ok = head < p.h;

  float sig = neg_inf();
  if (p.sink && head_ok) sig = p.sink[head] * kLog2e;
  if (p.n_chunks > 1) {
    // ---- split item. Every chunk stores its partial, acknowledged at the device-coherent
    // level, then counts itself in; the chunk that completes the count merges. It needs no
    // wait: every other chunk's stores were acknowledged before that chunk counted.
    const int64_t grp = (int64_t)it.t * p.n_hg + it.hg;
    uint32_t *arrived = p.arrivals + grp;
    // partial of chunk c: 16 KB of bf16 O / l, [value wave][d-block pair][lane][8]
    auto part = [&](int c) -> uint16_t * {
      return p.ws_o + ((grp * p.n_chunks + c) * 4 + u) * 2048 + 8 * lane;
    };
    auto ml_of = [&](int c) -> float * {
      return p.ws_ml + ((grp * p.n_chunks + c) * kDHeads + hl) * 2;
    };
    {
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      uint16_t *dst = part(it.chunk);
#pragma unroll
      for (int d2 = 0; d2 < 4; ++d2) {
        const f32x4 &a = oacc[2 * d2], &b = oacc[2 * d2 + 1];
        st_agent16(dst + 512 * d2,
                   u32x4{pack_bf16(a[0] * inv, a[1] * inv), pack_bf16(a[2] * inv, a[3] * inv),
                         pack_bf16(b[0] * inv, b[1] * inv), pack_bf16(b[2] * inv, b[3] * inv)});
      }
      if (u == 0 && kq == 0) st_agent(ml_of(it.chunk), u32x2{__float_as_uint(m), __float_as_uint(l)});
      // every store of this workgroup has reached the device-coherent level before the count
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();  // (7) partial stored; the logit waves end here
    if (u == 0 && lane == 0) {
      const uint32_t old = __hip_atomic_fetch_add(arrived, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      sm.last = old + 1 == (uint32_t)p.n_chunks;
      if (sm.last) __hip_atomic_store(arrived, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();  // (8) merger known (value waves only)
    if (!sm.last) return;
    // Merge every chunk in chunk order, each as O / l rounded to bf16 (this chunk's own from
    // registers), so the result does not depend on which chunk arrived last: chunk c weighs
    // l_c 2^(m_c - M).
    const float inv_own = l > 0.f ? 1.0f / l : 0.f;
    float mm = sig;
    for (int c = 0; c < p.n_chunks; ++c)
      mm = fmaxf(mm, c == it.chunk ? m : ld_agent_f32(ml_of(c)));
    f32x4 acc[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float inv = 0.f, lse = neg_inf();
    if (mm != neg_inf()) {
      float den = 0.f;
      for (int c = 0; c < p.n_chunks; ++c) {
        const bool me = c == it.chunk;
        const u32x2 ml = me ? u32x2{__float_as_uint(m), __float_as_uint(l)} : ld_agent(ml_of(c));
        const float mc = __uint_as_float(ml[0]), lc = __uint_as_float(ml[1]);
        const float fc = mc == neg_inf() ? 0.f : lc * fast_exp2(mc - mm);
        den += fc;
        const uint16_t *src = part(c);
#pragma unroll
        for (int d2 = 0; d2 < 4; ++d2) {
          u32x4 v;
          if (me) {
            const f32x4 &a = oacc[2 * d2], &b = oacc[2 * d2 + 1];
            v = u32x4{pack_bf16(a[0] * inv_own, a[1] * inv_own),
                      pack_bf16(a[2] * inv_own, a[3] * inv_own),
                      pack_bf16(b[0] * inv_own, b[1] * inv_own),
                      pack_bf16(b[2] * inv_own, b[3] * inv_own)};
          } else {
            v = ld_agent16(src + 512 * d2);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            f32x4 &dst = acc[2 * d2 + (e >> 1)];
            dst[2 * (e & 1)] += __uint_as_float(v[e] << 16) * fc;
            dst[2 * (e & 1) + 1] += __uint_as_float(v[e] & 0xffff0000u) * fc;
          }
        }
      }
      if (sig != neg_inf()) den += fast_exp2(sig - mm);
      inv = 1.0f / den;
      lse = (mm + __log2f(den)) * kLn2;
    }
    if (head_ok) {
      uint16_t *orow =
          p.out + (int64_t)it.t * p.out_st + (int64_t)head * p.out_sh + 128 * u + 4 * kq;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const u32x2 v = {pack_bf16(acc[db][0] * inv, acc[db][1] * inv),
                         pack_bf16(acc[db][2] * inv, acc[db][3] * inv)};
        *(u32x2 *)(orow + 16 * db) = v;
      }
      if (p.lse && u == 0 && kq == 0) p.lse[(int64_t)it.t * p.lse_st + head] = lse;
    }
    return;
  }

  // ---- whole item: finalize with the sink
  if (!head_ok) return;
  const float mf = fmaxf(m, sig);
  float scale = 0.f, lse = neg_inf();
  if (mf != neg_inf()) {
    const float fo = m == neg_inf() ? 0.f : fast_exp2(m - mf);
    const float fs = sig == neg_inf() ? 0.f : fast_exp2(sig - mf);
    const float den = l * fo + fs;
    scale = fo / den;
    lse = (mf + __log2f(den)) * kLn2;
  }
  uint16_t *orow =
      p.out + (int64_t)it.t * p.out_st + (int64_t)head * p.out_sh + 128 * u + 4 * kq;
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const u32x2 v = {pack_bf16(oacc[db][0] * scale, oacc[db][1] * scale),
                     pack_bf16(oacc[db][2] * scale, oacc[db][3] * scale)};
    *(u32x2 *)(orow + 16 * db) = v;
  }
  if (p.lse && u == 0 && kq == 0) p.lse[(int64_t)it.t * p.lse_st + head] = lse;
}

__global__ __launch_bounds__(kDThreads, 1) void smla_decode16_kernel(const KParams p) {
  __shared__ __attribute__((aligned(16))) DSmem sm;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // Item -> (token, head group, chunk). All items of a token are 8 apart, so they run on
  // one XCD (workgroups are dealt to the 8 XCDs round-robin): the token's head groups share
  // the gathered rows in that XCD's L2, and its chunks meet there.
  DItem it;
  {
    const int u = blockIdx.x, per = p.n_hg * p.n_chunks;
    const int full = (p.T >> 3) * 8 * per;
    int e;
    if (u < full) {
      const int s = u >> 3, grp = s / per;
      e = s - grp * per;
      it.t = 8 * grp + (u & 7);
    } else {
      const int r = u - full, dt = r / per;
      e = r - dt * per;
      it.t = (p.T & ~7) + dt;
    }
    it.hg = e / p.n_chunks;
    it.chunk = e - it.hg * p.n_chunks;
  }
  it.head0 = it.hg * kDHeads;
  it.tile0 = it.chunk * p.tiles_per_chunk;
  it.nt = min(p.tiles_per_chunk, p.n_tiles - it.tile0);
  if (w < 4)
    qk_role(p, sm, it, w, lane);
  else
    pv_role(p, sm, it, w, lane);
}

}  // namespace

hipError_t launch_decode16(const KParams &p, hipStream_t s) {
  hipLaunchKernelGGL(smla_decode16_kernel, dim3((unsigned)p.grid), dim3(kDThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace smla
