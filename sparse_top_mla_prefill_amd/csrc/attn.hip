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
//       . 64-wide index tiles and any head count in [1,128] (section "Runtime
//         envelopes"); its ragged decode widths (a partial last tile) are served by both
//         forms here, and so is a per-row topk_length (sections "swapAB prefill", "Test
//         plan"): entries past a row's width or live count are masked like -1;
//       . sinks and an optional out_lse (section Summary);
//       . the decode form's split-K partials and their merge (section "Runner and CUDA
//         graphs").
//
// Design (gfx950, wave64, one workgroup per CU; LDS holds two tiles of gathered rows).
//   - A workgroup serves one (token, head group, index chunk) and walks the chunk in tiles
//     of gathered rows, double-buffered in LDS as bf16.
//   - Pipeline. The slot ids of tile i+3 are loaded while tile i is computed. The rows of
//     tile i+2 are gathered into registers and written, dequantised, into the idle LDS
//     buffer one iteration later, so a gather has a whole tile of compute to land.
//   - 8 waves, two per SIMD, so one wave's vector and LDS work runs beside the other's
//     MFMAs. d_qk 576: 32 or 64 heads and 64 keys per tile; d_qk 1088: 32 heads and 32
//     keys per tile, with QK split over the two halves of d_qk.
//   - A workgroup walks its work items (token, head group, index chunk) as one stream of
//     tiles, so the gather pipeline runs on from one item into the next.
//   - MFMA with fp32 accumulation. QK: A = 8 latent elements of one gathered row
//     (ds_read_b128), B = q in registers. PV: A = V^T read straight from the row-major tile
//     by ds_read_b64_tr_b16 (LDS transpose read), so no transposed copy is stored.
//   - Online softmax in the log2 domain. The running max is rescaled lazily, only when it
//     grows by more than 2^8; the choice is made per head, so heads stay independent.
//   - fp8 rows are dequantised once per workgroup on the way into LDS: e4m3fn code ->
//     fp32, times the per-64 fp32 scale, rounded to bf16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "smla_internal.h"

namespace smla {

// Split-K partials of the no-allocation decode entry point. A __device__ variable exists
// once on every device the code object is loaded on, and holds its contents until the
// process ends. In host code `scratch` only names the variable: its device address comes
// from hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t scratch_region(void **ptr) {
  static std::mutex mu;
  static void *addr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef __attribute__((address_space(1))) const u32x4 gu32x4;
typedef __attribute__((address_space(1))) const float gf32;
typedef __attribute__((address_space(1))) const int32_t gi32;
// read-only for the whole launch and wave-uniform: fetched by scalar loads
typedef __attribute__((address_space(4))) const int32_t ci32;
typedef __attribute__((address_space(3))) u32x4 lu32x4;
typedef __attribute__((address_space(3))) i16x4 li16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.0f;  // lazy rescale threshold: P <= 2^8

struct RowAddr {
  const uint8_t *data;   // row bytes (slot 0 of the pool for an unused slot)
  const uint8_t *scale;  // fp8 scales of the row
};

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt with vmcnt <= N and no wait on the LDS/scalar or export counters (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};  // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// Two e4m3fn bytes (the low or high 16 bits of w) times an fp32 scale -> two packed bf16.
// The scaled convert instructions of gfx950 apply only the exponent of their scale operand
// (power-of-two block scales), so the codes are converted exactly with scale 1, multiplied
// by the full fp32 scale, and rounded once to bf16.
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, float s, bool hi) {
  const f32x2 f = hi ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true)
                     : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
  return pack_bf16(f[0] * s, f[1] * s);
}


// Tile numbers: the main row's tiles come first, then the extra row's.
template <int TILE>
__device__ __forceinline__ bool tile_is_fp8(const KParams &p, int tile) {
  return tile < p.main_tiles ? p.kv.fp8 != 0 : p.ex.fp8 != 0;
}

// The lane number, recomputed where it is needed rather than kept live across a tile loop
// (where the register allocator would spill it, and the reload would wait for every load).
__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Wave 0: a tile's raw slot ids, lane j loading entry j of the tile. The position is
// clamped into the row, so the load is one unconditional instruction inside the index
// array; entry_live() tells which lanes hold a live entry. Keeping the two apart leaves
// the wait for the load at the point where the ids are used.
template <int TILE>
__device__ __forceinline__ int32_t idx_load(const KParams &p, int t, int tile) {
  const bool main = tile < p.main_tiles;
  const int pos = (main ? tile : tile - p.main_tiles) * TILE + lane_id();
  const int width = main ? p.topk : p.topk_extra;
  const int32_t *row = main ? p.idx + (int64_t)t * p.idx_st : p.eidx + (int64_t)t * p.eidx_st;
  return *(gi32 *)(row + min(pos, width - 1));
}

// Lanes of tile `tile` of token t whose entries take part, as a wave-uniform bit mask: an
// entry lies inside the tile (lane < TILE), before the end of its row (a ragged last tile)
// and before the row's live count when one is given (a count below 0 acts as 0). Scalar
// arithmetic only, so it holds no vector register across the tile loop.
template <int TILE>
__device__ __forceinline__ uint64_t live_mask(const KParams &p, int t, int tile) {
  const bool main = tile < p.main_tiles;
  const int base = (main ? tile : tile - p.main_tiles) * TILE;
  const int width = main ? p.topk : p.topk_extra;
  const int32_t *lens = main ? p.len : p.elen;
  const int live = lens ? min(max(*(ci32 *)(lens + t), 0), width) : width;
  const int k = min(max(live - base, 0), TILE);
  return k >= 64 ? ~0ull : (1ull << k) - 1;
}

// v where lane's bit of the wave-uniform mask m is set, else -1.
__device__ __forceinline__ int32_t keep_lanes(uint64_t m, int32_t v, int lane) {
  return (m >> lane) & 1 ? v : -1;
}

// ---------------------------------------------------------------------------------------
// Wide kernel: d_qk 576, d_v 512, 32 or 64 heads per workgroup, 8 waves (two per SIMD).
//
// A workgroup serves one (token, head group, index chunk) and walks the chunk in 64-key
// tiles, double-buffered in LDS as bf16 rows. Each wave takes two roles per tile:
//   - QK: S^T = K Q^T for 16 heads and a part of the tile's keys on
//     v_mfma_f32_16x16x32_bf16. A = 8 latent elements of one gathered row (ds_read_b128),
//     B = q from registers (18 k-steps of 32). 16 heads per wave keep q (72 registers) and
//     O (64) inside the 256 registers a wave has at two waves per SIMD.
//   - softmax: P = 2^(S - m) in bf16 goes to an LDS exchange buffer, already in the
//     B-operand layout of the PV step; the tile maxima go beside it.
//   - PV: O^T += V^T P^T for 64 of the 512 d_v columns and all heads of the workgroup on
//     v_mfma_f32_32x32x16_bf16; A = V^T by transpose reads of the row-major tile, so each
//     element of V is read from LDS once, B = P^T from the exchange buffer.
// The running max m is kept per head and identically by every wave (each one reads the
// tile maxima of all heads), so the lazy rescale decision is workgroup-uniform.
// Key order inside a 16-key PV step follows the S^T accumulator layout: lane (li, g) of a
// QK wave holds keys 16kb + 4g + e (e < 4) of key block kb; the B-operand lane (j, kg) of
// PV step kb takes keys 16kb + {0..3, 8..11} (kg 0) or 16kb + {4..7, 12..15} (kg 1), so
// each QK lane writes one 8-byte half of one B-operand entry and P needs no shuffle.
// ---------------------------------------------------------------------------------------
// LDS row stride (bf16 elements). A ds_read_b128 is served 32 lanes at a time by 128 banks
// of 4 bytes; the QK operand read of 32 lanes is 16 rows x 2 adjacent 16-byte chunks, which
// hits 32 distinct 16-byte bank groups when the stride is 2 (mod 4) groups of 16 bytes:
// 592 elements = 74 groups (measured 218 B/clk per CU, against 117 at 584).
constexpr int kWRS = 576 + 16;
constexpr int kWRowSlots = kWRS * 2 / 16;  // 16-byte LDS slots per tile row (74)
constexpr int kWPaySlots = 576 * 2 / 16;   // of which bf16 payload (72)
constexpr int kWTileSlots = 64 * kWRowSlots;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((address_space(1))) const u32x2 gu32x2;

__device__ __forceinline__ RowAddr slot_addr(const PoolArgs &pl, int32_t s) {
  const int64_t ss = s < 0 ? 0 : s;  // unused slots read slot 0 (always in bounds)
  const int64_t page = ss >> 6, off = ss & 63;
  RowAddr a;
  a.data = pl.data + page * pl.page_stride + off * pl.row_stride;
  a.scale = pl.scales ? pl.scales + page * pl.scale_page_stride + off * pl.scale_row_stride
                      : pl.data;
  return a;
}

// Wave 0: a tile's checked slot ids (-1 when unused) and their valid mask.
__device__ __forceinline__ void slot_commit(const KParams &p, int tile, int32_t s32,
                                            uint64_t live, int32_t *sl, uint64_t *vmask,
                                            int lane) {
  const PoolArgs &pl = tile < p.main_tiles ? p.kv : p.ex;
  const uint64_t m = __ballot(s32 >= 0 && (int64_t)s32 < pl.num_slots) & live;
  sl[lane] = keep_lanes(m, s32, lane);
  if (lane == 0) *vmask = m;
}

// 8 e4m3fn codes times their group scale -> 8 bf16 (one 16-byte LDS chunk).
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(const u32x2 v, float s) {
  return u32x4{fp8x2_to_bf16x2(v[0], s, false), fp8x2_to_bf16x2(v[0], s, true),
               fp8x2_to_bf16x2(v[1], s, false), fp8x2_to_bf16x2(v[1], s, true)};
}

// Calls f(std::integral_constant<int, k>) for k = B .. E-1 (compile-time loop).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Index of the gather piece placed after step s of a loop of STEPS steps that carries N
// pieces spread evenly (the last one after the last step), or -1.
template <int N, int STEPS>
constexpr int piece_at(int s) {
  for (int p = 0; p < N; ++p)
    if ((p + 1) * STEPS / N - 1 == s) return p;
  return -1;
}

// 8-wave layout of the wide kernel: two waves per SIMD, so that one wave's vector and LDS
// work runs beside the other's MFMAs.
constexpr int kEThreads = 512;
constexpr int kEPieces = 576 / 8 / 8;  // 8-byte fp8 pieces per staging thread: 9

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane
// (global_load_lds_dwordx4; the LDS base goes in M0). Issued as inline assembly so that
// the compiler's wait-count bookkeeping does not see these loads: their number varies
// from tile to tile, and counted they would make every wait in the tile loop a full
// drain. Extra loads it does not know of only make the compiler's waits for its own
// loads wait longer, never shorter; the caller waits for these with an explicit
// s_waitcnt vmcnt(0) before the tile is read.
// M0 is a reserved register, so clang warns that its clobber may not be honoured; no
// compiled code of this file uses M0 (the only writers are these statements), which the
// CPU test test_m0_guard checks on the generated assembly, so the clobber list is
// documentation here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void *g, const void *lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// bf16 tile straight from global memory into LDS, 8 waves: wave w fills 16-byte slots
// 64*(w + 8j) + lane of the tile; unused rows get zeros, pad slots are skipped.
__device__ __forceinline__ void wide_dma16_8(const PoolArgs &pl, const int32_t *sl, uint64_t vm,
                                             uint16_t *tile, int w, int lane) {
#pragma unroll 1
  for (int j = 0; j < (kWTileSlots + 511) / 512; ++j) {
    const int m = w + 8 * j;
    if (64 * m < kWTileSlots) {
      const int slot = 64 * m + lane;
      const int r = min(slot / kWRowSlots, 63), c = slot - r * kWRowSlots;
      if (slot < kWTileSlots && c < kWPaySlots) {
        if ((vm >> r) & 1)
          lds_dma16(slot_addr(pl, sl[r]).data + 16 * c, tile + 512 * m);
        else
          *(lu32x4 *)(tile + 8 * slot) = u32x4{0, 0, 0, 0};
      }
    }
  }
}

// NHB head blocks of 32 per workgroup (2: 64 heads, 1: 32 heads). QK: 2*NHB sets of 16
// heads times 4/NHB key parts of 16*NHB keys; PV: 64 d and all 32*NHB heads per wave.
template <bool F8ONLY, int NHB, bool S64>
__global__ __launch_bounds__(kEThreads, 1) void smla_wide_kernel(const KParams p) {
  constexpr int TILE = 64, RS = kWRS, D_V = 512, QS = 576 / 32;
  constexpr int HG = 32 * NHB;        // heads per workgroup
  // 32 heads: QK on waves 0..3 only (one per SIMD, 32 keys each), so each q row is loaded by
  // two waves, not four, and waves 4..7 convert their gather pieces beside those MFMAs
  // (prefill at 32 heads, 4 tiles per token: 0.262 -> 0.248 ms). At 64 heads the same split
  // (S64: a QK wave covers its 64 keys in two passes of 32) is taken for split-K decode
  // only: it spills 12 bytes and was slower on long prefill items (6.35 vs 5.99 ms on the
  // large prefill) but faster on decode's one-tile items (21.4 vs 23.0 us per step), where
  // halving the q loads matters most.
  constexpr bool SPLIT = NHB == 1 || S64;
  constexpr int NQW = SPLIT ? 4 : 8;  // waves that compute QK
  constexpr int NHS = 2 * NHB;        // QK head sets of 16
  constexpr int NX = NQW / NHS;       // QK key parts
  constexpr int KPW = TILE / NX;      // keys per QK wave
  constexpr int KBW = KPW / 16;       // key blocks per QK wave (= NHB)
  // gather pieces converted between the QK MFMAs (the rest between the PV MFMAs)
  constexpr int kQkPieces = NHB == 2 ? 2 : 6;  // (measured best of 2..6; 6 and 9 at 32 heads)
  __shared__ __attribute__((aligned(16))) uint16_t tiles[2][TILE * RS];
  __shared__ __attribute__((aligned(16))) u32x4 pbuf[NHB][4][64];  // [head block][PV step][lane]
  __shared__ int32_t slots[4][TILE];
  __shared__ uint64_t vmask[4];
  __shared__ float tmx[NX][HG];   // tile maxima (log2 units), per key part
  constexpr int KBH = KBW > 2 ? 2 : KBW;  // key blocks per QK pass
  constexpr int NP = KBW / KBH;           // QK passes over the tile
  using VmT = std::conditional_t<(KPW > 32), uint64_t, uint32_t>;
  __shared__ float lsum[NX][HG];  // row sums at the end, per key part

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;  // QK role: head 16hq + li, key group g
  // (x is taken modulo NX: the waves past NQW compute no QK, and their key offsets stay
  // inside the tile)
  const int hq = w % NHS, x = (w / NHS) % NX;  // QK role: heads 16hq.., keys KPW*x..
  const bool qkw = !SPLIT || w < NQW;          // this wave computes QK
  const int j = lane & 31, q = lane >> 5;   // PV role: heads 32hb + j, key half q

  // Work items are (token, head group, chunk); block b takes items b, b + gridDim.x, ...
  // and walks their tiles as one stream, so the gather pipeline runs on across items.
  // Item -> (token, head group, chunk): all items of one token are items 8 apart, which
  // run on blocks of the same XCD (blocks are dealt to the 8 XCDs round-robin, and the
  // grid is a multiple of 8 or covers all items), so the token's q, slot ids and rows come
  // into that XCD's L2 once and its other head groups and chunks find them there.
  const int total = p.T * p.n_hg * p.n_chunks;
  const int tpc = p.tiles_per_chunk;  // tiles per item; past n_tiles a tile is empty
  const int n_tiles = p.n_tiles;
  const int n_items = (total - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int G_all = n_items * tpc;  // tiles of this block
  struct Item {
    int t, hg, chunk;
  };
  auto item_of = [&](int k) -> Item {
    const int u = (int)blockIdx.x + k * (int)gridDim.x;
    const int per = p.n_hg * p.n_chunks;  // items per token
    const int full = (p.T >> 3) * 8 * per;  // items of whole groups of 8 tokens
    int t, e;
    if (u < full) {
      const int s = u >> 3, grp = s / per;
      e = s - grp * per;
      t = 8 * grp + (u & 7);
    } else {
      const int r = u - full, dt = r / per;
      e = r - dt * per;
      t = (p.T & ~7) + dt;
    }
    return Item{t, e / p.n_chunks, e % p.n_chunks};
  };
  Item it = item_of(0);
  // Tile cursor: token t3 and tile number a3 (within the token's index list) of stream tile
  // min(i+3, n-1), in item k3, whose tiles end at e3; a1, a2: tile numbers of stream tiles
  // min(i+1, n-1) and min(i+2, n-1). Advanced one tile per iteration, so an item's
  // divisions are done once.
  int k3 = 0, t3 = it.t, a3 = it.chunk * tpc, e3 = a3 + tpc;
  auto step3 = [&]() __attribute__((always_inline)) {
    if (++a3 == e3) {
      ++k3;
      const Item c = item_of(k3);
      t3 = c.t;
      a3 = c.chunk * tpc;
      e3 = a3 + tpc;
    }
  };
  // Staging: thread (srow, sq) moves bf16 chunks 8m + sq (m < 9, scale group m) of row
  // srow, each from 8 fp8 bytes. The 16 lanes that the LDS serves together write 128
  // contiguous bytes of two rows 8 apart, which fall in distinct banks.
  const int srow = w + 8 * (lane >> 3), sq = lane & 7;

  // q (B operand of QK, 16x16x32): head head0 + 16hq + li, elements 32s + 8g .. +7. Heads
  // past h compute with the q of head 0: every head's column of S, P and O is independent
  // of the others, and their outputs are never stored.
  bf16x8 qop[QS];
  float snx[NHB];  // raw sink values of the current item's PV heads (see load_sink)
  auto load_q_from = [&](const uint16_t *qrow, int step) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < QS; ++s)
      qop[s] = __builtin_bit_cast(bf16x8, *(gu32x4 *)(qrow + (int64_t)step * s));
  };
  auto q_row = [&](const Item &itm) __attribute__((always_inline)) -> const uint16_t * {
    const int head = itm.hg * HG + 16 * hq + li;
    return p.q + (int64_t)itm.t * p.q_st + (int64_t)(head < p.h ? head : 0) * p.q_sh + 8 * g;
  };
  // sink logits of an item's PV heads j, 32 + j, loaded during its last tile so that their
  // latency is hidden (always a load: a valid dummy address when there is no sink)
  auto load_sink = [&](const Item &itm) __attribute__((always_inline)) {
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const int hd = min(itm.hg * HG + 32 * hb + j, p.h - 1);
      snx[hb] = *(gf32 *)(p.sink ? p.sink + hd : (const float *)p.q);
    }
  };
  f32x16 oacc[2][NHB];  // [d block][head block]
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][hb][r] = 0.f;
  // Running max (log2 units), the same for a head in every wave and lane that holds it:
  // m0, m1 for the PV heads j, 32 + j (m1 unused at NHB 1); mq for the QK head 16hq + li.
  float m0 = neg_inf(), m1 = neg_inf(), mq = neg_inf();
  float l_part = 0.f;  // QK role: head 16hq + li, this lane's keys

  // rolling gather registers: piece m of this thread's row and its group scale
  u32x2 cv[kEPieces];
  float cs[kEPieces];
  auto issue_piece = [&](int m, const RowAddr &a) __attribute__((always_inline)) {
    cv[m] = *(gu32x2 *)(a.data + 8 * (8 * m + sq));
    cs[m] = *(gf32 *)(a.scale + 4 * m);
  };
  auto commit_piece = [&](int m, uint16_t *row) __attribute__((always_inline)) {
    *(lu32x4 *)(row + 8 * (8 * m + sq)) = fp8x8_to_bf16x8(cv[m], cs[m]);
  };
  auto zero_row = [&](uint16_t *row) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < kEPieces; ++m) *(lu32x4 *)(row + 8 * (8 * m + sq)) = u32x4{0, 0, 0, 0};
  };
  // pool, fp8-ness, slot ids of tile g of the stream (an empty tile past n_tiles has no
  // valid slot and reads nothing)
  // pool, fp8-ness, indices and slot ids of tile number ab (an empty tile past n_tiles has
  // no valid slot and reads nothing)
  auto pool_of = [&](int ab) -> const PoolArgs & {
    return ab < p.main_tiles || ab >= n_tiles ? p.kv : p.ex;
  };
  auto fp8_at = [&](int ab) { return ab < n_tiles && tile_is_fp8<TILE>(p, ab); };
  // always one load (of the last real tile for an empty one), so the loads in flight stay
  // countable; the ids are masked when committed (slots_at runs with the t3 of the load)
  auto idx_at = [&](int t, int ab) -> int32_t {
    return idx_load<TILE>(p, t, min(ab, n_tiles - 1));
  };
  auto slots_at = [&](int gg, int ab, int32_t s32) __attribute__((always_inline)) {
    const int tl = min(ab, n_tiles - 1);
    const uint64_t live = ab < n_tiles ? live_mask<TILE>(p, t3, tl) : 0;
    slot_commit(p, tl, s32, live, slots[gg & 3], &vmask[gg & 3], lane);
  };

  // prologue: slots of tiles 0..2; tile 0 into buffer 0; tile 1 in flight
  const int n = G_all;
  auto prologue_tile = [&](int i) __attribute__((always_inline)) {
    const int ab = a3;
    if (w == 0 && i < n) slots_at(i, ab, idx_at(t3, ab));
    if (i + 1 < n) step3();
    return ab;
  };
  const int a0 = prologue_tile(0);
  int a1 = prologue_tile(1);
  int a2 = prologue_tile(2);
  __syncthreads();
  // The rows of tile 0 go out before q, so the first tile waits for one round trip after
  // the slot ids rather than for q as well.
  if (n > 0 && (F8ONLY || fp8_at(a0))) {
    const RowAddr a = slot_addr(pool_of(a0), slots[0][srow]);
    const bool ok = (vmask[0] >> srow) & 1;
#pragma unroll
    for (int m = 0; m < kEPieces; ++m) issue_piece(m, a);
    load_q_from(qkw ? q_row(it) : p.q, qkw ? 32 : 0);
#pragma unroll
    for (int m = 0; m < kEPieces; ++m) commit_piece(m, tiles[0] + srow * RS);
    if (!ok) zero_row(tiles[0] + srow * RS);
  } else {
    if (n > 0) wide_dma16_8(pool_of(a0), slots[0], vmask[0], tiles[0], w, lane);
    load_q_from(qkw ? q_row(it) : p.q, qkw ? 32 : 0);
  }
  // q has landed before the loop on every path, so no wait in the loop is for q
  __builtin_amdgcn_s_waitcnt(0);
  if (F8ONLY ? n > 0 : (n > 1 && fp8_at(a1))) {
    const int s1 = min(1, n - 1);
    const RowAddr a = slot_addr(pool_of(a1), slots[s1][srow]);
#pragma unroll
    for (int m = 0; m < kEPieces; ++m) issue_piece(m, a);
  }
  __syncthreads();

  int32_t idx3 = -1;
  f32x4 sacc[KBW];    // S^T of key blocks KBW*x + k2 (keys 16(KBW*x+k2) + 4g + e, head li)
  float psum = 0.f;   // this tile's row sum for head 16hq + li, this lane's keys
  float tpart = neg_inf();
  bool any_need = false;
  float tm0 = neg_inf(), tm1 = neg_inf();
  // Rolling-gather state of one iteration, shared by its QK half (pieces 0..5) and its PV
  // half (pieces 6..8).
  bool g_c8 = false, g_i8 = false, g_fix = false;
  RowAddr g_ai = {nullptr, nullptr};
  uint16_t *g_crow = nullptr;
  auto gather_step = [&](int m) __attribute__((always_inline)) {
    if (g_c8) commit_piece(m, g_crow);
    if (g_i8) issue_piece(m, g_ai);
  };

  // Softmax of key block KBW*x + k2 of tile i relative to reference mq: mask, tile max, P
  // (bf16) into the exchange buffer. The B-operand lane (j, kg) of PV step kb takes keys
  // 16kb + {0..3, 8..11} (kg 0) or 16kb + {4..7, 12..15} (kg 1), so this lane's 4 keys
  // 16kb + 4g + e are half g/2 of entry kg = g%2.
  VmT vm_half = ~VmT(0);
  auto softmax_block = [&](int k2, bool rewrite) __attribute__((always_inline)) {
    const float mu = mq == neg_inf() ? 0.0f : mq;
    const VmT vsh = vm_half >> (4 * g);  // bit 16*k2 + e: key 16(KBW*x+k2) + 4g + e
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float xv = sacc[k2][e];
      if (vm_half != ~VmT(0)) xv = ((uint32_t)(vsh >> (16 * k2 + e)) & 1u) ? xv : neg_inf();
      if (!rewrite) tpart = fmaxf(tpart, xv);
      pr[e] = fast_exp2(fmaf(xv, p.scale_log2, -mu));
      psum += pr[e];
    }
    const u32x2 v = {pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3])};
    typedef __attribute__((address_space(3))) u32x2 lu32x2;
    typedef __attribute__((address_space(3))) char lchar;
    *(lu32x2 *)((lchar *)&pbuf[hq >> 1][KBW * x + k2][(g & 1) * 32 + 16 * (hq & 1) + li] + 8 * (g >> 1)) = v;
  };

  // Front of tile i: DMA of a bf16 tile i+1; QK of this wave's keys with gather pieces
  // 0..5 between the MFMAs; softmax; barrier; rescale check.
  Item nxt = it;  // item whose q the last tile of the current item loads
  bool more = true;  // the current item is not this workgroup's last
  auto front = [&](int i, auto lastq) __attribute__((always_inline)) {
    const int cur = i & 1;
    // fp8-only workloads issue the same loads every iteration (tail tiles re-read the last
    // tile), so the compiler can count the loads in flight exactly and wait only for the
    // piece being converted. The commits stay conditional: the last tile needs none.
    const bool c8 = i + 1 < n && (F8ONLY || fp8_at(a1));
    // fp8 pieces of tile i+2 are loaded whatever its kind (a bf16 tile's row is read but
    // never committed), so the loads in flight stay countable
    const bool i8 = true;
    if (!F8ONLY && i + 1 < n && !c8)
      wide_dma16_8(pool_of(a1), slots[(i + 1) & 3], vmask[(i + 1) & 3], tiles[cur ^ 1], w, lane);
    idx3 = idx_at(t3, a3);
    const int s1 = min(i + 1, n - 1);
    const int s2 = min(i + 2, n - 1);
    const uint64_t vm1 = vmask[s1 & 3];
    g_c8 = c8;
    g_i8 = i8;
    g_fix = c8 && !((vm1 >> srow) & 1);
    g_ai = slot_addr(pool_of(a2), slots[s2 & 3][srow]);
    g_crow = tiles[cur ^ 1] + srow * RS;
    if constexpr (KPW > 32) {
      const uint64_t v = vmask[i & 3];
      // (readfirstlane returns a signed int: each half is widened as unsigned)
      vm_half = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
                (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    } else {
      vm_half = __builtin_amdgcn_readfirstlane((uint32_t)(vmask[i & 3] >> (KPW * x)));
      if constexpr (KPW < 32) vm_half |= 0xffffffffu << KPW;  // bits past this wave's keys
    }
    psum = 0.f;
    tpart = neg_inf();

    const uint16_t *kr = tiles[cur] + (KPW * x + li) * RS + 8 * g;  // this wave's key blocks
    constexpr int LA = 2;  // k-steps of A operands read ahead
    constexpr int NR = LA + 1;
    if (qkw) {
      static_for<0, NP>([&](auto pc) __attribute__((always_inline)) {
        constexpr int ph = decltype(pc)::value;
        const uint16_t *kp = kr + 16 * KBH * ph * RS;
        bf16x8 abuf[NR][KBH];
#pragma unroll
        for (int s = 0; s < LA; ++s)
#pragma unroll
          for (int k2 = 0; k2 < KBH; ++k2)
            abuf[s][k2] = *reinterpret_cast<const bf16x8 *>(kp + 16 * k2 * RS + 32 * s);
        static_for<0, QS>([&](auto sc) __attribute__((always_inline)) {
          constexpr int s = decltype(sc)::value;
          constexpr int st = ph * QS + s;
          if constexpr (s + LA < QS) {
#pragma unroll
            for (int k2 = 0; k2 < KBH; ++k2)
              abuf[(s + LA) % NR][k2] =
                  *reinterpret_cast<const bf16x8 *>(kp + 16 * k2 * RS + 32 * (s + LA));
          }
#pragma unroll
          for (int k2 = 0; k2 < KBH; ++k2) {
            if constexpr (s == 0)
              sacc[KBH * ph + k2] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(abuf[0][k2], qop[0], f32x4{}, 0, 0, 0);
            else
              sacc[KBH * ph + k2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  abuf[s % NR][k2], qop[s], sacc[KBH * ph + k2], 0, 0, 0);
          }
          if constexpr (piece_at<kQkPieces, NP * QS>(st) >= 0)
            gather_step(piece_at<kQkPieces, NP * QS>(st));
          __builtin_amdgcn_sched_barrier(0);
        });
      });
    } else {
      // the same gather steps at the same points of the instruction stream, so the loads
      // in flight are counted alike in both roles
      static_for<0, NP * QS>([&](auto sc) __attribute__((always_inline)) {
        constexpr int st = decltype(sc)::value;
        if constexpr (piece_at<kQkPieces, NP * QS>(st) >= 0)
          gather_step(piece_at<kQkPieces, NP * QS>(st));
      });
    }
    // last tile of an item: q of the next item goes out now that this one's is consumed
    // (after the last item the loads still go out, so the loads in flight stay countable,
    // but all of them read the same 16 bytes: one line instead of 147 KB per CU, whose
    // redundant fetch holds the waves for about 3 us)
    if constexpr (decltype(lastq)::value) {
      load_q_from(more && qkw ? q_row(nxt) : p.q, more && qkw ? 32 : 0);
      load_sink(it);
    }
    if (qkw) {
#pragma unroll
      for (int k2 = 0; k2 < KBW; ++k2) softmax_block(k2, false);
      float tmax = fmaxf(tpart, __shfl_xor(tpart, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * p.scale_log2;
      if (g == 0) tmx[x][16 * hq + li] = tmax;
    }
    __syncthreads();
    // every wave checks all heads, so the decision is the same in all of them
    tm0 = tmx[0][j];
#pragma unroll
    for (int xx = 1; xx < NX; ++xx) tm0 = fmaxf(tm0, tmx[xx][j]);
    bool need = tm0 > m0 + kRescaleLog2;
    if constexpr (NHB == 2) {
      tm1 = tmx[0][32 + j];
#pragma unroll
      for (int xx = 1; xx < NX; ++xx) tm1 = fmaxf(tm1, tmx[xx][32 + j]);
      need = need || tm1 > m1 + kRescaleLog2;
    }
    any_need = __any(need);
  };

  // Back of tile i: O^T += V^T P^T for this wave's 64 d and all 64 heads, with gather
  // pieces 6..8 between the MFMAs; slots of tile i+3; end of tile.
  auto back = [&](int i) __attribute__((always_inline)) {
    const int cur = i & 1;
    l_part += psum;
    const int G = lane >> 4, lt = lane & 15;
    // lane (G, lt): key row 4q + lt/4 (+16ks, +8 for the second read), elements
    // 4*(lt%4).. of the 16-wide d block 16*(G%2) of d block db of this wave's 64 d
    const uint16_t *vbase =
        tiles[cur] + (4 * q + (lt >> 2)) * RS + 64 * w + 16 * (G & 1) + 4 * (lt & 3);
    auto load_v = [&](int db, int ks) __attribute__((always_inline)) -> bf16x8 {
      const uint16_t *src = vbase + 16 * ks * RS + 32 * db;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4 *)(src));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4 *)(src + 8 * RS));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      const u32x4 a4 = {l2[0], l2[1], h2[0], h2[1]};
      return __builtin_bit_cast(bf16x8, a4);
    };
    constexpr int LV = 2;  // V^T operands read ahead
    constexpr int NV = LV + 1;
    bf16x8 vb[NV];
    bf16x8 pb[NHB];
#pragma unroll
    for (int k = 0; k < LV; ++k) vb[k] = load_v(k & 1, k >> 1);
    static_for<0, 8>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value, ks = k >> 1, db = k & 1;
      if constexpr (db == 0) {
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) pb[hb] = __builtin_bit_cast(bf16x8, pbuf[hb][ks][lane]);
      }
      if constexpr (k + LV < 8) vb[(k + LV) % NV] = load_v((k + LV) & 1, (k + LV) >> 1);
      const bf16x8 a = vb[k % NV];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
        oacc[db][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[hb], oacc[db][hb], 0, 0, 0);
      if constexpr (piece_at<kEPieces - kQkPieces, 8>(k) >= 0)
        gather_step(kQkPieces + piece_at<kEPieces - kQkPieces, 8>(k));
      __builtin_amdgcn_sched_barrier(0);
    });
    // rows of tile i+1 whose slots are unused: zeros over the converted bytes
    if (g_fix) zero_row(g_crow);
    if (w == 0 && i + 3 < n) slots_at(i + 3, a3, idx3);
    if (!F8ONLY && i + 1 < n && !fp8_at(a1)) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    a1 = a2;
    a2 = a3;
    if (i + 4 < n) step3();
  };

  // Rare: some head's max grew by more than 2^8 (always on the first tile of an item with a
  // valid key). Move the reference, rescale O and l, and redo this wave's P.
  auto rescale = [&]() __attribute__((always_inline)) {
    const bool n0 = tm0 > m0 + kRescaleLog2, n1 = NHB == 2 && tm1 > m1 + kRescaleLog2;
    const float nm0 = n0 ? tm0 : m0, nm1 = n1 ? tm1 : m1;
    const float f0 = n0 ? fast_exp2(m0 - nm0) : 1.0f, f1 = n1 ? fast_exp2(m1 - nm1) : 1.0f;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      oacc[db][0] *= f0;
      if constexpr (NHB == 2) oacc[db][1] *= f1;
    }
    m0 = nm0;
    m1 = nm1;
    if (qkw) {
      float tq = tmx[0][16 * hq + li];
#pragma unroll
      for (int xx = 1; xx < NX; ++xx) tq = fmaxf(tq, tmx[xx][16 * hq + li]);
      if (tq > mq + kRescaleLog2) {
        l_part *= fast_exp2(mq - tq);
        mq = tq;
      }
      psum = 0.f;
#pragma unroll
      for (int k2 = 0; k2 < KBW; ++k2) softmax_block(k2, true);
    }
    __syncthreads();
  };

  int i = 0;  // tile of the stream
  for (int k = 0; k < n_items; ++k) {
    const int ilast = i + tpc - 1;
    more = k + 1 < n_items;
    nxt = more ? item_of(k + 1) : it;
    while (i < ilast) {
      for (; i < ilast; ++i) {
        front(i, std::false_type{});
        if (any_need) break;
        back(i);
      }
      if (i >= ilast) break;
      rescale();
      back(i);
      ++i;
    }
    front(i, std::true_type{});
    if (any_need) rescale();
    back(i);
    ++i;
    // Item done: row sums of the QK heads, then of the PV heads.
    const Item done = it;
    it = nxt;
    {
      float lw = l_part + __shfl_xor(l_part, 16);
      lw += __shfl_xor(lw, 32);
      // (the address is derived from a fresh copy of tid, so it is not kept live through the
      // item)
      int t2 = tid;
      asm volatile("" : "+v"(t2));
      const int w2 = t2 >> 6, l2 = t2 & 63;
      if ((l2 >> 4) == 0 && w2 < NQW) lsum[w2 / NHS][16 * (w2 % NHS) + (l2 & 15)] = lw;
    }
    __syncthreads();
    // q and the sinks land here: only the fp8 pieces issued after them in the last tile's
    // PV half (two loads each) stay in flight for the next item's tiles
    wait_vmcnt<2 * (kEPieces - kQkPieces)>();
    float l0 = 0.f, l1 = 0.f;
#pragma unroll
    for (int xx = 0; xx < NX; ++xx) {
      l0 += lsum[xx][j];
      if constexpr (NHB == 2) l1 += lsum[xx][32 + j];
    }

    // Outputs. Each wave stages its bf16 rows (all heads x its 64 columns) in the tile buffer
    // just consumed, then stores 16 contiguous bytes per lane, 8 lanes per 128-byte row
    // segment (the accumulator layout would scatter 8-byte pieces over 32 rows per store).
    // Staging rows are 72 elements apart, so the 32 heads of one write hit distinct banks.
    constexpr int SR = 72;
    // (staging addresses come from a fresh copy of tid, so no lane offset is kept live
    // through the tile loop)
    int ts = tid;
    asm volatile("" : "+v"(ts));
    const int js = ts & 31, qs = (ts >> 5) & 1;
    uint16_t *stg = tiles[(i - 1) & 1] + (ts >> 6) * (HG * SR);
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const int head = done.hg * HG + 32 * hb + j;
      const float m = hb ? m1 : m0, l = hb ? l1 : l0;
      float scale;
      if (p.n_chunks > 1) {
        // split-K partial: O / l in bf16, running max (log2 units), sum
        scale = l > 0.f ? 1.0f / l : 0.f;
        if (head < p.h && w == 0 && q == 0) {
          const int64_t row = ((int64_t)done.t * p.n_chunks + done.chunk) * p.h + head;
          p.ws_ml[row * 2 + 0] = m;
          p.ws_ml[row * 2 + 1] = l;
        }
      } else {
        const float sig = p.sink ? snx[hb] * kLog2e : neg_inf();
        const float mf = fmaxf(m, sig);
        float lse = neg_inf();
        scale = 0.f;
        if (mf != neg_inf()) {
          const float fo = m == neg_inf() ? 0.f : fast_exp2(m - mf);
          const float fs = sig == neg_inf() ? 0.f : fast_exp2(sig - mf);
          const float den = l * fo + fs;
          scale = fo / den;
          lse = (mf + __log2f(den)) * kLn2;
        }
        if (p.lse && head < p.h && w == 0 && q == 0) p.lse[(int64_t)done.t * p.lse_st + head] = lse;
      }
      typedef __attribute__((address_space(3))) u32x2 lu32x2;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const u32x2 pk = {pack_bf16(oacc[db][hb][4 * b] * scale, oacc[db][hb][4 * b + 1] * scale),
                            pack_bf16(oacc[db][hb][4 * b + 2] * scale, oacc[db][hb][4 * b + 3] * scale)};
          *(lu32x2 *)(stg + (32 * hb + js) * SR + 32 * db + 8 * b + 4 * qs) = pk;
        }
    }
    {
      const int c = ts & 7;  // 8-column chunk of this wave's 64
#pragma unroll
      for (int r = 0; r < HG / 8; ++r) {
        const int hl = 8 * r + ((ts >> 3) & 7);
        const int head = done.hg * HG + hl;
        const u32x4 v = *(lu32x4 *)(stg + hl * SR + 8 * c);
        if (head < p.h) {
          uint16_t *dst =
              p.n_chunks > 1
                  ? p.ws_o + (((int64_t)done.t * p.n_chunks + done.chunk) * p.h + head) * D_V
                  : p.out + (int64_t)done.t * p.out_st + (int64_t)head * p.out_sh;
          *reinterpret_cast<u32x4 *>(dst + 64 * w + 8 * c) = v;
        }
      }
    }
    // the staging area is the buffer the next item's first commits write
    __syncthreads();

    // next item: fresh state (the lsum and tile-max arrays are rewritten before reuse)
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][hb][r] = 0.f;
    m0 = m1 = mq = neg_inf();
    l_part = 0.f;
  }
}

// ---------------------------------------------------------------------------------------
// Wide kernel for d_qk 1088, d_v 1024: 32 heads per workgroup, 32-key tiles, 8 waves (two
// per SIMD), the same tile walk, rolling gather and lazy softmax as the 576 kernel.
//
// q of 16 heads over all 1088 elements would take 136 registers, so QK is cut three ways:
// wave (hq, kb, dh) computes the partial S^T of heads 16hq.., keys 16kb.. over the d half
// 544dh.. (17 k-steps of v_mfma_f32_16x16x32_bf16; q in 68 registers). The two d halves
// are summed through LDS (one 16x16 block per wave), so both partners hold the full S of
// their block; the dh 0 partner writes P and the tile maxima. PV: wave w accumulates O^T
// for d 128w..128w+127 and all 32 heads on v_mfma_f32_32x32x16_bf16 (64 registers).
// Gather: thread (row tid/16, s = tid%16) moves the 8-byte fp8 pieces 16m + s (m < 9; the
// last only for s < 8) of one row per tile; bf16 tiles go global -> LDS directly.
// ---------------------------------------------------------------------------------------
constexpr int kXRS = 1088 + 16;               // LDS row stride: 138 = 2 (mod 4) 16-byte groups
constexpr int kXRowSlots = kXRS * 2 / 16;     // 16-byte LDS slots per row (138)
constexpr int kXPaySlots = 1088 * 2 / 16;     // of which bf16 payload (136)
constexpr int kXTileSlots = 32 * kXRowSlots;
constexpr int kXPieces = 9;

// bf16 tile straight from global memory into LDS, 8 waves (see wide_dma16_8).
__device__ __forceinline__ void x_dma16(const PoolArgs &pl, const int32_t *sl, uint64_t vm,
                                        uint16_t *tile, int w, int lane) {
#pragma unroll 1
  for (int j = 0; j < (kXTileSlots + 511) / 512; ++j) {
    const int m = w + 8 * j;
    if (64 * m < kXTileSlots) {
      const int slot = 64 * m + lane;
      const int r = min(slot / kXRowSlots, 31), c = slot - r * kXRowSlots;
      if (slot < kXTileSlots && c < kXPaySlots) {
        if ((vm >> r) & 1)
          lds_dma16(slot_addr(pl, sl[r]).data + 16 * c, tile + 512 * m);
        else
          *(lu32x4 *)(tile + 8 * slot) = u32x4{0, 0, 0, 0};
      }
    }
  }
}

template <bool F8ONLY>
__global__ __launch_bounds__(kEThreads, 1) void smla_wide1088_kernel(const KParams p) {
  constexpr int TILE = 32, RS = kXRS, D_V = 1024, QS = 17, HG = 32;
  __shared__ __attribute__((aligned(16))) uint16_t tiles[2][TILE * RS];
  __shared__ __attribute__((aligned(16))) u32x4 pbuf[2][64];   // [PV step][lane]
  __shared__ __attribute__((aligned(16))) f32x4 exch[8][64];   // partial S^T per wave
  __shared__ int32_t slots[4][64];
  __shared__ uint64_t vmask[4];
  __shared__ float tmx[2][HG];   // tile maxima (log2 units), per key block
  __shared__ float lsum[2][HG];  // row sums at the end, per key block

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;                 // QK role: head 16hq + li, keys 4g..
  const int hq = w & 1, kb = (w >> 1) & 1, dh = w >> 2;    // QK role: head set, key block, d half
  const int j = lane & 31, q = lane >> 5;                  // PV role: head j, key half q

  // Work items and their mapping to blocks: as in the 576 kernel.
  const int total = p.T * p.n_hg * p.n_chunks;
  const int tpc = p.tiles_per_chunk;
  const int n_tiles = p.n_tiles;
  const int n_items = (total - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int G_all = n_items * tpc;
  struct Item {
    int t, hg, chunk;
  };
  auto item_of = [&](int k) -> Item {
    const int u = (int)blockIdx.x + k * (int)gridDim.x;
    const int per = p.n_hg * p.n_chunks;
    const int full = (p.T >> 3) * 8 * per;
    int t, e;
    if (u < full) {
      const int s = u >> 3, grp = s / per;
      e = s - grp * per;
      t = 8 * grp + (u & 7);
    } else {
      const int r = u - full, dt = r / per;
      e = r - dt * per;
      t = (p.T & ~7) + dt;
    }
    return Item{t, e / p.n_chunks, e % p.n_chunks};
  };
  Item it = item_of(0);
  int k3 = 0, t3 = it.t, a3 = it.chunk * tpc, e3 = a3 + tpc;
  auto step3 = [&]() __attribute__((always_inline)) {
    if (++a3 == e3) {
      ++k3;
      const Item c = item_of(k3);
      t3 = c.t;
      a3 = c.chunk * tpc;
      e3 = a3 + tpc;
    }
  };
  const int srow = tid >> 4, sq = tid & 15;

  bf16x8 qop[QS];
  float snx;  // raw sink value of the current item's PV head (see load_sink)
  auto load_q_from = [&](const uint16_t *qrow, int step) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < QS; ++s)
      qop[s] = __builtin_bit_cast(bf16x8, *(gu32x4 *)(qrow + (int64_t)step * s));
  };
  auto q_row = [&](const Item &itm) __attribute__((always_inline)) -> const uint16_t * {
    const int head = itm.hg * HG + 16 * hq + li;
    return p.q + (int64_t)itm.t * p.q_st + (int64_t)(head < p.h ? head : 0) * p.q_sh + 544 * dh +
           8 * g;
  };
  auto load_q = [&](const Item &itm) __attribute__((always_inline)) { load_q_from(q_row(itm), 32); };
  // sink logit of an item's PV head j, loaded during its last tile (a valid dummy address
  // when there is none)
  auto load_sink = [&](const Item &itm) __attribute__((always_inline)) {
    snx = *(gf32 *)(p.sink ? p.sink + min(itm.hg * HG + j, p.h - 1) : (const float *)p.q);
  };
  f32x16 oacc[4];  // O^T of d 128w + 32db .., heads j
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  // Running max (log2 units): m0 for the PV head j, mq for the QK head 16hq + li; the same
  // for a head in every wave and lane that holds it.
  float m0 = neg_inf(), mq = neg_inf();
  float l_part = 0.f;  // QK role (dh 0): head 16hq + li, this lane's keys

  // rolling gather registers: piece m (bytes 8(16m + s) ..) of this thread's row and its
  // group scale; the ninth piece exists for s < 8 only (others reload piece 128 + s%8)
  u32x2 cv[kXPieces];
  float cs[kXPieces];
  auto piece_of = [&](int m) { return m < 8 ? 16 * m + sq : 128 + (sq & 7); };
  // per-thread byte offsets, so each piece is a base plus an immediate: data 8s (+128m),
  // scale of group 2m + s/8 at 4(s/8) (+8m); the ninth piece at 1024 + 8(s%8), group 16
  const int doff = 8 * sq, soff = 4 * (sq >> 3), doff8 = 1024 + 8 * (sq & 7);
  auto issue_piece = [&](int m, const RowAddr &a) __attribute__((always_inline)) {
    if (m < 8) {
      cv[m] = *(gu32x2 *)(a.data + doff + 128 * m);
      cs[m] = *(gf32 *)(a.scale + soff + 8 * m);
    } else {
      cv[m] = *(gu32x2 *)(a.data + doff8);
      cs[m] = *(gf32 *)(a.scale + 64);
    }
  };
  auto commit_piece = [&](int m, uint16_t *row) __attribute__((always_inline)) {
    if (m < 8 || sq < 8) *(lu32x4 *)(row + 8 * piece_of(m)) = fp8x8_to_bf16x8(cv[m], cs[m]);
  };
  auto zero_row = [&](uint16_t *row) __attribute__((always_inline)) {
    // (lanes s and s + 8 both clear the ninth piece)
#pragma unroll
    for (int m = 0; m < kXPieces; ++m) *(lu32x4 *)(row + 8 * piece_of(m)) = u32x4{0, 0, 0, 0};
  };
  auto pool_of = [&](int ab) -> const PoolArgs & {
    return ab < p.main_tiles || ab >= n_tiles ? p.kv : p.ex;
  };
  auto fp8_at = [&](int ab) { return ab < n_tiles && tile_is_fp8<TILE>(p, ab); };
  // one unconditional load per tile; the ids are masked when committed (slots_at runs with
  // the t3 of the load)
  auto idx_at = [&](int t, int ab) -> int32_t {
    return idx_load<TILE>(p, t, min(ab, n_tiles - 1));
  };
  auto slots_at = [&](int gg, int ab, int32_t s32) __attribute__((always_inline)) {
    const int tl = min(ab, n_tiles - 1);
    const PoolArgs &pl = tl < p.main_tiles ? p.kv : p.ex;
    const uint64_t live = ab < n_tiles ? live_mask<TILE>(p, t3, tl) : 0;
    const uint64_t m = __ballot(s32 >= 0 && (int64_t)s32 < pl.num_slots) & live;
    slots[gg & 3][lane] = keep_lanes(m, s32, lane);
    if (lane == 0) vmask[gg & 3] = m;
  };

  // prologue: slots of tiles 0..2; tile 0 into buffer 0; tile 1 in flight
  const int n = G_all;
  auto prologue_tile = [&](int i) __attribute__((always_inline)) {
    const int ab = a3;
    if (w == 0 && i < n) slots_at(i, ab, idx_at(t3, ab));
    if (i + 1 < n) step3();
    return ab;
  };
  const int a0 = prologue_tile(0);
  int a1 = prologue_tile(1);
  int a2 = prologue_tile(2);
  __syncthreads();
  if (n > 0 && (F8ONLY || fp8_at(a0))) {
    const RowAddr a = slot_addr(pool_of(a0), slots[0][srow]);
    const bool ok = (vmask[0] >> srow) & 1;
#pragma unroll
    for (int m = 0; m < kXPieces; ++m) issue_piece(m, a);
    load_q(it);
#pragma unroll
    for (int m = 0; m < kXPieces; ++m) commit_piece(m, tiles[0] + srow * RS);
    if (!ok) zero_row(tiles[0] + srow * RS);
  } else {
    if (n > 0) x_dma16(pool_of(a0), slots[0], vmask[0], tiles[0], w, lane);
    load_q(it);
  }
  // q has landed before the loop on every path, so no wait in the loop is for q
  __builtin_amdgcn_s_waitcnt(0);
  if (F8ONLY ? n > 0 : (n > 1 && fp8_at(a1))) {
    const int s1 = min(1, n - 1);
    const RowAddr a = slot_addr(pool_of(a1), slots[s1][srow]);
#pragma unroll
    for (int m = 0; m < kXPieces; ++m) issue_piece(m, a);
  }
  __syncthreads();

  int32_t idx3 = -1;
  f32x4 sacc;         // partial, then full S^T: keys 16kb + 4g + e, head 16hq + li
  float psum = 0.f;   // this tile's row sum for head 16hq + li, this lane's keys (dh 0)
  float tpart = neg_inf();
  bool any_need = false;
  float tm0 = neg_inf();
  bool g_c8 = false, g_i8 = false, g_fix = false;
  RowAddr g_ai = {nullptr, nullptr};
  uint16_t *g_crow = nullptr;
  auto gather_step = [&](int m) __attribute__((always_inline)) {
    if (g_c8) commit_piece(m, g_crow);
    if (g_i8) issue_piece(m, g_ai);
  };
  uint32_t vm16 = 0xffffu;  // valid bits of this wave's key block
  // Softmax of this wave's block relative to mq: mask, tile max, P (bf16) into the exchange
  // buffer in the PV B-operand layout (dh 0 writes; its partner computes the same values).
  auto softmax = [&](bool rewrite) __attribute__((always_inline)) {
    const float mu = mq == neg_inf() ? 0.0f : mq;
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float xv = sacc[e];
      if (vm16 != 0xffffu) xv = __builtin_amdgcn_ubfe(vm16, 4 * g + e, 1) ? xv : neg_inf();
      if (!rewrite) tpart = fmaxf(tpart, xv);
      pr[e] = fast_exp2(fmaf(xv, p.scale_log2, -mu));
      psum += pr[e];
    }
    if (dh == 0) {
      const u32x2 v = {pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3])};
      typedef __attribute__((address_space(3))) u32x2 lu32x2;
      typedef __attribute__((address_space(3))) char lchar;
      *(lu32x2 *)((lchar *)&pbuf[kb][(g & 1) * 32 + 16 * hq + li] + 8 * (g >> 1)) = v;
    }
  };

  Item nxt = it;  // item whose q the last tile of the current item loads
  bool more = true;  // the current item is not this workgroup's last
  auto front = [&](int i, auto lastq) __attribute__((always_inline)) {
    const int cur = i & 1;
    const bool c8 = i + 1 < n && (F8ONLY || fp8_at(a1));
    // fp8 pieces of tile i+2 are loaded whatever its kind (a bf16 tile's row is read but
    // never committed), so the loads in flight stay countable
    const bool i8 = true;
    if (!F8ONLY && i + 1 < n && !c8)
      x_dma16(pool_of(a1), slots[(i + 1) & 3], vmask[(i + 1) & 3], tiles[cur ^ 1], w, lane);
    idx3 = idx_at(t3, a3);
    const int s1 = min(i + 1, n - 1);
    const int s2 = min(i + 2, n - 1);
    const uint64_t vm1 = vmask[s1 & 3];
    g_c8 = c8;
    g_i8 = i8;
    g_fix = c8 && !((vm1 >> srow) & 1);
    g_ai = slot_addr(pool_of(a2), slots[s2 & 3][srow]);
    g_crow = tiles[cur ^ 1] + srow * RS;
    vm16 = __builtin_amdgcn_readfirstlane((uint32_t)(vmask[i & 3] >> (16 * kb)) & 0xffffu);
    psum = 0.f;
    tpart = neg_inf();

    const uint16_t *kr = tiles[cur] + (16 * kb + li) * RS + 544 * dh + 8 * g;
    constexpr int LA = 2;
    constexpr int NR = LA + 1;
    bf16x8 abuf[NR];
#pragma unroll
    for (int s = 0; s < LA; ++s) abuf[s] = *reinterpret_cast<const bf16x8 *>(kr + 32 * s);
    static_for<0, QS>([&](auto sc) __attribute__((always_inline)) {
      constexpr int s = decltype(sc)::value;
      if constexpr (s + LA < QS)
        abuf[(s + LA) % NR] = *reinterpret_cast<const bf16x8 *>(kr + 32 * (s + LA));
      if constexpr (s == 0)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abuf[0], qop[0], f32x4{}, 0, 0, 0);
      else
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abuf[s % NR], qop[s], sacc, 0, 0, 0);
      if constexpr (s % 3 == 2) gather_step(s / 3);  // pieces 0..4
      if constexpr (s == QS - 1) gather_step(5);
      __builtin_amdgcn_sched_barrier(0);
    });
    // last tile of an item: q of the next item goes out now that this one's is consumed
    // (after the last item the loads still go out, so the loads in flight stay countable,
    // but all of them read the same 16 bytes: one line instead of 147 KB per CU, whose
    // redundant fetch holds the waves for about 3 us)
    if constexpr (decltype(lastq)::value) {
      load_q_from(more ? q_row(nxt) : p.q, more ? 32 : 0);
      load_sink(it);
    }
    // sum the two d halves
    exch[w][lane] = sacc;
    __syncthreads();
    sacc += exch[w ^ 4][lane];
    softmax(false);
    float tmax = fmaxf(tpart, __shfl_xor(tpart, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * p.scale_log2;
    if (dh == 0 && g == 0) tmx[kb][16 * hq + li] = tmax;
    __syncthreads();
    tm0 = fmaxf(tmx[0][j], tmx[1][j]);
    any_need = __any(tm0 > m0 + kRescaleLog2);
  };

  auto back = [&](int i) __attribute__((always_inline)) {
    const int cur = i & 1;
    if (dh == 0) l_part += psum;
    const int G = lane >> 4, lt = lane & 15;
    const uint16_t *vbase =
        tiles[cur] + (4 * q + (lt >> 2)) * RS + 128 * w + 16 * (G & 1) + 4 * (lt & 3);
    auto load_v = [&](int db, int ks) __attribute__((always_inline)) -> bf16x8 {
      const uint16_t *src = vbase + 16 * ks * RS + 32 * db;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4 *)(src));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((li16x4 *)(src + 8 * RS));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      const u32x4 a4 = {l2[0], l2[1], h2[0], h2[1]};
      return __builtin_bit_cast(bf16x8, a4);
    };
    constexpr int LV = 2;
    constexpr int NV = LV + 1;
    bf16x8 vb[NV];
    bf16x8 pb;
#pragma unroll
    for (int k = 0; k < LV; ++k) vb[k] = load_v(k & 3, k >> 2);
    static_for<0, 8>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value, ks = k >> 2, db = k & 3;
      if constexpr (db == 0) pb = __builtin_bit_cast(bf16x8, pbuf[ks][lane]);
      if constexpr (k + LV < 8) vb[(k + LV) % NV] = load_v((k + LV) & 3, (k + LV) >> 2);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[k % NV], pb, oacc[db], 0, 0, 0);
      if constexpr (k == 1 || k == 4 || k == 7) gather_step(6 + k / 3);  // pieces 6..8
      __builtin_amdgcn_sched_barrier(0);
    });
    if (g_fix) zero_row(g_crow);
    if (w == 0 && i + 3 < n) slots_at(i + 3, a3, idx3);
    if (!F8ONLY && i + 1 < n && !fp8_at(a1)) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    a1 = a2;
    a2 = a3;
    if (i + 4 < n) step3();
  };

  // Rare: some head's max grew by more than 2^8 (always on the first tile of an item with a
  // valid key). Move the reference, rescale O and l, and redo this wave's P.
  auto rescale = [&]() __attribute__((always_inline)) {
    const bool n0 = tm0 > m0 + kRescaleLog2;
    const float nm0 = n0 ? tm0 : m0;
    const float f0 = n0 ? fast_exp2(m0 - nm0) : 1.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] *= f0;
    m0 = nm0;
    const float tq = fmaxf(tmx[0][16 * hq + li], tmx[1][16 * hq + li]);
    if (tq > mq + kRescaleLog2) {
      l_part *= fast_exp2(mq - tq);
      mq = tq;
    }
    psum = 0.f;
    softmax(true);
    __syncthreads();
  };

  int i = 0;  // tile of the stream
  for (int k = 0; k < n_items; ++k) {
    const int ilast = i + tpc - 1;
    more = k + 1 < n_items;
    nxt = more ? item_of(k + 1) : it;
    while (i < ilast) {
      for (; i < ilast; ++i) {
        front(i, std::false_type{});
        if (any_need) break;
        back(i);
      }
      if (i >= ilast) break;
      rescale();
      back(i);
      ++i;
    }
    front(i, std::true_type{});
    if (any_need) rescale();
    back(i);
    ++i;
    // Item done: row sums of the QK heads, then of the PV heads.
    const Item done = it;
    it = nxt;
    {
      float lw = l_part + __shfl_xor(l_part, 16);
      lw += __shfl_xor(lw, 32);
      if (dh == 0 && g == 0) lsum[kb][16 * hq + li] = lw;
    }
    __syncthreads();
    // q and the sinks land here; the three fp8 pieces of the PV half stay in flight
    wait_vmcnt<6>();
    const float l = lsum[0][j] + lsum[1][j];
    // Outputs, staged as in the 576 kernel: each wave writes its bf16 rows (32 heads x its
    // 128 columns, rows 136 elements apart) into the consumed tile buffer, then stores 16
    // contiguous bytes per lane, 16 lanes per 256-byte row segment.
    constexpr int SR = 136;
    uint16_t *stg = tiles[(i - 1) & 1] + w * (HG * SR);
    {
      const int head = done.hg * HG + j;
      const float m = m0;
      float scale;
      if (p.n_chunks > 1) {
        scale = l > 0.f ? 1.0f / l : 0.f;
        if (head < p.h && w == 0 && q == 0) {
          const int64_t row = ((int64_t)done.t * p.n_chunks + done.chunk) * p.h + head;
          p.ws_ml[row * 2 + 0] = m;
          p.ws_ml[row * 2 + 1] = l;
        }
      } else {
        const float sig = p.sink ? snx * kLog2e : neg_inf();
        const float mf = fmaxf(m, sig);
        float lse = neg_inf();
        scale = 0.f;
        if (mf != neg_inf()) {
          const float fo = m == neg_inf() ? 0.f : fast_exp2(m - mf);
          const float fs = sig == neg_inf() ? 0.f : fast_exp2(sig - mf);
          const float den = l * fo + fs;
          scale = fo / den;
          lse = (mf + __log2f(den)) * kLn2;
        }
        if (p.lse && head < p.h && w == 0 && q == 0) p.lse[(int64_t)done.t * p.lse_st + head] = lse;
      }
      typedef __attribute__((address_space(3))) u32x2 lu32x2;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const u32x2 pk = {pack_bf16(oacc[db][4 * b] * scale, oacc[db][4 * b + 1] * scale),
                            pack_bf16(oacc[db][4 * b + 2] * scale, oacc[db][4 * b + 3] * scale)};
          *(lu32x2 *)(stg + j * SR + 32 * db + 8 * b + 4 * q) = pk;
        }
    }
    {
      const int c = lane & 15;  // 8-column chunk of this wave's 128
#pragma unroll
      for (int r = 0; r < HG / 4; ++r) {
        const int hl = 4 * r + (lane >> 4);
        const int head = done.hg * HG + hl;
        const u32x4 v = *(lu32x4 *)(stg + hl * SR + 8 * c);
        if (head < p.h) {
          uint16_t *dst =
              p.n_chunks > 1
                  ? p.ws_o + (((int64_t)done.t * p.n_chunks + done.chunk) * p.h + head) * D_V
                  : p.out + (int64_t)done.t * p.out_st + (int64_t)head * p.out_sh;
          *reinterpret_cast<u32x4 *>(dst + 128 * w + 8 * c) = v;
        }
      }
    }
    // the staging area is the buffer the next item's first commits write
    __syncthreads();
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    m0 = mq = neg_inf();
    l_part = 0.f;
  }
}

// Merge split-K partials of one (token, head) with the sink; 64 threads.
template <int D_V>
__global__ __launch_bounds__(64) void smla_combine_kernel(const KParams p) {
  // (token, head) -> block as the attention kernel maps its items: the heads of a token
  // run on the XCD whose L2 its partials were written through.
  const int u = blockIdx.x, full = (p.T >> 3) * 8 * p.h;
  int t, head;
  if (u < full) {
    const int s = u >> 3, grp = s / p.h;
    head = s - grp * p.h;
    t = 8 * grp + (u & 7);
  } else {
    const int r = u - full;
    t = (p.T & ~7) + r / p.h;
    head = r % p.h;
  }
  const int lane = threadIdx.x;
  const int64_t base = (int64_t)t * p.n_chunks * p.h + head;
  float mmax = neg_inf();
#pragma unroll 8
  for (int c = 0; c < p.n_chunks; ++c) mmax = fmaxf(mmax, p.ws_ml[(base + (int64_t)c * p.h) * 2]);
  const float sig = p.sink ? p.sink[head] * kLog2e : neg_inf();
  const float mf = fmaxf(mmax, sig);
  constexpr int PER = D_V / 64;
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  float den = 0.f, lse = neg_inf();
  if (mf != neg_inf()) {
    // chunk c holds O_c / l_c (zeros when empty); its weight in the merge is
    // l_c 2^(m_c - mf). No branch per chunk, so the loads of several chunks are in flight.
#pragma unroll 8
    for (int c = 0; c < p.n_chunks; ++c) {
      const int64_t row = base + (int64_t)c * p.h;
      const float mc = p.ws_ml[row * 2], lc = p.ws_ml[row * 2 + 1];
      const float f = mc == neg_inf() ? 0.f : lc * fast_exp2(mc - mf);
      den += f;
      const uint16_t *src = p.ws_o + row * D_V + PER * lane;
#pragma unroll
      for (int j = 0; j < PER; j += 8) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(src + j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[j + 2 * e] += __uint_as_float(v[e] << 16) * f;
          acc[j + 2 * e + 1] += __uint_as_float(v[e] & 0xffff0000u) * f;
        }
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


}  // namespace

Variant choose_variant(int d_qk, int h) {
  // 576: the wide kernel, 64 heads per workgroup above 32 heads, else 32.
  // 1088: the 1088 wide kernel, 32 heads per workgroup.
  if (d_qk == 576) return h > 32 ? Variant{576, 512, 64, 2} : Variant{576, 512, 64, 1};
  return {1088, 1024, 32, 1};
}

template <bool F8ONLY, int NHB, bool S64 = false>
hipError_t launch_wide(const KParams &p, hipStream_t s) {
  hipLaunchKernelGGL((smla_wide_kernel<F8ONLY, NHB, S64>), dim3((unsigned)p.grid),
                     dim3(kEThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attention(const Variant &v, const KParams &p, hipStream_t s) {
  if (v.d_qk == 576) {
    const bool f8only = p.kv.fp8 && (p.topk_extra == 0 || p.ex.fp8);
    if (v.hb == 1) return f8only ? launch_wide<true, 1>(p, s) : launch_wide<false, 1>(p, s);
    if (p.n_chunks > 1)  // split-K decode: QK on one wave per SIMD (see the kernel)
      return f8only ? launch_wide<true, 2, true>(p, s) : launch_wide<false, 2, true>(p, s);
    return f8only ? launch_wide<true, 2>(p, s) : launch_wide<false, 2>(p, s);
  }
  const bool f8only = p.kv.fp8 && (p.topk_extra == 0 || p.ex.fp8);
  if (f8only)
    hipLaunchKernelGGL(smla_wide1088_kernel<true>, dim3((unsigned)p.grid), dim3(kEThreads), 0, s, p);
  else
    hipLaunchKernelGGL(smla_wide1088_kernel<false>, dim3((unsigned)p.grid), dim3(kEThreads), 0, s, p);
  return hipGetLastError();
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
