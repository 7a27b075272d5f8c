// Internal interface between the C-ABI host layer (api.cpp) and the HIP kernels (attn.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

// One pool as the kernels see it; page_block_size is fixed at 64 (shift 6).
struct PoolArgs {
  const uint8_t *data;
  const uint8_t *scales;
  int64_t num_slots;
  int64_t page_stride, row_stride;
  int64_t scale_page_stride, scale_row_stride;
  int32_t fp8;  // 1: e4m3fn + per-64 fp32 scales, 0: bf16
  // The strides again in 32 bits, for the decode and narrow kernels, which the host takes
  // only when the page strides fit 32 bits and the row strides 24 (so that a row address is
  // one 32 x 32 -> 64-bit multiply-add and one 24-bit multiply)
  uint32_t page_stride32, row_stride32, scale_page_stride32, scale_row_stride32;
  int32_t pad_;
};

struct KParams {
  const uint16_t *q;
  int64_t q_st, q_sh;
  PoolArgs kv, ex;
  const int32_t *idx;
  int64_t idx_st;
  const int32_t *eidx;
  int64_t eidx_st;
  int32_t topk, topk_extra;
  int32_t main_tiles;  // index tiles of the main row, ceil(topk / tile); extra tiles follow
  int32_t n_tiles;     // main_tiles + ceil(topk_extra / tile)
  const int32_t *len;   // [T] live main entries per row, or nullptr (all topk)
  const int32_t *elen;  // [T] live extra entries per row, or nullptr (all topk_extra)
  const float *sink;  // nullptr: no sink
  float scale_log2;   // sm_scale * log2(e)
  uint16_t *out;
  int64_t out_st, out_sh;
  float *lse;  // nullptr: not written
  int64_t lse_st;
  int32_t T, h;
  int32_t n_hg;      // head groups per token
  int32_t n_chunks;  // index chunks per token (1: finalize in place)
  int32_t tiles_per_chunk;
  int32_t grid;      // workgroups launched; each walks work items grid apart
  uint16_t *ws_o;  // [T][n_chunks][h][d_v] partial O / l in bf16, when n_chunks > 1
  float *ws_ml;  // [T][n_chunks][h][2]  (m in log2 units, l)
  uint32_t *arrivals;  // decode16 split items: [T][n_hg] counters of chunks whose partial
                       // is stored, zero on entry and on exit
};

// Kernel variant. d_qk 576: the wide kernel with hb head blocks of 32 per workgroup (2 for
// more than 32 heads, else 1). d_qk 1088: the 1088 wide kernel, 32 heads per workgroup.
struct Variant {
  int d_qk, d_v, tile, hb;
  int heads_per_group() const { return 32 * hb; }
};

// Packing: bf16 rows [n, d_qk] -> e4m3fn payload and per-64 fp32 scales in their slots.
struct PackParams {
  const uint16_t *rows;
  int64_t rows_st;  // elements
  const int32_t *slots;
  int64_t n;
  int32_t d_qk;
  PoolArgs kv;         // destination geometry
  uint8_t *kv_data;    // writable views of kv.data and kv.scales
  uint8_t *kv_scales;
};

// Scratch of the no-allocation decode entry point (sparse_mla_decode_noalloc): a
// file-scope device array of kScratchBytes in attn.hip, one copy per device. *ptr receives
// the current device's copy (its address is looked up once per device).
constexpr size_t kScratchBytes = size_t(32) << 20;
hipError_t scratch_region(void **ptr);

// Decode kernel (decode.hip): 16 heads per workgroup, d_qk 576, fp8 pools, one work item
// (token, head group, chunk of at most kDMaxTiles index tiles of 64) per workgroup. Split
// items keep their partials in the workspace as T * n_hg * n_chunks blocks of 16 KB (bf16 O / l
// of 16 heads x 512, in the kernel's register order) followed by [T][n_hg][n_chunks][16][2]
// fp32 (m, l), and meet in arrival counters.
constexpr int kDMaxTiles = 4;
constexpr int kArrivalSlots = 1 << 18;
// The current device's pool of arrival counters (kArrivalSlots, zero when idle).
hipError_t arrival_region(uint32_t **ptr);
hipError_t launch_decode16(const KParams &p, hipStream_t s);

// Narrow kernel (narrow_kernel.h; instances in narrow.hip and narrow_fp8.hip): prefill form,
// d_qk 576, fp8 pools, heads_per_group (32) heads per work item and every item walking its
// token's whole index list (n_tiles >= 2); one workgroup per CU walks items grid apart.
// fp8_q: the fp8 compute mode (q rounded to e4m3fn per (token, head), QK on fp8 MFMA over
// the raw rows).
hipError_t launch_narrow(const KParams &p, int heads_per_group, bool fp8_q, hipStream_t s);
hipError_t launch_narrow_fp8(const KParams &p, hipStream_t s);  // the fp8_q instance

// Role-split kernel (roles.hip): prefill form, d_qk 576, fp8 pools, bf16 compute, 64 heads
// per work item (n_hg = ceil(h / 64)), every item walking its token's whole index list; one
// workgroup per CU walks items grid apart.
hipError_t launch_roles(const KParams &p, hipStream_t s);

Variant choose_variant(int d_qk, int h);
hipError_t launch_pack(const PackParams &p, hipStream_t s);
// fp8 compute mode: 32 heads per workgroup, 32-key tiles, one workgroup per (token, group).
hipError_t launch_fp8qk(const KParams &p, hipStream_t s);
hipError_t launch_attention(const Variant &v, const KParams &p, hipStream_t s);
hipError_t launch_combine(const Variant &v, const KParams &p, hipStream_t s);

}  // namespace smla
