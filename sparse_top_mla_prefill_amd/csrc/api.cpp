// C-ABI host layer of libsparse_mla: validation, envelope query, work decomposition, launch.
//
// The error convention follows the pages:
//   - "fix(sparse-mla-sm120): add topk=256 prefill-dsv4 dispatch", section Description:
//     an unsupported call fails loudly with a fixed prefix that lists num_heads, topk,
//     page_block_size, topk_extra and extra_page_block_size.
//   - "fix(sm120): explain sparse-MLA decode dispatch misses; add config query API",
//     description: after that prefix the message names the parameter that missed and
//     lists the supported values.
//   - The FlashInfer 4802 message, section "Plan layer": page_block_size is checked.
//     Section Summary: a T = 0 call is a no-op, and out_lse and index rows may be
//     strided.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/sparse_mla.h"
#include "smla_internal.h"

namespace {

thread_local std::string g_last_error;

int set_error(int code, const char *fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

std::string prefix(const smla_args *a, const char *form) {
  char buf[512];
  snprintf(buf, sizeof(buf),
           "Unsupported sparse-MLA %s configuration: num_heads=%d topk=%d page_block_size=%d "
           "topk_extra=%d extra_page_block_size=%d d_qk=%d d_v=%d",
           form, a->h, a->topk, a->kv.page_block_size, a->topk_extra,
           a->topk_extra > 0 ? a->extra.page_block_size : 0, a->d_qk, a->d_v);
  return buf;
}

constexpr int kMaxHeads = 128;
constexpr int kTopkMultiple = 1;  // any width; a partial last index tile is masked
constexpr int kPageBlock = 64;
constexpr int kDecodeMaxTokens = 64;
constexpr int kMaxTopkTotal = 1 << 24;  // keeps every entry position inside int32

int ceil_div(int a, int b) { return (a + b - 1) / b; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_cache(int d_qk, const smla_cache &c, const char *name, const std::string &pre) {
  if (c.dtype != SMLA_BF16 && c.dtype != SMLA_FP8_E4M3_G64)
    return set_error(SMLA_ERR_UNSUPPORTED, "%s: %s dtype=%d is not one of {0 (bf16), 1 (fp8 e4m3 "
                     "+ fp32 scale per 64)}", pre.c_str(), name, c.dtype);
  if (c.page_block_size != kPageBlock)
    return set_error(SMLA_ERR_UNSUPPORTED, "%s: %s page_block_size=%d is not supported "
                     "(supported: 64)", pre.c_str(), name, c.page_block_size);
  if (!c.data) return set_error(SMLA_ERR_INVALID, "%s: %s data is NULL", pre.c_str(), name);
  if (!aligned(c.data, 16))
    return set_error(SMLA_ERR_INVALID, "%s: %s data is not 16-byte aligned", pre.c_str(), name);
  if (c.num_pages < 1)
    return set_error(SMLA_ERR_INVALID, "%s: %s num_pages=%lld must be >= 1", pre.c_str(), name,
                     (long long)c.num_pages);
  if (c.num_pages > (int64_t(1) << 40))
    return set_error(SMLA_ERR_INVALID, "%s: %s num_pages=%lld is too large", pre.c_str(), name,
                     (long long)c.num_pages);
  const int64_t payload = (int64_t)d_qk * (c.dtype == SMLA_BF16 ? 2 : 1);
  if (c.row_stride < payload || c.row_stride % 16)
    return set_error(SMLA_ERR_INVALID, "%s: %s row_stride=%lld must be a multiple of 16 and >= "
                     "the %lld-byte row payload", pre.c_str(), name, (long long)c.row_stride,
                     (long long)payload);
  if (c.page_stride < kPageBlock * c.row_stride || c.page_stride % 16)
    return set_error(SMLA_ERR_INVALID, "%s: %s page_stride=%lld must be a multiple of 16 and >= "
                     "page_block_size * row_stride = %lld", pre.c_str(), name,
                     (long long)c.page_stride, (long long)(kPageBlock * c.row_stride));
  if (c.dtype == SMLA_FP8_E4M3_G64) {
    const int64_t sbytes = 4 * (d_qk / 64);
    if (!c.scales) return set_error(SMLA_ERR_INVALID, "%s: %s scales is NULL for an fp8 pool",
                                    pre.c_str(), name);
    if (!aligned(c.scales, 4))
      return set_error(SMLA_ERR_INVALID, "%s: %s scales is not 4-byte aligned", pre.c_str(), name);
    if (c.scale_row_stride < sbytes || c.scale_row_stride % 4)
      return set_error(SMLA_ERR_INVALID, "%s: %s scale_row_stride=%lld must be a multiple of 4 "
                       "and >= %lld", pre.c_str(), name, (long long)c.scale_row_stride,
                       (long long)sbytes);
    if (c.scale_page_stride < kPageBlock * c.scale_row_stride || c.scale_page_stride % 4)
      return set_error(SMLA_ERR_INVALID, "%s: %s scale_page_stride=%lld must be a multiple of 4 "
                       "and >= page_block_size * scale_row_stride = %lld", pre.c_str(), name,
                       (long long)c.scale_page_stride,
                       (long long)(kPageBlock * c.scale_row_stride));
  }
  return SMLA_OK;
}

// Validate everything except the workspace. Returns SMLA_OK, or an error with text set.
// Entry point forms: the two regimes, and the routed entry that picks one of them.
enum Form { kPrefill = 0, kDecode = 1, kForward = 2 };
const char *form_name(int f) {
  return f == kDecode ? "decode" : f == kForward ? "forward" : "prefill";
}

int validate(const smla_args *a, int f) {
  if (!a) return set_error(SMLA_ERR_INVALID, "sparse-MLA: args is NULL");
  const char *form = form_name(f);
  const bool decode = f == kDecode;
  const std::string pre = prefix(a, form);
  if (a->T < 0) return set_error(SMLA_ERR_INVALID, "%s: T=%d is negative", pre.c_str(), a->T);
  if (decode && a->T > kDecodeMaxTokens)
    return set_error(SMLA_ERR_UNSUPPORTED, "%s: num_tokens=%d exceeds the decode limit of %d rows "
                     "(use sparse_mla_prefill, which serves any T)", pre.c_str(), a->T,
                     kDecodeMaxTokens);
  if (a->h < 1 || a->h > kMaxHeads)
    return set_error(SMLA_ERR_UNSUPPORTED, "%s: num_heads=%d outside [1,%d] (supported: any head "
                     "count from 1 to 128)", pre.c_str(), a->h, kMaxHeads);
  if (!((a->d_qk == 576 && a->d_v == 512) || (a->d_qk == 1088 && a->d_v == 1024)))
    return set_error(SMLA_ERR_UNSUPPORTED, "%s: (d_qk, d_v)=(%d, %d) is not supported (supported: "
                     "(576, 512), (1088, 1024))", pre.c_str(), a->d_qk, a->d_v);
  if (a->topk <= 0)
    return set_error(SMLA_ERR_UNSUPPORTED, "%s: topk=%d must be >= 1 (supported: any positive "
                     "width)", pre.c_str(), a->topk);
  if (a->topk_extra < 0)
    return set_error(SMLA_ERR_UNSUPPORTED, "%s: topk_extra=%d must be >= 0", pre.c_str(),
                     a->topk_extra);
  if ((int64_t)a->topk + a->topk_extra > kMaxTopkTotal)
    return set_error(SMLA_ERR_UNSUPPORTED, "%s: topk + topk_extra = %lld exceeds %d",
                     pre.c_str(), (long long)a->topk + a->topk_extra, kMaxTopkTotal);
  if (!std::isfinite(a->sm_scale) || !(a->sm_scale > 0.f))
    return set_error(SMLA_ERR_INVALID, "%s: sm_scale=%g must be finite and > 0", pre.c_str(),
                     (double)a->sm_scale);
  if (a->compute_mode != SMLA_COMPUTE_BF16 && a->compute_mode != SMLA_COMPUTE_FP8)
    return set_error(SMLA_ERR_INVALID, "%s: compute_mode=%d is not 0 (bf16) or 1 (fp8)",
                     pre.c_str(), a->compute_mode);
  if (a->compute_mode == SMLA_COMPUTE_FP8) {
    if (decode)
      return set_error(SMLA_ERR_UNSUPPORTED, "%s: compute_mode=1 (fp8) serves the prefill and "
                       "routed forms only", pre.c_str());
    if (a->d_qk != 576 || a->kv.dtype != SMLA_FP8_E4M3_G64 || a->topk_extra != 0)
      return set_error(SMLA_ERR_UNSUPPORTED, "%s: compute_mode=1 (fp8) serves d_qk 576 over an "
                       "fp8 main pool with no extra cache (got kv dtype=%d)", pre.c_str(),
                       a->kv.dtype);
  }
  if (a->T == 0) return SMLA_OK;

  if (!a->q) return set_error(SMLA_ERR_INVALID, "%s: q is NULL", pre.c_str());
  if (!aligned(a->q, 16) || a->q_stride_t % 8 || a->q_stride_h % 8 || a->q_stride_h < 0 ||
      a->q_stride_t < 0)
    return set_error(SMLA_ERR_INVALID, "%s: q must be 16-byte aligned with non-negative strides "
                     "that are multiples of 8 elements (q_stride_t=%lld q_stride_h=%lld)",
                     pre.c_str(), (long long)a->q_stride_t, (long long)a->q_stride_h);
  int rc = check_cache(a->d_qk, a->kv, "kv", pre);
  if (rc) return rc;
  if (!a->indices) return set_error(SMLA_ERR_INVALID, "%s: indices is NULL", pre.c_str());
  if (!aligned(a->indices, 4) || a->indices_stride < a->topk)
    return set_error(SMLA_ERR_INVALID, "%s: indices_stride=%lld must be >= topk=%d (and indices "
                     "4-byte aligned)", pre.c_str(), (long long)a->indices_stride, a->topk);
  if (a->topk_extra > 0) {
    rc = check_cache(a->d_qk, a->extra, "extra", pre);
    if (rc) return rc;
    if (!a->extra_indices)
      return set_error(SMLA_ERR_INVALID, "%s: extra_indices is NULL with topk_extra=%d",
                       pre.c_str(), a->topk_extra);
    if (!aligned(a->extra_indices, 4) || a->extra_indices_stride < a->topk_extra)
      return set_error(SMLA_ERR_INVALID, "%s: extra_indices_stride=%lld must be >= topk_extra=%d",
                       pre.c_str(), (long long)a->extra_indices_stride, a->topk_extra);
  }
  if (!aligned(a->topk_length, 4) || (a->topk_extra > 0 && !aligned(a->extra_topk_length, 4)))
    return set_error(SMLA_ERR_INVALID, "%s: topk_length / extra_topk_length must be 4-byte "
                     "aligned", pre.c_str());
  if (!a->out) return set_error(SMLA_ERR_INVALID, "%s: out is NULL", pre.c_str());
  if (!aligned(a->out, 8) || a->out_stride_t % 4 || a->out_stride_h % 4 || a->out_stride_h < 0 ||
      a->out_stride_t < 0)
    return set_error(SMLA_ERR_INVALID, "%s: out must be 8-byte aligned with non-negative strides "
                     "that are multiples of 4 elements", pre.c_str());
  if (a->lse && (!aligned(a->lse, 4) || a->lse_stride_t < a->h))
    return set_error(SMLA_ERR_INVALID, "%s: lse_stride_t=%lld must be >= num_heads=%d",
                     pre.c_str(), (long long)a->lse_stride_t, a->h);
  return SMLA_OK;
}

struct Plan {
  smla::Variant v;
  int kind;  // 0: wide kernels (plus the combine pass when split), 1: the decode kernel,
             // 2: the narrow kernel (prefill, few heads), 3: the role-split kernel (prefill,
             // more heads)
  int n_hg, n_chunks, tiles_per_chunk;
  size_t ws_bytes;
};

// Largest chunk count the decode kernel takes: its last chunk to finish reads the others'
// partials, 16 KB each.
constexpr int kD16MaxChunks = 8;

// The decode and narrow kernels form row addresses from 32-bit strides: page strides below
// 2^32 and row strides below 2^24 bytes (every layout of a real pool); other pools take the
// wide kernels.
bool short_strides(const smla_cache &c) {
  const int64_t p32 = int64_t(1) << 32, r24 = int64_t(1) << 24;
  return c.page_stride < p32 && c.row_stride < r24 &&
         (c.dtype != SMLA_FP8_E4M3_G64 || (c.scale_page_stride < p32 && c.scale_row_stride < r24));
}

bool fp8_only(const smla_args *a) {
  return a->kv.dtype == SMLA_FP8_E4M3_G64 && short_strides(a->kv) &&
         (a->topk_extra == 0 || (a->extra.dtype == SMLA_FP8_E4M3_G64 && short_strides(a->extra)));
}

// Split model of the decode form (times in microseconds, fitted to cold HIP-graph timings
// of both forms on MI355X). One index tile on one CU takes t_tile; a workgroup pays one
// tile of start-up (slot ids, then rows, before its first tile) and each work item 0.4 tile
// of output epilogue. Items of at most 8 tiles are walked by one workgroup per CU in rounds
// of `cus` items; longer ones get one workgroup each, so every round pays a start-up. A
// split adds the combine pass: a fixed cost plus the bf16 partials written and read back.
constexpr double kCombineUs = 4.0;
constexpr double kPartialBytesPerUs = 10.0e6;  // partials stay in the 256 MB MALL

double split_cost_us(const smla_args *a, const smla::Variant &v, int64_t base, int n_tiles,
                     int nc, int cus) {
  const double t_tile = v.d_qk == 1088 ? 2.1 : v.hb == 2 ? 2.6 : 2.0;
  const int tpc = ceil_div(n_tiles, nc);
  const int64_t items = base * nc;
  const double rounds = (double)((items + cus - 1) / cus);
  const bool per_item = tpc > 8 && items >= cus;
  double t = per_item ? rounds * (tpc + 1.4) * t_tile : (rounds * (tpc + 0.4) + 1.0) * t_tile;
  if (nc > 1)
    t += kCombineUs + (double)a->T * a->h * nc * a->d_v * 2 * 2 / kPartialBytesPerUs;
  return t;
}

// Test hook: SMLA_TEST_DECODE_KERNEL=wide keeps decode plans on the wide kernels and their
// combine pass, so that the tests reach that split path on the shapes the decode kernel
// would otherwise take. It changes no result beyond rounding.
bool decode16_enabled() {
  const char *v = getenv("SMLA_TEST_DECODE_KERNEL");
  return !(v && strcmp(v, "wide") == 0);
}

// Test hook: SMLA_TEST_PREFILL_KERNEL=wide keeps prefill plans on the wide kernels (the
// fp8qk kernel in the fp8 compute mode), so that the tests reach the wide instances and the
// fp8qk kernel on the shapes the narrow and role-split kernels would take.
bool narrow_enabled() {
  const char *v = getenv("SMLA_TEST_PREFILL_KERNEL");
  return !(v && strcmp(v, "wide") == 0);
}

Plan make_plan(const smla_args *a, bool decode, int cus) {
  Plan pl;
  pl.v = smla::choose_variant(a->d_qk, a->h);
  pl.kind = 0;
  const int all_tiles = ceil_div(a->topk, 64) + ceil_div(a->topk_extra, 64);
  if (!decode && a->T > 0 && a->d_qk == 576 && fp8_only(a) && all_tiles >= 2 &&
      narrow_enabled() && (a->h <= 32 || a->compute_mode == SMLA_COMPUTE_FP8)) {
    // The narrow kernel: 32 heads per work item (fewer heads are padded, so that a head's
    // result does not depend on the head count), every item walks its token's whole list.
    // The fp8 compute mode takes it at every head count (one item per 32 heads).
    pl.kind = 2;
    pl.n_hg = ceil_div(a->h, 32);
    pl.n_chunks = 1;
    pl.tiles_per_chunk = all_tiles;
    pl.ws_bytes = 0;
    return pl;
  }
  if (!decode && a->T > 0 && a->d_qk == 576 && fp8_only(a) && all_tiles >= 1 &&
      narrow_enabled() && a->h > 32 && a->compute_mode != SMLA_COMPUTE_FP8) {
    // The role-split kernel: 64 heads per work item (a last partial group is padded), every
    // item walks its token's whole list.
    pl.kind = 3;
    pl.n_hg = ceil_div(a->h, 64);
    pl.n_chunks = 1;
    pl.tiles_per_chunk = all_tiles;
    pl.ws_bytes = 0;
    return pl;
  }
  if (decode && a->T > 0 && a->d_qk == 576 && fp8_only(a) && decode16_enabled()) {
    // The decode kernel: 16 heads per workgroup, every chunk resident in LDS, so the chunk
    // count is the least that fits (the gathers of an item are all issued at once). It wins
    // while its work items fit one round of workgroups (one per CU); past that the wide
    // kernels' split plan is faster (measured cold over T <= 64, h 16-128, topk 128-2048:
    // at h 128, topk 2048, T 64 the decode kernel's 8 rounds take 251 us, the split plan 90).
    const int n_tiles = ceil_div(a->topk, 64) + ceil_div(a->topk_extra, 64);
    const int nc = ceil_div(n_tiles, smla::kDMaxTiles);
    const int64_t items16 = (int64_t)a->T * ceil_div(a->h, 16) * nc;
    if (nc <= kD16MaxChunks && items16 <= cus) {
      pl.kind = 1;
      pl.n_hg = ceil_div(a->h, 16);
      pl.tiles_per_chunk = ceil_div(n_tiles, nc);
      pl.n_chunks = ceil_div(n_tiles, pl.tiles_per_chunk);
      pl.ws_bytes = 0;
      if (pl.n_chunks > 1) {
        const size_t rows = (size_t)a->T * pl.n_hg * pl.n_chunks * 16;
        pl.ws_bytes = (rows * 512 * sizeof(uint16_t) + 255) / 256 * 256 + rows * 2 * sizeof(float);
      }
      return pl;
    }
  }
  const int hg = pl.v.heads_per_group();
  pl.n_hg = (a->h + hg - 1) / hg;
  const int n_tiles = ceil_div(a->topk, pl.v.tile) + ceil_div(a->topk_extra, pl.v.tile);
  pl.n_chunks = 1;
  if (decode && a->T > 0) {
    // The chunk count with the least modelled time; every distinct chunk length is tried
    // once, and on a tie the fewer chunks win.
    const int64_t base = (int64_t)a->T * pl.n_hg;
    double best = split_cost_us(a, pl.v, base, n_tiles, 1, cus);
    // A split stays within one round of items: measured, splits whose items need several
    // rounds lose to fewer chunks (their partials outgrow what the caches absorb).
    for (int nc = 2; nc <= n_tiles && base * nc <= cus; ++nc) {
      if (ceil_div(n_tiles, ceil_div(n_tiles, nc)) != nc) continue;
      const double c = split_cost_us(a, pl.v, base, n_tiles, nc, cus);
      if (c < best) {
        best = c;
        pl.n_chunks = nc;
      }
    }
  }
  pl.tiles_per_chunk = ceil_div(n_tiles, pl.n_chunks);
  pl.n_chunks = ceil_div(n_tiles, pl.tiles_per_chunk);
  pl.ws_bytes = 0;
  if (pl.n_chunks > 1) {
    const size_t rows = (size_t)a->T * pl.n_chunks * a->h;
    const size_t o_bytes = (rows * a->d_v * sizeof(uint16_t) + 255) / 256 * 256;
    pl.ws_bytes = o_bytes + rows * 2 * sizeof(float);
  }
  return pl;
}

std::mutex g_dev_mu;
int g_dev_ok[64];   // 0 unknown, 1 gfx950, -1 other
int g_dev_cus[64];  // compute units of the device
std::string g_dev_arch[64];

constexpr int kDefaultCUs = 256;  // MI355X

// Reads the current device's properties once. Returns the device number, or -1 (with the
// HIP error in *err) when there is no usable device.
int probe_device(hipError_t *err) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) {
    *err = e == hipSuccess ? hipErrorInvalidDevice : e;
    return -1;
  }
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      *err = e;
      return -1;
    }
    g_dev_arch[dev] = prop.gcnArchName;
    g_dev_cus[dev] = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : kDefaultCUs;
    g_dev_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  return dev;
}

int check_device(int *cus) {
  hipError_t e = hipSuccess;
  const int dev = probe_device(&e);
  if (dev < 0)
    return set_error(SMLA_ERR_DEVICE, "sparse-MLA: no usable HIP device: %s",
                     hipGetErrorString(e));
  if (g_dev_ok[dev] < 0)
    return set_error(SMLA_ERR_DEVICE, "sparse-MLA: device %d is %s; only gfx950 (MI355X) is "
                     "supported", dev, g_dev_arch[dev].c_str());
  *cus = g_dev_cus[dev];
  return SMLA_OK;
}

// Compute units a plan is made for: the current device's, or MI355X's 256 when the call has
// no device (a workspace-size query may run on a host without one). A launch and a size
// query on the same device therefore make the same plan.
int plan_cus() {
  hipError_t e = hipSuccess;
  const int dev = probe_device(&e);
  return dev < 0 ? kDefaultCUs : g_dev_cus[dev];
}

// Test hook: SMLA_TEST_GRID_CAP=n (n >= 1) launches at most n workgroups, so that a small
// input makes each workgroup walk several work items. It changes no result; the parity
// tests use it to reach the multi-item walk of every kernel instance.
int grid_cap() {
  const char *v = getenv("SMLA_TEST_GRID_CAP");
  if (!v || !*v) return 0;
  const int n = atoi(v);
  return n > 0 ? n : 0;
}

// Arrival counters for one call of the decode kernel: n consecutive counters of the current
// device's pool, handed out round-robin. Every call leaves its counters at zero, so a range
// is free again once the call that held it has finished; the pool holds kArrivalSlots, so
// a range comes round again only after hundreds of calls.
std::mutex g_arr_mu;
int64_t g_arr_next[64];

int arrival_range(int64_t n, uint32_t **out) {
  uint32_t *base = nullptr;
  const hipError_t e = smla::arrival_region(&base);
  int dev = 0;
  if (e != hipSuccess || hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return set_error(SMLA_ERR_DEVICE, "sparse-MLA decode: arrival counter lookup failed: %s",
                     hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_arr_mu);
  if (g_arr_next[dev] + n > smla::kArrivalSlots) g_arr_next[dev] = 0;
  *out = base + g_arr_next[dev];
  g_arr_next[dev] += n;
  return SMLA_OK;
}

smla::PoolArgs pool_args(const smla_cache &c, int d_qk) {
  smla::PoolArgs p{};
  p.data = static_cast<const uint8_t *>(c.data);
  p.scales = c.dtype == SMLA_FP8_E4M3_G64 ? static_cast<const uint8_t *>(c.scales) : nullptr;
  p.num_slots = c.num_pages * c.page_block_size;
  p.page_stride = c.page_stride;
  p.row_stride = c.row_stride;
  p.scale_page_stride = c.scale_page_stride;
  p.scale_row_stride = c.scale_row_stride;
  p.fp8 = c.dtype == SMLA_FP8_E4M3_G64;
  p.page_stride32 = (uint32_t)c.page_stride;
  p.row_stride32 = (uint32_t)c.row_stride;
  p.scale_page_stride32 = (uint32_t)c.scale_page_stride;
  p.scale_row_stride32 = (uint32_t)c.scale_row_stride;
  (void)d_qk;
  return p;
}

// The routed entry takes the decode form's split plan for up to kDecodeMaxTokens rows (the
// plan itself keeps a single chunk, i.e. the prefill form, where a split would not pay) and
// the prefill form above that.
bool split_plan(const smla_args *a, int f) {
  if (a->compute_mode == SMLA_COMPUTE_FP8) return false;  // one workgroup per item, no split
  return f == kDecode || (f == kForward && a->T <= kDecodeMaxTokens);
}

int run(const smla_args *a, hipStream_t stream, int f) {
  g_last_error.clear();
  int rc = validate(a, f);
  if (rc) return rc;
  if (a->T == 0) return SMLA_OK;
  const bool decode = split_plan(a, f);
  const Plan pl = make_plan(a, decode, plan_cus());
  if (pl.ws_bytes > 0) {
    if (!a->workspace || a->workspace_bytes < pl.ws_bytes)
      return set_error(SMLA_ERR_WORKSPACE, "%s: workspace of %zu bytes at %p is smaller than the "
                       "%zu bytes sparse_mla_workspace_size() reports", prefix(a, form_name(f)).c_str(),
                       a->workspace_bytes, a->workspace, pl.ws_bytes);
    if (!aligned(a->workspace, 256))
      return set_error(SMLA_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned",
                       prefix(a, form_name(f)).c_str());
  }
  int cus = 0;
  rc = check_device(&cus);
  if (rc) return rc;

  smla::KParams p{};
  p.q = static_cast<const uint16_t *>(a->q);
  p.q_st = a->q_stride_t;
  p.q_sh = a->q_stride_h;
  p.kv = pool_args(a->kv, a->d_qk);
  if (a->topk_extra > 0) p.ex = pool_args(a->extra, a->d_qk);
  p.idx = a->indices;
  p.idx_st = a->indices_stride;
  p.eidx = a->topk_extra > 0 ? a->extra_indices : nullptr;
  p.eidx_st = a->extra_indices_stride;
  p.topk = a->topk;
  p.topk_extra = a->topk_extra;
  p.main_tiles = ceil_div(a->topk, pl.v.tile);
  p.n_tiles = p.main_tiles + ceil_div(a->topk_extra, pl.v.tile);
  p.len = a->topk_length;
  p.elen = a->topk_extra > 0 ? a->extra_topk_length : nullptr;
  p.sink = a->attn_sink;
  p.scale_log2 = a->sm_scale * 1.4426950408889634f;
  p.out = static_cast<uint16_t *>(a->out);
  p.out_st = a->out_stride_t;
  p.out_sh = a->out_stride_h;
  p.lse = a->lse;
  p.lse_st = a->lse_stride_t;
  p.T = a->T;
  p.h = a->h;
  p.n_hg = pl.n_hg;
  p.n_chunks = pl.n_chunks;
  p.tiles_per_chunk = pl.tiles_per_chunk;
  // One workgroup per CU (the LDS tiles fill a CU), each walking items grid apart, so the
  // gather pipeline never drains between items and no item pays a start-up round trip.
  // The items of a token are 8 apart, on blocks of one XCD that start together and walk in
  // step, so its other head groups and chunks find the rows in that XCD's L2.
  const int64_t items = (int64_t)a->T * pl.n_hg * pl.n_chunks;
  p.grid = (int32_t)(items < cus ? items : cus);
  if (const int cap = grid_cap()) p.grid = p.grid < cap ? p.grid : cap;
  if (pl.n_chunks > 1) {
    const size_t rows = (size_t)a->T * pl.n_chunks * a->h;
    const size_t o_bytes = (rows * a->d_v * sizeof(uint16_t) + 255) / 256 * 256;
    p.ws_o = static_cast<uint16_t *>(a->workspace);
    p.ws_ml = reinterpret_cast<float *>(static_cast<char *>(a->workspace) + o_bytes);
  }
  hipError_t e;
  if (pl.kind == 2) {
    e = smla::launch_narrow(p, 32, a->compute_mode == SMLA_COMPUTE_FP8, stream);
  } else if (pl.kind == 3) {
    e = smla::launch_roles(p, stream);
  } else if (pl.kind == 1) {
    // decode kernel: one workgroup per item
    p.grid = (int32_t)items;
    if (pl.n_chunks > 1) {
      const size_t rows = (size_t)a->T * pl.n_hg * pl.n_chunks * 16;
      const size_t o_bytes = (rows * 512 * sizeof(uint16_t) + 255) / 256 * 256;
      p.ws_o = static_cast<uint16_t *>(a->workspace);
      p.ws_ml = reinterpret_cast<float *>(static_cast<char *>(a->workspace) + o_bytes);
      rc = arrival_range((int64_t)a->T * pl.n_hg, &p.arrivals);
      if (rc) return rc;
    }
    e = smla::launch_decode16(p, stream);
  } else if (a->compute_mode == SMLA_COMPUTE_FP8) {
    p.n_hg = ceil_div(a->h, 32);
    p.main_tiles = p.n_tiles = ceil_div(a->topk, 32);
    p.n_chunks = 1;
    e = smla::launch_fp8qk(p, stream);
  } else {
    e = smla::launch_attention(pl.v, p, stream);
    if (e == hipSuccess && pl.n_chunks > 1) e = smla::launch_combine(pl.v, p, stream);
  }
  if (e != hipSuccess)
    return set_error(SMLA_ERR_DEVICE, "sparse-MLA %s: kernel launch failed: %s",
                     form_name(f), hipGetErrorString(e));
  return SMLA_OK;
}

}  // namespace

extern "C" {

int sparse_mla_prefill(const smla_args *args, hipStream_t stream) {
  return run(args, stream, kPrefill);
}

int sparse_mla_decode(const smla_args *args, hipStream_t stream) {
  return run(args, stream, kDecode);
}

int sparse_mla_forward(const smla_args *args, hipStream_t stream) {
  return run(args, stream, kForward);
}

int sparse_mla_decode_noalloc(const smla_args *args, hipStream_t stream) {
  g_last_error.clear();
  int rc = validate(args, kDecode);
  if (rc) return rc;
  if (args->T == 0) return SMLA_OK;
  const size_t need = make_plan(args, true, plan_cus()).ws_bytes;
  if (need > smla::kScratchBytes)
    return set_error(SMLA_ERR_WORKSPACE, "%s: the plan needs %zu bytes of split-K scratch, more "
                     "than the %zu bytes that sparse_mla_decode_noalloc holds per device (use "
                     "sparse_mla_decode with a workspace)", prefix(args, "decode").c_str(), need,
                     smla::kScratchBytes);
  int cus = 0;
  rc = check_device(&cus);
  if (rc) return rc;
  smla_args a = *args;
  a.workspace = nullptr;
  a.workspace_bytes = 0;
  if (need > 0) {
    const hipError_t e = smla::scratch_region(&a.workspace);
    if (e != hipSuccess)
      return set_error(SMLA_ERR_DEVICE, "sparse-MLA decode_noalloc: scratch lookup failed: %s",
                       hipGetErrorString(e));
    a.workspace_bytes = smla::kScratchBytes;
  }
  return run(&a, stream, kDecode);
}

int sparse_mla_workspace_size(const smla_args *args, int form, size_t *bytes) {
  g_last_error.clear();
  if (!bytes) return set_error(SMLA_ERR_INVALID, "sparse-MLA: bytes is NULL");
  if (form < kPrefill || form > kForward)
    return set_error(SMLA_ERR_INVALID, "sparse-MLA: form=%d is not 0 (prefill), 1 (decode) or "
                     "2 (forward)", form);
  const int rc = validate(args, form);
  if (rc) return rc;
  *bytes = args->T == 0 ? 0 : make_plan(args, split_plan(args, form), plan_cus()).ws_bytes;
  return SMLA_OK;
}

int sparse_mla_supported_configs(smla_config *out, int capacity, int *count) {
  g_last_error.clear();
  static const int geo[2][2] = {{576, 512}, {1088, 1024}};
  static const int extra[3] = {-1, SMLA_BF16, SMLA_FP8_E4M3_G64};
  const int total = 2 * 2 * 3;
  if (!count) return set_error(SMLA_ERR_INVALID, "sparse-MLA: count is NULL");
  if (capacity < 0 || (capacity > 0 && !out))
    return set_error(SMLA_ERR_INVALID, "sparse-MLA: out is NULL with capacity=%d", capacity);
  int n = 0;
  for (int gi = 0; gi < 2; ++gi)
    for (int kd = 0; kd < 2; ++kd)
      for (int ex = 0; ex < 3; ++ex) {
        if (n < capacity) {
          smla_config &c = out[n];
          c.d_qk = geo[gi][0];
          c.d_v = geo[gi][1];
          c.kv_dtype = kd;
          c.extra_kv_dtype = extra[ex];
          c.min_h = 1;
          c.max_h = kMaxHeads;
          c.topk_multiple = kTopkMultiple;
          c.page_block_size = kPageBlock;
          c.decode_max_tokens = kDecodeMaxTokens;
        }
        ++n;
      }
  *count = total;
  return SMLA_OK;
}

int sparse_mla_pack_kv(const smla_pack_args *a, hipStream_t stream) {
  g_last_error.clear();
  if (!a) return set_error(SMLA_ERR_INVALID, "sparse-MLA pack: args is NULL");
  char buf[160];
  snprintf(buf, sizeof(buf), "sparse-MLA pack (n=%lld d_qk=%d)", (long long)a->n, a->d_qk);
  const std::string pre = buf;
  if (a->n < 0) return set_error(SMLA_ERR_INVALID, "%s: n is negative", pre.c_str());
  if (a->d_qk != 576 && a->d_qk != 1088)
    return set_error(SMLA_ERR_UNSUPPORTED, "%s: d_qk=%d is not supported (supported: 576, 1088)",
                     pre.c_str(), a->d_qk);
  if (a->kv.dtype != SMLA_FP8_E4M3_G64)
    return set_error(SMLA_ERR_UNSUPPORTED, "%s: kv dtype=%d; packing writes fp8 pools only "
                     "(dtype 1, e4m3 + fp32 scale per 64)", pre.c_str(), a->kv.dtype);
  if (a->n == 0) return SMLA_OK;
  int rc = check_cache(a->d_qk, a->kv, "kv", pre);
  if (rc) return rc;
  if (!a->rows || !aligned(a->rows, 16) || a->rows_stride < a->d_qk || a->rows_stride % 8)
    return set_error(SMLA_ERR_INVALID, "%s: rows must be non-NULL and 16-byte aligned, with "
                     "rows_stride=%lld a multiple of 8 and >= d_qk", pre.c_str(),
                     (long long)a->rows_stride);
  if (!a->slots || !aligned(a->slots, 4))
    return set_error(SMLA_ERR_INVALID, "%s: slots must be non-NULL and 4-byte aligned",
                     pre.c_str());
  const int64_t blocks = (a->n * (a->d_qk / 8) + 255) / 256;
  if (blocks > INT32_MAX)
    return set_error(SMLA_ERR_UNSUPPORTED, "%s: too many rows for one launch", pre.c_str());
  int cus = 0;
  rc = check_device(&cus);
  if (rc) return rc;
  smla::PackParams p{};
  p.rows = static_cast<const uint16_t *>(a->rows);
  p.rows_st = a->rows_stride;
  p.slots = a->slots;
  p.n = a->n;
  p.d_qk = a->d_qk;
  p.kv = pool_args(a->kv, a->d_qk);
  p.kv_data = static_cast<uint8_t *>(const_cast<void *>(a->kv.data));
  p.kv_scales = static_cast<uint8_t *>(const_cast<void *>(a->kv.scales));
  const hipError_t e = smla::launch_pack(p, stream);
  if (e != hipSuccess)
    return set_error(SMLA_ERR_DEVICE, "%s: kernel launch failed: %s", pre.c_str(),
                     hipGetErrorString(e));
  return SMLA_OK;
}

const char *sparse_mla_last_error(void) { return g_last_error.c_str(); }

int sparse_mla_abi_version(void) { return SMLA_ABI_VERSION; }

}  // extern "C"
