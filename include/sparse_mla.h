/*
 * sparse_mla.h - C ABI of libsparse_mla: sparse top-k MLA attention over a paged latent KV
 * pool, for AMD MI355X (gfx950).
 *
 * The operation. One call serves T query tokens. All h heads of a token share one latent
 * KV head (MLA keeps a single KV head):
 *   - "[SM12x] Drop the 64-head TP pad on the DSv4 MLA prefill path", section Problem;
 *   - the same page, section "Correctness - what is and is not established": attention
 *     is independent per (token, head), and attn_sink has one entry per head.
 *
 * For token t:
 *   - The token gathers the latent rows whose slot ids appear in indices[t, 0:L_t].
 *     L_t is topk, or min(max(topk_length[t], 0), topk) when a per-row count is given.
 *     With an extra cache, it also gathers extra_indices[t, 0:L'_t] from that pool (L'_t
 *     likewise from topk_extra and extra_topk_length).
 *     A call carries num_heads, topk, page_block_size, topk_extra and
 *     extra_page_block_size ("fix(sparse-mla-sm120): add topk=256 prefill-dsv4 dispatch",
 *     sections Description and Change).
 *   - A slot id s < 0 (-1 by convention) or s >= num_pages * page_block_size marks an
 *     unused entry.
 *   - Rows are stored as bf16, or as fp8 e4m3fn with one fp32 scale per 64 elements.
 *     The FlashInfer 4802 merge message embedded in "fix(sm120): explain sparse-MLA
 *     decode dispatch misses; add config query API" names the scale formats in sections
 *     "swapAB prefill" and Compatibility. Any byte layout a strided descriptor reaches is
 *     accepted: scales inline after the payload, in a page footer, or in their own buffer.
 *   - For each head:
 *       z_j = sm_scale * <q[t,h,:], row_j>                   over d_qk elements
 *       m   = max(max_j z_j, attn_sink[h])
 *       D   = sum_j exp(z_j - m) + exp(attn_sink[h] - m)
 *       out[t,h,:] = sum_j exp(z_j - m) * row_j[0:d_v] / D   (V = the first d_v elements)
 *       lse[t,h]   = m + ln D                                (optional output)
 *   - A token with no used entry and no sink gets out = 0 and lse = -inf.
 *   - The 4802 message also gives the rest of the call surface:
 *       . optional out_lse and row-strided indices / out_lse (section Summary);
 *       . a T = 0 call is a no-op (section Summary);
 *       . any head count in [1, 128] (section "Runtime envelopes");
 *       . ragged widths: the same section has decode serve topk = 500, a width with a
 *         partial last 64-wide index tile. Here both forms serve any topk >= 1 and any
 *         topk_extra >= 0;
 *       . a variable per-row topk_length that truncates a row (sections "swapAB prefill"
 *         and "Test plan");
 *       . caller-owned split-K scratch for the decode form (section "Runner and CUDA
 *         graphs").
 *
 * Ownership and threading.
 *   - The caller allocates every buffer.
 *   - The library never allocates or frees device memory, never synchronises, and keeps no
 *     pointer after a call returns. All work is enqueued on the given stream.
 *   - out, lse and workspace must not alias any input.
 *   - Calls are thread-safe. Error text is per thread.
 *
 * Errors.
 *   - Every host-checkable condition is validated before any HIP call. On failure, a call
 *     returns a non-zero status, enqueues nothing and leaves the outputs untouched.
 *     sparse_mla_last_error() then names the mismatch and lists the supported values.
 *   - Slot values live on the device and are not checked on the host. The kernels treat
 *     out-of-range slots as unused and never dereference them.
 */
#ifndef SPARSE_MLA_H
#define SPARSE_MLA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SMLA_ABI_VERSION 2

/* KV row encodings. */
enum {
  SMLA_BF16 = 0,        /* d_qk bf16 values per row                                        */
  SMLA_FP8_E4M3_G64 = 1 /* d_qk OCP e4m3fn bytes per row + d_qk/64 fp32 scales (one per 64) */
};

/* Compute modes (smla_args.compute_mode). */
enum { SMLA_COMPUTE_BF16 = 0, SMLA_COMPUTE_FP8 = 1 };

/* Status codes. */
enum {
  SMLA_OK = 0,
  SMLA_ERR_INVALID = 1,     /* a null pointer, a bad stride or size, an inconsistent argument */
  SMLA_ERR_UNSUPPORTED = 2, /* valid but outside the supported envelope (head count, topk...) */
  SMLA_ERR_WORKSPACE = 3,   /* decode: workspace missing or smaller than required           */
  SMLA_ERR_DEVICE = 4       /* HIP error, or the current device is not gfx950                */
};

/*
 * One paged latent KV pool in device memory (caller-owned, read-only).
 *   Slot s lives in page s / page_block_size at offset o = s % page_block_size.
 *   Its payload starts at  data   + page * page_stride       + o * row_stride        (bytes)
 *   and its scales start at scales + page * scale_page_stride + o * scale_row_stride  (bytes).
 *
 * Requirements:
 *   - data, page_stride and row_stride are multiples of 16 bytes;
 *   - for fp8, scales and the scale strides are multiples of 4 bytes;
 *   - page_block_size is 64;
 *   - page_stride >= 64 * row_stride, and the payload fits in a row
 *     (row_stride >= d_qk * element size);
 *   - num_pages >= 1.
 * A pool with 0 used entries still needs a valid descriptor.
 */
typedef struct {
  const void *data;
  const void *scales; /* fp8 only; ignored (may be NULL) for bf16 */
  int32_t dtype;      /* SMLA_BF16 or SMLA_FP8_E4M3_G64           */
  int32_t page_block_size;
  int64_t num_pages;
  int64_t page_stride, row_stride;             /* bytes */
  int64_t scale_page_stride, scale_row_stride; /* bytes */
} smla_cache;

typedef struct {
  int32_t T;    /* query tokens, >= 0                          */
  int32_t h;    /* heads, in [1, 128]                          */
  int32_t d_qk; /* 576 or 1088                                 */
  int32_t d_v;  /* 512 (d_qk 576) or 1024 (d_qk 1088)          */

  /* q: bf16 [T, h, d_qk] with strides in elements; the last dimension is dense.
     q_stride_t and q_stride_h are multiples of 8, and q is 16-byte aligned. */
  const void *q;
  int64_t q_stride_t, q_stride_h;

  /* Main cache: indices int32 [T, topk] with a row stride in elements (>= topk).
     topk is any positive width; only entries [0, topk) of a row are read. */
  smla_cache kv;
  const int32_t *indices;
  int32_t topk;
  int64_t indices_stride;

  /* Optional extra cache, joined into the same softmax. topk_extra = 0 means none; then
     extra, extra_indices and extra_topk_length are ignored. Otherwise the extra pool has
     the same d_qk (its dtype may differ from the main pool's). */
  smla_cache extra;
  const int32_t *extra_indices;
  int32_t topk_extra;
  int64_t extra_indices_stride;

  const float *attn_sink; /* fp32 [h] natural-log logits, or NULL for no sink (-inf) */
  float sm_scale;         /* finite and > 0; the usual value is 1/sqrt(d_qk)          */

  /* out: bf16 [T, h, d_v], strides in elements, last dimension dense. out_stride_t and
     out_stride_h are multiples of 4, and out is 8-byte aligned. */
  void *out;
  int64_t out_stride_t, out_stride_h;

  /* lse: optional fp32 [T, h], natural log, row stride in elements (>= h); NULL = none. */
  float *lse;
  int64_t lse_stride_t;

  /* Device scratch for the decode form's split-K partials. Its size comes from
     sparse_mla_workspace_size(); prefill needs none. 256-byte aligned. */
  void *workspace;
  size_t workspace_bytes;

  /* Optional per-row live counts, int32 [T] dense device arrays, 4-byte aligned; NULL means
     every entry of a row is live. Entry j of token t's main row takes part only when
     j < topk_length[t]; a count below 0 acts as 0 and one above topk as topk.
     extra_topk_length does the same for the extra row (ignored when topk_extra is 0). */
  const int32_t *topk_length;
  const int32_t *extra_topk_length;

  /* Compute mode. 0 (SMLA_COMPUTE_BF16): rows are dequantised to bf16 and both products run
     on bf16 MFMA. 1 (SMLA_COMPUTE_FP8): q is quantised per (token, head) to e4m3fn (scale
     amax / 448, multiplier 448 / amax) and QK runs on fp8 MFMA over the raw pool payload, one
     64-wide scale group at a time; P and PV stay bf16. The fp8 mode serves d_qk 576 over an
     fp8 main pool with no extra cache, in the prefill and routed forms (the decode form
     returns SMLA_ERR_UNSUPPORTED). "fix(sparse-mla-sm120): add topk=256 prefill-dsv4
     dispatch" forks prefill on this mode (FP8 / BF16), and the 4802 message ("Performance vs
     main") names the q quantisation step.
     Accuracy: mode 1 is an approximation of the operation above, not the operation. The
     rounding of q moves a logit by up to about 2^-4 of |q||row| and is not averaged away
     when a row has few live entries: against the exact result, rows with 2048 entries stay
     within max 2e-2 / mean 2e-3 of the output, while rows with a few entries miss that bound
     (max up to 5e-2, mean up to 7e-3 measured). It is also slower than mode 0 on MI355X, so
     mode 0 is the default and the one to use when the exact result is wanted. */
  int32_t compute_mode;
} smla_args;

/* One supported envelope, as reported by sparse_mla_supported_configs(). */
typedef struct {
  int32_t d_qk, d_v;
  int32_t kv_dtype;        /* SMLA_BF16 or SMLA_FP8_E4M3_G64                        */
  int32_t extra_kv_dtype;  /* -1 = no extra cache, else a dtype                       */
  int32_t min_h, max_h;    /* 1, 128                                                  */
  int32_t topk_multiple;   /* 1: any topk >= 1 and topk_extra >= 0 (ragged tail masked)   */
  int32_t page_block_size; /* 64                                                      */
  int32_t decode_max_tokens; /* 64: sparse_mla_decode serves T <= this                */
} smla_config;

/*
 * Prefill form: any T >= 0. Work is split per (token, head group), and each workgroup
 * walks all of its token's index tiles.
 * The FlashInfer 4802 message ("Runtime envelopes") has prefill serve any T; its topk
 * rule is widened here to ragged widths, as its decode has. It needs no workspace.
 */
int sparse_mla_prefill(const smla_args *args, hipStream_t stream);

/*
 * Decode form: T <= 64 (larger T returns SMLA_ERR_UNSUPPORTED). Work is also split over
 * index chunks of one token, and a combine pass merges the partial softmax states
 * through the caller's workspace.
 * sglang's "[SM12x] Drop the 64-head TP pad ..." page (section Problem) gives decode as
 * the few-row, KV-bandwidth-bound regime. The row fork at 64 is its section Fix; the
 * split-K scratch is "Runner and CUDA graphs" of the 4802 message.
 * It computes the same function as sparse_mla_prefill.
 */
int sparse_mla_decode(const smla_args *args, hipStream_t stream);

/*
 * Decode form without allocation, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). It computes what
 * sparse_mla_decode computes, with the same plan and kernels, but ignores args->workspace:
 * the split-K partials go to a scratch array of 32 MiB (33554432 bytes) that the library
 * holds on each device it runs on until the process ends. A plan that needs more returns
 * SMLA_ERR_WORKSPACE (on MI355X, 256 CUs, no decode plan does: its partials stay under 17
 * MB). The call allocates nothing and synchronises nothing. Every call on one device
 * shares that device's scratch: calls whose kernels overlap in time on one device (two
 * streams, or two threads) race and give wrong results; calls ordered on one stream do not.
 * The scratch needs no clearing: every call writes all the partials it reads.
 */
int sparse_mla_decode_noalloc(const smla_args *args, hipStream_t stream);

/*
 * Routed form: one entry for any T. Up to decode_max_tokens (64) rows it takes the decode
 * form's plan, whose split model (a makespan over the CUs, with a start-up and a combine
 * cost per split) keeps a single chunk, which is the prefill form, when a split does not
 * pay. Above 64 rows it is the prefill form. It computes the same function as the other
 * two, and needs the workspace that sparse_mla_workspace_size(args, 2, ...) reports (0
 * when it does not split).
 * The 4802 message (section "Dispatch: cpb model + crossover") routes each call between
 * the decode and the prefill kernels by a split model and a measured crossover
 * (decode_max_tokens); its section "Plan layer" keeps that policy in one planner.
 */
int sparse_mla_forward(const smla_args *args, hipStream_t stream);

/*
 * Bytes of workspace that a form needs for these arguments: form 0 = sparse_mla_prefill
 * (always 0), 1 = sparse_mla_decode, 2 = sparse_mla_forward. The args are validated as the
 * matching entry point validates them, except the workspace fields. Another form value
 * returns SMLA_ERR_INVALID.
 * The 4802 message, section "Runner and CUDA graphs", has the caller own the split-K
 * scratch of the decode kernels (so that a captured graph keeps it alive), which needs a
 * query for its size: this is that query. *bytes is written only on SMLA_OK.
 */
int sparse_mla_workspace_size(const smla_args *args, int form, size_t *bytes);

/*
 * Report the supported envelopes. The FlashInfer 4551 page's description adds a config
 * query API; the 4802 message, section "Runtime envelopes", exposes envelopes rather
 * than pairs.
 * Up to `capacity` entries are written to `out` (which may be NULL when capacity is 0).
 * *count receives the total number available.
 */
int sparse_mla_supported_configs(smla_config *out, int capacity, int *count);

/*
 * Packing: write bf16 latent rows into an fp8 pool (SMLA_FP8_E4M3_G64), the step before the
 * attention path. "fix(sparse-mla-sm120): add topk=256 prefill-dsv4 dispatch" packs its KV
 * input with quantize_kv_dsv4 (comment thread, compute-mode comparison); the 4802 message
 * (sections Summary and Compatibility) gives the inline and footer scale placements. The
 * pages print no formula; the reading taken: for each group of 64 consecutive elements
 * with largest magnitude amax,
 *   scale = fl32(amax / 448) (IEEE fp32 division; 0 for an all-zero group),
 *   m     = min(fl32(448 / amax), FLT_MAX) (one division per group, not per element),
 *   code  = the e4m3fn value nearest to clamp(fl32(x * m), -448, 448) (ties to even; a zero
 *           keeps its sign),
 * so that the group's largest magnitude maps onto e4m3fn's largest finite value, and a
 * reader decodes code * scale.
 *   rows:        bf16 [n, d_qk] device memory, 16-byte aligned, row stride rows_stride
 *                elements (a multiple of 8, >= d_qk);
 *   slots:       int32 [n] device memory: the slot row r is written to. A slot outside
 *                [0, num_pages * 64) skips its row. Valid slots must be distinct (two rows
 *                aimed at one slot race);
 *   kv:          the destination pool descriptor, dtype SMLA_FP8_E4M3_G64, same rules as
 *                for the attention calls. Only the payload bytes [0, d_qk) and the d_qk / 64
 *                scales of each written slot change.
 * rows and slots must not overlap the pool. n = 0 is a no-op. Errors as for the attention
 * calls: validated on the host before any HIP call.
 */
typedef struct {
  int64_t n;
  int32_t d_qk; /* 576 or 1088 */
  const void *rows;
  int64_t rows_stride;
  const int32_t *slots;
  smla_cache kv;
} smla_pack_args;

int sparse_mla_pack_kv(const smla_pack_args *args, hipStream_t stream);

/*
 * Text of this thread's last error ("" if none). Valid until the next call on the thread;
 * the library owns the string. The text starts with the fixed prefix that
 * "fix(sparse-mla-sm120): add topk=256 prefill-dsv4 dispatch" (section Description) prints
 * for an unsupported call ("Unsupported sparse-MLA <form> configuration: num_heads=...
 * topk=... page_block_size=... topk_extra=... extra_page_block_size=..."), then names the
 * parameter that missed and lists the supported values, as the description of
 * "fix(sm120): explain sparse-MLA decode dispatch misses; add config query API" asks.
 */
const char *sparse_mla_last_error(void);

/*
 * SMLA_ABI_VERSION of the built library, so that a caller can check that the header it was
 * compiled against describes the structs the library reads. No passage of the pages defines
 * this call: it belongs to this C ABI, not to the method.
 */
int sparse_mla_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPARSE_MLA_H */
