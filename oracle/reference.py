"""Plain CPU oracle for sparse top-k MLA attention over a paged latent KV pool.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this module. The GPU library never calls it and shares no code with it.

What it computes. The pages build their decoding steps on these facts:

* "[SM12x] Drop the 64-head TP pad on the DSv4 MLA prefill path" (sglang PR 35104),
  section Problem: all query heads of a token share one latent KV head (MLA keeps a
  single KV head), and prefill cost scales with the head count.
* The same page, section "Correctness - what is and is not established": attention is
  independent per (token, head). It also checks that the sink has one entry per head.
* "fix(sparse-mla-sm120): add topk=256 prefill-dsv4 dispatch" (FlashInfer PR 3896),
  sections Description and Change: a call carries num_heads, topk, a page block size of
  64, and an optional extra cache (topk_extra, extra_page_block_size). topk=256 is
  4 x BI(64) index tiles. The tests run with_sink on and off.
* The FlashInfer 4802 merge message embedded in "fix(sm120): explain sparse-MLA decode
  dispatch misses; add config query API" (PR 4551):
  - section Summary: sinks, an optional out_lse, dual-cache joins, row-strided indices;
  - section swapAB prefill: both scale formats;
  - section Compatibility: inline-scale and footer-scale KV byte formats.

The arithmetic is the plain definition of attention with a sink logit, where the pages
leave it open.

For token t, the list J_t holds every entry j < L_t of the token's index row whose slot
s satisfies 0 <= s < num_slots (-1 marks an invalid entry). L_t is topk, or, when a
per-row count topk_length is given, topk_length[t] clamped to [0, topk]: the 4802
message (sections swapAB prefill and Test plan) names a variable topk_length that
truncates a row. topk itself is any positive width, a multiple of 64 or not (section
Runtime envelopes: decode serves ragged widths such as 500). With an extra cache, the
extra list's valid entries (up to its own optional count) are appended to J_t. Each entry's row r_j is decoded from the
pool:
    page = s // page_block_size, offset = s % page_block_size;
    bf16 rows are taken exactly;
    fp8 rows: r_j[d] = e4m3fn(byte[d]) * scale[d // 64].
For each head:
    z_j = sm_scale * sum_d q[t,h,d] * r_j[d]
    m   = max({z_j} U {sink_h})              (sink_h = -inf when no sink is given)
    D   = sum_j exp(z_j - m) + exp(sink_h - m)
    o   = sum_j exp(z_j - m) * r_j[:d_v] / D
    lse = m + ln D.
An empty list with no sink gives o = 0 and lse = -inf.

Everything is computed in float64 on the exactly decoded inputs.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

GROUP = 64  # fp8 scale group width


# --------------------------------------------------------------------------- decoders
def e4m3fn_value(code: int) -> float:
    """OCP FP8 E4M3 ("fn": no infinities) from its definition.

    The format has 1 sign bit, 4 exponent bits with bias 7 and 3 mantissa bits.
    Exponent field 0 holds the subnormals m/8 * 2^-6. S.1111.111 is NaN; every other
    code is finite, so the largest value is 1.75 * 2^8 = 448.
    """
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def e4m3fn_table() -> np.ndarray:
    return _E4M3_TABLE.copy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float64.

    A bf16 value is the float32 whose upper 16 bits are the pattern and whose lower
    16 bits are zero.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------- gather
def _scale_group(d: np.ndarray) -> np.ndarray:
    """Scale group of element d: one fp32 scale covers 64 consecutive elements."""
    return d // GROUP


def _slot_location(pool, slot: np.ndarray):
    """(page, offset-in-page) of physical slot ids."""
    return slot // pool.page_block_size, slot % pool.page_block_size


def valid_mask(pool, slots: np.ndarray) -> np.ndarray:
    """An entry is used iff 0 <= slot < num_pages * page_block_size."""
    s = np.asarray(slots, dtype=np.int64)
    return (s >= 0) & (s < pool.num_pages * pool.page_block_size)


def decode_rows(pool, slots: np.ndarray) -> np.ndarray:
    """Decode the latent rows of valid slot ids to float64 [n, d_qk]."""
    s = np.asarray(slots, dtype=np.int64)
    page, off = _slot_location(pool, s)
    d = np.arange(pool.d_qk)
    start = pool.data_offset + page * pool.page_stride + off * pool.row_stride
    if pool.dtype == "bf16":
        lo = pool.data[start[:, None] + 2 * d[None, :]].astype(np.uint16)
        hi = pool.data[start[:, None] + 2 * d[None, :] + 1].astype(np.uint16)
        return bf16_to_f64(lo | (hi << 8))
    if pool.dtype != "fp8":
        raise ValueError(pool.dtype)
    codes = pool.data[start[:, None] + d[None, :]]
    vals = _E4M3_TABLE[codes]
    groups = pool.d_qk // GROUP
    sstart = pool.scale_offset + page * pool.scale_page_stride + off * pool.scale_row_stride
    sb = pool.scales[sstart[:, None] + np.arange(4 * groups)[None, :]]
    scales = np.ascontiguousarray(sb).view("<f4").reshape(len(s), groups).astype(np.float64)
    return vals * scales[:, _scale_group(d)]


def live_entries(row, lengths, t: int) -> np.ndarray:
    """The first L_t entries of an index row (all of them when no per-row count is given)."""
    row = np.asarray(row, dtype=np.int64)
    if lengths is None:
        return row
    n = min(max(int(lengths[t]), 0), row.shape[0])
    return row[:n]


def gather_token(p, t: int) -> np.ndarray:
    """Rows of J_t (main entries, then extra entries; order and repeats kept)."""
    parts = []
    idx = live_entries(p.indices[t], getattr(p, "topk_length", None), t)
    parts.append(decode_rows(p.kv, idx[valid_mask(p.kv, idx)]))
    if p.extra is not None and p.extra_indices is not None and p.extra_indices.shape[1]:
        eidx = live_entries(p.extra_indices[t], getattr(p, "extra_topk_length", None), t)
        parts.append(decode_rows(p.extra, eidx[valid_mask(p.extra, eidx)]))
    return np.concatenate(parts, axis=0)


# --------------------------------------------------------------------------- attention
def _value_part(rows: np.ndarray, d_v: int) -> np.ndarray:
    """V is the first d_v elements of each latent row."""
    return rows[:, :d_v]


def attend(q: np.ndarray, rows: np.ndarray, sink: np.ndarray, sm_scale: float, d_v: int):
    """Softmax attention of h query rows over n shared rows, with one sink logit per head.

    q [h, d_qk], rows [n, d_qk], sink [h] (-inf for none). Returns (o [h, d_v], lse [h]).
    """
    h = q.shape[0]
    n = rows.shape[0]
    z = sm_scale * (q @ rows.T) if n else np.zeros((h, 0))
    zmax = z.max(axis=1) if n else np.full(h, -np.inf)
    m = np.maximum(zmax, sink)
    o = np.zeros((h, d_v))
    lse = np.full(h, -np.inf)
    live = np.isfinite(m)
    if not live.any():
        return o, lse
    ml = m[live]
    e = np.exp(z[live] - ml[:, None])
    denom = e.sum(axis=1) + np.exp(sink[live] - ml)
    o[live] = (e @ _value_part(rows, d_v)) / denom[:, None]
    lse[live] = ml + np.log(denom)
    return o, lse


def sparse_mla_reference(p, tokens: Optional[np.ndarray] = None):
    """The oracle: (o float64 [n_tok, h, d_v], lse float64 [n_tok, h]).

    ``p`` carries q_bits (bf16 patterns [T, h, d_qk]), kv / extra pools, indices /
    extra_indices (int32), attn_sink (float32 [h] or None), sm_scale and d_v.
    ``tokens`` restricts the computation to those token rows (default: all).
    """
    toks = np.arange(p.T) if tokens is None else np.asarray(tokens)
    sink = (np.full(p.h, -np.inf) if p.attn_sink is None
            else np.asarray(p.attn_sink, dtype=np.float64))
    o = np.zeros((len(toks), p.h, p.d_v))
    lse = np.zeros((len(toks), p.h))
    for i, t in enumerate(toks):
        q = bf16_to_f64(p.q_bits[t])
        o[i], lse[i] = attend(q, gather_token(p, int(t)), sink, float(p.sm_scale), p.d_v)
    return o, lse


# The problem a parallel call works on, set before its worker processes are forked so that
# each worker inherits it instead of receiving a pickled copy (a large prefill's q alone is
# hundreds of MB).
_PAR_PROBLEM = None


def _worker(toks):
    p = _PAR_PROBLEM
    try:  # one BLAS thread per worker process
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            return sparse_mla_reference(p, toks)
    except ImportError:
        return sparse_mla_reference(p, toks)


def sparse_mla_reference_parallel(p, tokens: Optional[np.ndarray] = None, workers: int = 0):
    """Same result as sparse_mla_reference, computed over token blocks in worker processes.

    The token list is cut into `workers` contiguous blocks (np.array_split: sizes differ by
    at most one); each worker runs the same per-token function with one BLAS thread, and the
    blocks' rows are concatenated in order, so row i of the result is token tokens[i].
    Returns (o, lse, workers_used).
    """
    import concurrent.futures as cf
    import multiprocessing as mp
    import os

    global _PAR_PROBLEM
    toks = np.arange(p.T) if tokens is None else np.asarray(tokens)
    n = workers or os.cpu_count() or 1
    n = max(1, min(n, len(toks)))
    if n == 1:
        o, lse = sparse_mla_reference(p, toks)
        return o, lse, 1
    blocks = np.array_split(toks, n)
    _PAR_PROBLEM = p
    try:
        with cf.ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("fork")) as ex:
            res = list(ex.map(_worker, blocks))
    finally:
        _PAR_PROBLEM = None
    return (np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res]), n)
