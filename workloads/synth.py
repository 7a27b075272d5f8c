"""Seeded synthetic inputs for sparse top-k MLA attention over a paged latent KV pool.

This module only draws random numbers and lays bytes out in memory. It holds none of the
attention arithmetic: no gather, no dequantisation, no softmax. Both the CPU oracle (in
``oracle/``) and the GPU path read what it produces, each with its own decoder.

What is drawn (the workloads the pages describe, with the sizes of the five benchmark
workloads below):

* q is N(0,1) fp32 rounded to bf16 (round-to-nearest-even, by torch's cast).
* bf16 latent rows are N(0,1) rounded to bf16.
* fp8 latent rows: x ~ N(0,1) and one fp32 scale s = 2**U(-4, 4) per 64-element group;
  the stored byte is e4m3fn(clamp(x / s, +-448)) (torch's round-to-nearest-even cast), so
  the dequantised value byte * s is close to N(0,1).
* attn_sink is N(0,1) fp32, one logit per head.
* indices are distinct slot ids per query token, drawn uniformly from the token's range;
  -1 marks an invalid entry.

A pool is one or two byte buffers plus a descriptor (page stride, row stride, scale
strides), the same numbers the C ABI takes. Three byte layouts are produced for fp8
pools: ``inline`` (scales right after each row's payload, rows padded to 64 B),
``footer`` (each page holds its 64 payload rows, then the 64 rows' scales) and
``separate`` (scales in their own buffer). bf16 pools are dense rows, optionally padded.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

PAGE_BLOCK_SIZE = 64
GROUP = 64  # elements per fp8 scale group
E4M3_MAX = 448.0


def _round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


@dataclasses.dataclass
class Pool:
    """One paged latent KV pool: bytes plus the descriptor numbers the C ABI takes.

    ``data`` and ``scales`` are uint8 numpy buffers (``scales`` may be the same object as
    ``data``). Slot s lives in page s // page_block_size at offset s % page_block_size;
    its payload starts at ``data_offset + page*page_stride + off*row_stride`` and its
    fp32 scales at ``scale_offset + page*scale_page_stride + off*scale_row_stride`` in
    ``scales``.
    """

    dtype: str  # "bf16" or "fp8"
    d_qk: int
    page_block_size: int
    num_pages: int
    data: np.ndarray
    data_offset: int
    page_stride: int
    row_stride: int
    scales: Optional[np.ndarray] = None
    scale_offset: int = 0
    scale_page_stride: int = 0
    scale_row_stride: int = 0
    layout: str = "dense"

    @property
    def num_slots(self) -> int:
        return self.num_pages * self.page_block_size

    @property
    def payload_bytes(self) -> int:
        return self.d_qk * (2 if self.dtype == "bf16" else 1)


@dataclasses.dataclass
class Problem:
    """One call's inputs. Arrays are numpy; q is bf16 bit patterns (uint16)."""

    name: str
    T: int
    h: int
    d_qk: int
    d_v: int
    q_bits: np.ndarray  # uint16 [T, h, d_qk]
    kv: Pool
    indices: np.ndarray  # int32 [T, topk]
    sm_scale: float
    attn_sink: Optional[np.ndarray] = None  # float32 [h]
    extra: Optional[Pool] = None
    extra_indices: Optional[np.ndarray] = None  # int32 [T, topk_extra]
    topk_length: Optional[np.ndarray] = None  # int32 [T]: live main entries per row
    extra_topk_length: Optional[np.ndarray] = None  # int32 [T]: live extra entries per row

    @property
    def topk(self) -> int:
        return int(self.indices.shape[1])

    @property
    def topk_extra(self) -> int:
        return 0 if self.extra_indices is None else int(self.extra_indices.shape[1])


# --------------------------------------------------------------------------- encoders
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even, via torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_e4m3_bytes(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3fn bytes, round-to-nearest-even with saturation at +-448."""
    x = np.clip(np.asarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def draw_scales(rng: np.random.Generator, n: int, groups: int) -> np.ndarray:
    """Per-group fp32 scales, log-uniform in [2^-4, 2^4]."""
    return np.exp2(rng.uniform(-4.0, 4.0, size=(n, groups))).astype(np.float32)


# --------------------------------------------------------------------------- pools
def pack_pool(
    payload: np.ndarray,
    scales: Optional[np.ndarray],
    dtype: str,
    d_qk: int,
    layout: str = "inline",
    page_block_size: int = PAGE_BLOCK_SIZE,
    row_pad: int = 0,
    page_pad: int = 0,
) -> Pool:
    """Lay encoded rows out as a paged pool.

    payload: uint8 [slots, payload_bytes] (bf16 rows are given as their bytes);
    scales: float32 [slots, d_qk/64] for fp8, else None.
    """
    slots = payload.shape[0]
    assert slots % page_block_size == 0
    num_pages = slots // page_block_size
    pb = payload.shape[1]
    if dtype == "bf16":
        row_stride = _round_up(pb + row_pad, 16)
        page_stride = _round_up(page_block_size * row_stride + page_pad, 16)
        buf = np.zeros(num_pages * page_stride, dtype=np.uint8)
        view = buf.reshape(num_pages, page_stride)[:, : page_block_size * row_stride]
        view = view.reshape(num_pages, page_block_size, row_stride)
        view[:, :, :pb] = payload.reshape(num_pages, page_block_size, pb)
        return Pool(dtype, d_qk, page_block_size, num_pages, buf, 0, page_stride, row_stride,
                    layout="dense" if row_pad == 0 else "padded")

    groups = d_qk // GROUP
    sbytes = scales.astype(np.float32).view(np.uint8).reshape(slots, groups * 4)
    if layout == "inline":
        row_stride = _round_up(pb + groups * 4 + row_pad, 64)
        page_stride = _round_up(page_block_size * row_stride + page_pad, 64)
        buf = np.zeros(num_pages * page_stride, dtype=np.uint8)
        view = buf.reshape(num_pages, page_stride)[:, : page_block_size * row_stride]
        view = view.reshape(num_pages, page_block_size, row_stride)
        view[:, :, :pb] = payload.reshape(num_pages, page_block_size, pb)
        view[:, :, pb : pb + groups * 4] = sbytes.reshape(num_pages, page_block_size, -1)
        return Pool(dtype, d_qk, page_block_size, num_pages, buf, 0, page_stride, row_stride,
                    buf, pb, page_stride, row_stride, layout)
    if layout == "footer":
        row_stride = _round_up(pb + row_pad, 16)
        body = page_block_size * row_stride
        page_stride = _round_up(body + page_block_size * groups * 4 + page_pad, 64)
        buf = np.zeros(num_pages * page_stride, dtype=np.uint8)
        pages = buf.reshape(num_pages, page_stride)
        pv = pages[:, :body].reshape(num_pages, page_block_size, row_stride)
        pv[:, :, :pb] = payload.reshape(num_pages, page_block_size, pb)
        pages[:, body : body + page_block_size * groups * 4] = sbytes.reshape(num_pages, -1)
        return Pool(dtype, d_qk, page_block_size, num_pages, buf, 0, page_stride, row_stride,
                    buf, body, page_stride, groups * 4, layout)
    if layout == "separate":
        row_stride = _round_up(pb + row_pad, 16)
        page_stride = _round_up(page_block_size * row_stride + page_pad, 16)
        buf = np.zeros(num_pages * page_stride, dtype=np.uint8)
        view = buf.reshape(num_pages, page_stride)[:, : page_block_size * row_stride]
        view = view.reshape(num_pages, page_block_size, row_stride)
        view[:, :, :pb] = payload.reshape(num_pages, page_block_size, pb)
        sbuf = np.ascontiguousarray(sbytes).reshape(-1)
        return Pool(dtype, d_qk, page_block_size, num_pages, buf, 0, page_stride, row_stride,
                    sbuf, 0, page_block_size * groups * 4, groups * 4, layout)
    raise ValueError(f"unknown layout {layout!r}")


def draw_pool(
    rng: np.random.Generator,
    dtype: str,
    d_qk: int,
    num_pages: int,
    layout: str = "inline",
    page_block_size: int = PAGE_BLOCK_SIZE,
    row_pad: int = 0,
    page_pad: int = 0,
    row_std: float = 1.0,
) -> Pool:
    """Draw N(0, row_std^2) latent rows (N(0,1) by default) and store them as bf16, or as fp8
    with per-64 scales."""
    slots = num_pages * page_block_size
    x = rng.standard_normal((slots, d_qk), dtype=np.float32)
    if row_std != 1.0:
        x *= np.float32(row_std)
    if dtype == "bf16":
        payload = to_bf16_bits(x).view(np.uint8).reshape(slots, 2 * d_qk)
        return pack_pool(payload, None, dtype, d_qk, layout, page_block_size, row_pad, page_pad)
    s = draw_scales(rng, slots, d_qk // GROUP)
    payload = to_e4m3_bytes(x / np.repeat(s, GROUP, axis=1))
    return pack_pool(payload, s, dtype, d_qk, layout, page_block_size, row_pad, page_pad)


def pool_payload(pool: Pool) -> tuple[np.ndarray, Optional[np.ndarray]]:
    """Read back the stored rows as (payload bytes [slots, payload_bytes], scales fp32).

    Only byte copies through the descriptor; used to build re-laid-out copies of a pool.
    """
    pb = pool.payload_bytes
    slots = np.arange(pool.num_slots)
    page, off = slots // pool.page_block_size, slots % pool.page_block_size
    start = pool.data_offset + page * pool.page_stride + off * pool.row_stride
    payload = pool.data[start[:, None] + np.arange(pb)[None, :]]
    if pool.dtype == "bf16":
        return payload, None
    g4 = (pool.d_qk // GROUP) * 4
    s0 = pool.scale_offset + page * pool.scale_page_stride + off * pool.scale_row_stride
    sb = pool.scales[s0[:, None] + np.arange(g4)[None, :]]
    return payload, np.ascontiguousarray(sb).view(np.float32).reshape(pool.num_slots, -1)


def relayout(pool: Pool, layout: str, row_pad: int = 0, page_pad: int = 0) -> Pool:
    payload, scales = pool_payload(pool)
    return pack_pool(payload, scales, pool.dtype, pool.d_qk, layout, pool.page_block_size,
                     row_pad, page_pad)


# --------------------------------------------------------------------------- indices
def distinct(rng: np.random.Generator, lo: int, hi: int, k: int) -> np.ndarray:
    """k distinct ints drawn uniformly from [lo, hi] (inclusive), in random order.

    If the range holds fewer than k values, all of them are returned (shuffled) followed
    by -1 padding.
    """
    n = hi - lo + 1
    if n <= k:
        out = np.full(k, -1, dtype=np.int64)
        out[:n] = lo + rng.permutation(n)
        return out
    if k * 4 >= n:
        return lo + rng.permutation(n)[:k]
    while True:
        cand = np.unique(rng.integers(lo, hi + 1, size=k + k // 4 + 16))
        if cand.size >= k:
            return rng.permutation(cand)[:k]


def knock_out(rng: np.random.Generator, idx: np.ndarray, count: int) -> np.ndarray:
    """Set ``count`` uniformly chosen entries of each row to -1 (in place)."""
    T, k = idx.shape
    for t in range(T):
        idx[t, rng.choice(k, size=count, replace=False)] = -1
    return idx


def draw_q(rng: np.random.Generator, T: int, h: int, d_qk: int) -> np.ndarray:
    return to_bf16_bits(rng.standard_normal((T, h, d_qk), dtype=np.float32))


def draw_sink(rng: np.random.Generator, h: int) -> np.ndarray:
    return rng.standard_normal(h, dtype=np.float32).astype(np.float32)


# --------------------------------------------------------------------------- workloads
GEOMETRIES = {576: 512, 1088: 1024}


def workload_tiny_bf16(seed: int = 1000) -> Problem:
    """T=4, h=16, topk=128 (8 entries -1 per row), 1024-slot bf16 pool, scale 1/24."""
    rng = np.random.default_rng(seed)
    T, h, d_qk, d_v, topk = 4, 16, 576, 512, 128
    kv = draw_pool(rng, "bf16", d_qk, 16)
    q = draw_q(rng, T, h, d_qk)
    sink = draw_sink(rng, h)
    idx = np.stack([distinct(rng, 0, 1023, topk) for _ in range(T)]).astype(np.int32)
    knock_out(rng, idx, 8)
    return Problem("tiny_bf16_T4_h16_k128", T, h, d_qk, d_v, q, kv, idx, 1.0 / 24.0, sink)


def workload_decode(seed: int = 1001, T: int = 32, h: int = 64, topk: int = 512,
                    ctx: int = 18432) -> Problem:
    """Decode: T sequences x 1 token, fp8 pool, pages scattered by a random page table."""
    rng = np.random.default_rng(seed)
    d_qk, d_v = 576, 512
    pages_per_seq = ctx // PAGE_BLOCK_SIZE
    num_pages = T * pages_per_seq
    kv = draw_pool(rng, "fp8", d_qk, num_pages)
    page_table = rng.permutation(num_pages).reshape(T, pages_per_seq)
    q = draw_q(rng, T, h, d_qk)
    sink = draw_sink(rng, h)
    idx = np.empty((T, topk), dtype=np.int32)
    for t in range(T):
        pos = distinct(rng, 0, ctx - 1, topk)
        idx[t] = page_table[t, pos // PAGE_BLOCK_SIZE] * PAGE_BLOCK_SIZE + pos % PAGE_BLOCK_SIZE
    return Problem(f"decode_fp8_T{T}_h{h}_k{topk}", T, h, d_qk, d_v, q, kv, idx,
                   1.0 / math.sqrt(d_qk), sink)


def workload_causal_prefill(seed: int, T: int, h: int, topk: int, ctx: int,
                            name: str, token_rows: Optional[np.ndarray] = None) -> Problem:
    """Causal prefill over one sequence: token t draws from [0, ctx - T + t], fp8 pool."""
    rng = np.random.default_rng(seed)
    d_qk, d_v = 576, 512
    kv = draw_pool(rng, "fp8", d_qk, ctx // PAGE_BLOCK_SIZE)
    q = draw_q(rng, T, h, d_qk)
    sink = draw_sink(rng, h)
    base = ctx - T
    idx = np.empty((T, topk), dtype=np.int32)
    for t in range(T):
        idx[t] = distinct(rng, 0, base + t, topk)
    return Problem(name, T, h, d_qk, d_v, q, kv, idx, 1.0 / math.sqrt(d_qk), sink)


def workload_tp2_prefill(seed: int = 1002) -> Problem:
    """T=4096, h=32, topk=256, fp8, context 8192 (the tensor-parallel-2 shard shape)."""
    return workload_causal_prefill(seed, 4096, 32, 256, 8192, "prefill_fp8_T4096_h32_k256")


def workload_large_prefill(seed: int = 1003) -> Problem:
    """T=8192, h=128, topk=2048, fp8, context 65536."""
    return workload_causal_prefill(seed, 8192, 128, 2048, 65536,
                                   "prefill_fp8_T8192_h128_k2048")


def workload_dual_window(seed: int = 1004, T: int = 512, h: int = 64) -> Problem:
    """Dual cache, d_qk=1088/d_v=1024: fp8 main (512 from a 4096 window) + bf16 extra
    (128 from 2048 slots); 64 of each token's 640 entries set to -1."""
    rng = np.random.default_rng(seed)
    d_qk, d_v = 1088, 1024
    window, topk, topk_extra, extra_slots = 4096, 512, 128, 2048
    kv = draw_pool(rng, "fp8", d_qk, (window + T) // PAGE_BLOCK_SIZE)
    extra = draw_pool(rng, "bf16", d_qk, extra_slots // PAGE_BLOCK_SIZE)
    q = draw_q(rng, T, h, d_qk)
    sink = draw_sink(rng, h)
    idx = np.empty((T, topk), dtype=np.int32)
    eidx = np.empty((T, topk_extra), dtype=np.int32)
    for t in range(T):
        idx[t] = distinct(rng, t + 1, window + t, topk)
        eidx[t] = distinct(rng, 0, extra_slots - 1, topk_extra)
    both = np.concatenate([idx, eidx], axis=1)
    knock_out(rng, both, (topk + topk_extra) // 10)
    idx[:], eidx[:] = both[:, :topk], both[:, topk:]
    return Problem(f"dual_fp8_bf16_T{T}_h{h}_k{topk}+{topk_extra}", T, h, d_qk, d_v, q, kv,
                   idx, 1.0 / math.sqrt(d_qk), sink, extra, eidx)


WORKLOADS = {
    "tiny_bf16": workload_tiny_bf16,
    "decode_fp8": workload_decode,
    "prefill_tp2": workload_tp2_prefill,
    "prefill_large": workload_large_prefill,
    "dual_window": workload_dual_window,
}


def small_problem(
    seed: int,
    T: int = 2,
    h: int = 3,
    d_qk: int = 576,
    topk: int = 64,
    dtype: str = "fp8",
    layout: str = "inline",
    num_pages: int = 4,
    sink: Optional[str] = "normal",  # "normal", "none", "neginf"
    invalid: float = 0.25,
    out_of_range: int = 0,
    extra_dtype: Optional[str] = None,
    extra_layout: str = "inline",
    extra_pages: int = 2,
    topk_extra: int = 64,
    sm_scale: Optional[float] = None,
    duplicates: bool = False,
    lengths: bool = False,
    row_std: float = 1.0,
) -> Problem:
    """A small seeded problem for oracle pins and GPU parity sweeps. Rows are N(0, row_std^2)
    (row_std 1 draws exactly what earlier versions drew)."""
    rng = np.random.default_rng(seed)
    d_v = GEOMETRIES[d_qk]
    kv = draw_pool(rng, dtype, d_qk, num_pages, layout, row_std=row_std)
    q = draw_q(rng, T, h, d_qk)
    attn_sink = None
    if sink == "normal":
        attn_sink = draw_sink(rng, h)
    elif sink == "neginf":
        attn_sink = np.full(h, -np.inf, dtype=np.float32)

    def _idx(nslots: int, k: int) -> np.ndarray:
        out = np.empty((T, k), dtype=np.int32)
        for t in range(T):
            if duplicates:
                out[t] = rng.integers(0, nslots, size=k)
            else:
                out[t] = distinct(rng, 0, nslots - 1, k)
            bad = rng.random(k) < invalid
            out[t, bad] = -1
            if out_of_range:
                pos = rng.choice(k, size=min(out_of_range, k), replace=False)
                out[t, pos] = rng.choice([nslots, nslots + 7, 2**31 - 1, -5, -(2**31)],
                                         size=pos.size)
        return out

    idx = _idx(kv.num_slots, topk)
    extra = eidx = None
    if extra_dtype is not None:
        extra = draw_pool(rng, extra_dtype, d_qk, extra_pages, extra_layout, row_std=row_std)
        eidx = _idx(extra.num_slots, topk_extra)
    scale = (1.0 / math.sqrt(d_qk)) if sm_scale is None else sm_scale
    tl = etl = None
    if lengths:
        tl = draw_lengths(rng, T, topk)
        if eidx is not None:
            etl = draw_lengths(rng, T, topk_extra)
    return Problem(f"small_s{seed}", T, h, d_qk, d_v, q, kv, idx, scale, attn_sink, extra, eidx,
                   tl, etl)


def draw_lengths(rng: np.random.Generator, T: int, k: int) -> np.ndarray:
    """Per-row live counts for an index list of width k: uniform in [0, k], with the edge
    values 0, 1, k - 1, k, a negative count and one above k placed first when T allows."""
    out = rng.integers(0, k + 1, size=T).astype(np.int32)
    edges = [0, k, 1, k + 5, k - 1, -3]
    n = min(T, len(edges))
    out[:n] = edges[:n]
    return out


def draw_pack_rows(seed: int, n: int, d_qk: int = 576, spread: float = 6.0) -> np.ndarray:
    """bf16 rows to pack: N(0,1) scaled per group of 64 by 2^U(-spread,spread). When n
    allows, row 0 has an all-zero group (with a -0.0) and a group with a single nonzero
    value, row 1 a group of negative values only, and row 2 a group of values near 1e-38."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d_qk)).astype(np.float32)
    x *= np.repeat(2.0 ** rng.uniform(-spread, spread, (n, d_qk // GROUP)), GROUP,
                   axis=1).astype(np.float32)
    if n > 0:
        x[0, 64:128] = 0.0
        x[0, 100] = -0.0
        x[0, 128:192] = 0.0
        x[0, 130] = -3.0
    if n > 1:
        x[1, :64] = -np.abs(x[1, :64])
    if n > 2 and d_qk >= 256:
        x[2, 192:256] *= np.float32(1e-38)  # tiny and subnormal values (multiplier clamps)
    return to_bf16_bits(x)
