"""Plain CPU oracle for packing bf16 latent rows into the fp8 paged pool.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this module. The GPU library never calls it and shares no code with it.

What it computes. The step before the attention path writes each new latent row into its
paged slot in the fp8 format the path reads. The pages name that step without printing it:
"fix(sparse-mla-sm120): add topk=256 prefill-dsv4 dispatch" (FlashInfer PR 3896), in the
comment thread's compute-mode comparison, packs the KV input with quantize_kv_dsv4 on both
sides; the FlashInfer 4802 merge message (sections Summary and Compatibility) gives the
inline and footer placements of the per-64 scales. The plainest reading is taken for the
arithmetic: each group of 64 consecutive elements is multiplied onto e4m3fn's range so that
its largest magnitude lands on the largest finite value, 448, and the stored scale is the
factor that maps the codes back.

For a row x (bf16 values, exact in fp32) and each group g of 64 elements:
    amax_g  = max_d |x_d|                                   (exact)
    scale_g = fl32(amax_g / 448)                            (stored; 0 for an all-zero group)
    inv_g   = min(fl32(448 / amax_g), FLT_MAX)              (the quantising multiplier)
    v_d     = clamp(fl32(x_d * inv_g), -448, 448)           (x_d itself when amax_g is 0)
(inv_g reaches the clamp only for amax_g below about 2^-118, where 448 / amax_g overflows.)
    code_d  = the e4m3fn code nearest to v_d, ties to the even code (sign kept for 0)
fl32 is one IEEE float32 operation rounded to nearest even: the quantised code is an
integer decided in floating point, so the oracle takes that decision in the precision the
kernel takes it. A slot outside [0, num_slots) is skipped; its bytes stay as they were.
"""
from __future__ import annotations

import numpy as np

from .reference import GROUP, bf16_to_f64, e4m3fn_table

E4M3_MAX = 448.0

_TABLE = e4m3fn_table()
_FINITE = np.array([c for c in range(256) if not np.isnan(_TABLE[c]) and c != 0x80])
_ORDER = np.argsort(_TABLE[_FINITE], kind="stable")
_SORTED_VALS = _TABLE[_FINITE][_ORDER]    # the 253 distinct finite values, ascending
_SORTED_CODES = _FINITE[_ORDER]


def e4m3fn_nearest_even(v: np.ndarray) -> np.ndarray:
    """Codes of the e4m3fn values nearest to v (|v| <= 448), ties to the even code.

    The finite values sorted ascending (one code per value; zero is taken as +0): for each
    v its two neighbours in that list, the nearer one, and on equal distances the code whose
    mantissa's last bit is 0. A zero result takes the sign of v (0x80 for v < 0 or -0.0).
    """
    v = np.asarray(v, dtype=np.float64)
    flat = v.reshape(-1)
    hi = np.clip(np.searchsorted(_SORTED_VALS, flat), 1, len(_SORTED_VALS) - 1)
    lo = hi - 1
    dlo, dhi = flat - _SORTED_VALS[lo], _SORTED_VALS[hi] - flat
    clo, chi = _SORTED_CODES[lo], _SORTED_CODES[hi]
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((chi & 1) == 0) & ((clo & 1) == 1))
    out = np.where(pick_hi, chi, clo).astype(np.uint8)
    zero = _TABLE[out] == 0.0
    out[zero] = np.where(np.signbit(flat[zero]), 0x80, 0x00)
    return out.reshape(v.shape)


def quantize_row(x_bits: np.ndarray):
    """One row of bf16 bit patterns [d_qk] -> (codes uint8 [d_qk], scales float32 [d_qk/64])."""
    x = bf16_to_f64(x_bits).astype(np.float32)  # exact
    d_qk = x.shape[0]
    codes = np.empty(d_qk, dtype=np.uint8)
    scales = np.empty(d_qk // GROUP, dtype=np.float32)
    for g in range(d_qk // GROUP):
        xs = x[g * GROUP:(g + 1) * GROUP]
        amax = np.float32(np.max(np.abs(xs)))
        scales[g] = np.float32(amax / np.float32(E4M3_MAX))
        if amax == 0.0:
            codes[g * GROUP:(g + 1) * GROUP] = np.where(np.signbit(xs), 0x80, 0x00)
            continue
        with np.errstate(over="ignore"):
            inv = np.minimum(np.float32(E4M3_MAX) / amax, np.finfo(np.float32).max)
        v = np.clip((xs * inv).astype(np.float32), -E4M3_MAX, E4M3_MAX)
        codes[g * GROUP:(g + 1) * GROUP] = e4m3fn_nearest_even(v)
    return codes, scales


def pack_kv_reference(rows_bits: np.ndarray, slots: np.ndarray, pool) -> None:
    """Write every row into its slot of ``pool`` (an fp8 pool, modified in place).

    rows_bits: bf16 bit patterns [n, d_qk]; slots: int [n]. Payload bytes go to
    data_offset + page * page_stride + offset * row_stride, scales (fp32, little-endian)
    to scale_offset + page * scale_page_stride + offset * scale_row_stride.
    """
    if pool.dtype != "fp8":
        raise ValueError("the packed pool is fp8")
    nslots = pool.num_pages * pool.page_block_size
    for r, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if not 0 <= s < nslots:
            continue
        codes, scales = quantize_row(np.asarray(rows_bits[r], dtype=np.uint16))
        page, off = divmod(int(s), pool.page_block_size)
        base = pool.data_offset + page * pool.page_stride + off * pool.row_stride
        pool.data[base:base + pool.d_qk] = codes
        sbase = pool.scale_offset + page * pool.scale_page_stride + off * pool.scale_row_stride
        pool.scales[sbase:sbase + 4 * len(scales)] = scales.astype("<f4").view(np.uint8)
