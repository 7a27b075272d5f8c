"""Pure-Python brute force of sparse top-k MLA attention, for tiny inputs.

TEST INFRASTRUCTURE ONLY. It shares no code with ``oracle.reference``; its job is to pin
that module. It decodes raw bytes with ``struct`` and bit arithmetic of its own, walks the
descriptor one slot at a time, and sums with ``math.fsum``. The function it computes is
the one stated in ``oracle.reference``: dense softmax attention over the valid gathered
rows, with the per-head sink logit in the denominator only.
"""
from __future__ import annotations

import math
import struct


def _fp8_e4m3fn(byte: int) -> float:
    # Bit fields: s eeee mmm, exponent bias 7, no infinities, S.1111.111 is NaN.
    s, e, m = byte >> 7, (byte >> 3) & 15, byte & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = math.ldexp(m, -9) if e == 0 else math.ldexp(8 + m, e - 10)
    return -mag if s else mag


def _bf16(lo: int, hi: int) -> float:
    return struct.unpack("<f", bytes([0, 0, lo, hi]))[0]


def _row(pool, slot: int) -> list[float]:
    page, off = divmod(slot, pool.page_block_size)
    base = pool.data_offset + page * pool.page_stride + off * pool.row_stride
    data = pool.data
    if pool.dtype == "bf16":
        return [_bf16(int(data[base + 2 * d]), int(data[base + 2 * d + 1]))
                for d in range(pool.d_qk)]
    sbase = pool.scale_offset + page * pool.scale_page_stride + off * pool.scale_row_stride
    sc = pool.scales
    scales = [struct.unpack("<f", bytes(int(sc[sbase + 4 * g + i]) for i in range(4)))[0]
              for g in range(pool.d_qk // 64)]
    return [_fp8_e4m3fn(int(data[base + d])) * scales[d // 64] for d in range(pool.d_qk)]


def _rows(pool, index_row) -> list[list[float]]:
    nslots = pool.num_pages * pool.page_block_size
    return [_row(pool, int(s)) for s in index_row if 0 <= int(s) < nslots]


def _count(lengths, t: int, width: int) -> int:
    # entries past a row's live count (clamped to [0, width]) take no part
    if lengths is None:
        return width
    c = int(lengths[t])
    return 0 if c < 0 else min(c, width)


def brute_force(p):
    """Return (o, lse) as nested lists [T][h][d_v] and [T][h]."""
    o_all, lse_all = [], []
    for t in range(p.T):
        row = list(p.indices[t])
        rows = _rows(p.kv, row[:_count(getattr(p, "topk_length", None), t, len(row))])
        if p.extra is not None and p.extra_indices is not None:
            erow = list(p.extra_indices[t])
            rows += _rows(p.extra,
                          erow[:_count(getattr(p, "extra_topk_length", None), t, len(erow))])
        o_t, lse_t = [], []
        for h in range(p.h):
            q = [_bf16(int(b) & 0xFF, int(b) >> 8) for b in p.q_bits[t, h]]
            sink = -math.inf if p.attn_sink is None else float(p.attn_sink[h])
            z = [p.sm_scale * math.fsum(a * b for a, b in zip(q, r)) for r in rows]
            m = max(z + [sink])
            if m == -math.inf:
                o_t.append([0.0] * p.d_v)
                lse_t.append(-math.inf)
                continue
            w = [math.exp(zj - m) for zj in z]
            denom = math.fsum(w + [math.exp(sink - m)])
            o_t.append([math.fsum(wj * r[d] for wj, r in zip(w, rows)) / denom
                        for d in range(p.d_v)])
            lse_t.append(m + math.log(denom))
        o_all.append(o_t)
        lse_all.append(lse_t)
    return o_all, lse_all
