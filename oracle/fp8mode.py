"""CPU oracle of the fp8 compute mode (test infrastructure only).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this module. The GPU library never calls it and shares no code with it.

What it computes. The fp8 compute mode is an approximation of the attention in
oracle.reference: "fix(sparse-mla-sm120): add topk=256 prefill-dsv4 dispatch" forks the
prefill kernels on a compute mode (FP8 / BF16) and the FlashInfer 4802 merge message
(section "Performance vs main") quantises q on the fp8 side. The pages print no rule; the
reading taken mirrors the KV packing (oracle.pack): per (token, head) row of q,
    amax = max_d |q_d|                                 (bf16 values, exact in fp32)
    qs   = fl32(amax / 448)                            (the factor the logits take back)
    inv  = min(fl32(448 / amax), FLT_MAX)
    code_d = the e4m3fn value nearest to clamp(fl32(q_d * inv), -448, 448), ties to even
and the attention then runs in float64 on q'_d = e4m3fn(code_d) * qs with everything else
unchanged. The codes are integers decided in fp32, as the kernel decides them.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .pack import E4M3_MAX, e4m3fn_nearest_even
from .reference import attend, bf16_to_f64, e4m3fn_table, gather_token

_TABLE = e4m3fn_table()


def quantize_q_rows(q_bits: np.ndarray):
    """bf16 rows [..., d] -> (codes uint8 [..., d], qs float32 [..., 1])."""
    x = bf16_to_f64(q_bits).astype(np.float32)  # exact
    amax = np.max(np.abs(x), axis=-1, keepdims=True).astype(np.float32)
    qs = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        inv = np.minimum(np.float32(E4M3_MAX) / amax, np.finfo(np.float32).max).astype(np.float32)
    v = np.clip((x * inv).astype(np.float32), -E4M3_MAX, E4M3_MAX)
    return e4m3fn_nearest_even(v), qs


def dequantized_q(q_bits: np.ndarray) -> np.ndarray:
    """The q the fp8 mode attends with: e4m3fn(code) * qs, float64."""
    codes, qs = quantize_q_rows(q_bits)
    return _TABLE[codes] * qs.astype(np.float64)


def sparse_mla_reference_fp8q(p, tokens: Optional[np.ndarray] = None):
    """(o, lse) of the fp8 compute mode: the exact attention with q replaced by its e4m3fn
    rounding per (token, head)."""
    toks = np.arange(p.T) if tokens is None else np.asarray(tokens)
    qd = dequantized_q(np.asarray(p.q_bits)[toks])  # [n_tok, h, d]
    o = np.zeros((len(toks), p.h, p.d_v))
    lse = np.zeros((len(toks), p.h))
    sink = (np.full(p.h, -np.inf) if p.attn_sink is None
            else np.asarray(p.attn_sink, dtype=np.float64))
    for i, t in enumerate(toks):
        o[i], lse[i] = attend(qd[i], gather_token(p, int(t)), sink, float(p.sm_scale), p.d_v)
    return o, lse
