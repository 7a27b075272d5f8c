"""Pins for the CPU oracle: independent checks, not a retyping of its formula.

* brute force: a pure-Python second implementation with its own byte decoders;
* torch's scaled_dot_product_attention: with no sink and every entry valid, the method is
  plain softmax attention over the gathered rows;
* closed forms (q = 0, a single valid row, all-invalid rows) and hand-derived cases in
  tests/golden/hand_cases.json;
* invariants: permutation of the index list, head prefix, dual cache equal to one
  concatenated pool, -1 compaction, byte-layout invariance, power-of-two scale covariance,
  a row's live count equal to knocking out its later entries, a ragged width equal to the
  same row padded with -1;
* the e4m3fn and bf16 code tables checked against torch's dtypes;
* planted mistakes: each plausible error in the oracle fails at least one of these pins.
"""
from __future__ import annotations

import copy
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.reference as R
from oracle.brute import brute_force
from workloads import synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


# --------------------------------------------------------------------------- helpers
def torch_rows(pool: S.Pool) -> torch.Tensor:
    """All rows of a pool decoded with torch's own dtypes (an independent decoder)."""
    payload, scales = S.pool_payload(pool)
    if pool.dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(payload)).view(torch.bfloat16)
        return t.to(torch.float64)
    v = torch.from_numpy(np.ascontiguousarray(payload)).view(torch.float8_e4m3fn)
    v = v.to(torch.float64)
    s = torch.from_numpy(scales).to(torch.float64)
    return v * s.repeat_interleave(64, dim=1)


def torch_q(p: S.Problem) -> torch.Tensor:
    return torch.from_numpy(p.q_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64)


def valid_entries(pool: S.Pool, row) -> list[int]:
    return [int(s) for s in row if 0 <= int(s) < pool.num_slots]


def sdpa_reference(p: S.Problem) -> np.ndarray:
    """Dense softmax attention (no sink) over the gathered rows, via torch SDPA."""
    rows = torch_rows(p.kv)
    erows = torch_rows(p.extra) if p.extra is not None else None
    q = torch_q(p)
    out = []
    for t in range(p.T):
        k = rows[valid_entries(p.kv, p.indices[t])]
        if erows is not None:
            k = torch.cat([k, erows[valid_entries(p.extra, p.extra_indices[t])]])
        qt = q[t][None, :, None, :]  # [1, h, 1, d_qk]
        kk = k[None, None].expand(1, p.h, -1, -1).contiguous()
        vv = k[:, : p.d_v][None, None].expand(1, p.h, -1, -1).contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(qt, kk, vv, scale=p.sm_scale)
        out.append(o[0, :, 0, :].numpy())
    return np.stack(out)


def close(a, b, tol):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        diff = np.where(both_inf, 0.0, np.abs(a - b))
    return bool(np.all(diff <= tol))


BRUTE_CASES = [
    dict(seed=1, dtype="fp8", layout="inline", sink="normal", invalid=0.25, out_of_range=3),
    dict(seed=2, dtype="fp8", layout="footer", sink="none", invalid=0.1),
    dict(seed=3, dtype="fp8", layout="separate", d_qk=1088, sink="neginf", invalid=0.2),
    dict(seed=4, dtype="bf16", layout="inline", sink="normal", invalid=0.3, out_of_range=2),
    dict(seed=5, dtype="bf16", d_qk=1088, sink="normal", extra_dtype="fp8", invalid=0.1),
    dict(seed=6, dtype="fp8", sink="normal", extra_dtype="bf16", invalid=0.1, out_of_range=1),
    dict(seed=7, dtype="fp8", d_qk=1088, sink="normal", extra_dtype="bf16", T=1, h=2),
    dict(seed=8, dtype="fp8", sink="normal", duplicates=True, invalid=0.0),
    dict(seed=9, dtype="fp8", sink="normal", invalid=1.0, extra_dtype="bf16"),
    dict(seed=10, dtype="bf16", sink="normal", topk=128, T=1, h=4, num_pages=3),
    dict(seed=11, dtype="fp8", sink="none", invalid=1.0),
    # ragged widths (not multiples of 64) and per-row live counts
    dict(seed=12, dtype="fp8", sink="normal", topk=37, invalid=0.2, out_of_range=2),
    dict(seed=13, dtype="fp8", sink="normal", topk=50, extra_dtype="bf16", topk_extra=21,
         lengths=True, T=6, h=2, invalid=0.1),
    dict(seed=14, dtype="bf16", d_qk=1088, sink="none", topk=33, lengths=True, T=6, h=2,
         invalid=0.1),
]


# --------------------------------------------------------------------------- decoders
def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = R.e4m3fn_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(tab), nan)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(tab[~nan], ref[~nan])
    assert np.array_equal(np.signbit(tab[~nan]), np.signbit(ref[~nan]))


def test_e4m3_named_codes():
    v = R.e4m3fn_value
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0
    assert v(0x08) == 2.0 ** -6  # smallest normal
    assert v(0x01) == 2.0 ** -9  # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9  # largest subnormal
    assert v(0x38) == 1.0 and v(0x40) == 2.0 and v(0x30) == 0.5
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0


def test_bf16_decoder_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    with np.errstate(invalid="ignore"):
        got = R.bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_encoders_round_trip_exactly():
    # e4m3fn codes re-encode to themselves (except NaN); saturation clamps to 448.
    vals = R.e4m3fn_table()
    ok = ~np.isnan(vals)
    codes = S.to_e4m3_bytes(vals[ok].astype(np.float32))
    assert np.array_equal(R.e4m3fn_table()[codes], vals[ok])
    assert S.to_e4m3_bytes(np.array([1e6, -1e6], np.float32)).tolist() == [0x7E, 0xFE]


# --------------------------------------------------------------------------- brute force
@pytest.mark.parametrize("case", BRUTE_CASES, ids=lambda c: f"seed{c['seed']}")
def test_oracle_matches_brute_force(case):
    p = S.small_problem(**case)
    o, lse = R.sparse_mla_reference(p)
    bo, blse = brute_force(p)
    assert close(o, bo, 1e-12)
    assert close(lse, blse, 1e-12)


def test_brute_force_sees_extra_cache():
    # The extra list is part of the same softmax: dropping it changes the answer.
    p = S.small_problem(seed=21, dtype="fp8", extra_dtype="bf16", invalid=0.0)
    q = copy.copy(p)
    q.extra, q.extra_indices = None, None
    assert not close(R.sparse_mla_reference(p)[0], R.sparse_mla_reference(q)[0], 1e-3)


# --------------------------------------------------------------------------- SDPA
def test_live_count_equals_knock_out():
    # Entries past a row's live count act exactly like -1 entries; a count below 0 keeps
    # nothing and one above the width keeps the whole row.
    p = S.small_problem(seed=58, T=6, h=3, topk=70, lengths=True, extra_dtype="fp8",
                        topk_extra=30, invalid=0.2)
    assert p.topk_length.tolist()[:6] == [0, 70, 1, 75, 69, -3]
    q = copy.deepcopy(p)
    for idx, lens in ((q.indices, p.topk_length), (q.extra_indices, p.extra_topk_length)):
        for t in range(p.T):
            idx[t, max(int(lens[t]), 0):] = -1
    q.topk_length = q.extra_topk_length = None
    a, b = R.sparse_mla_reference(p), R.sparse_mla_reference(q)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_ragged_width_equals_padded_width():
    # A width that is not a multiple of 64 computes what the same row padded with -1 does.
    p = S.small_problem(seed=59, T=3, h=2, topk=100, extra_dtype="bf16", topk_extra=10,
                        invalid=0.1)
    q = copy.deepcopy(p)
    q.indices = np.concatenate([p.indices, np.full((3, 28), -1, np.int32)], axis=1)
    q.extra_indices = np.concatenate([p.extra_indices, np.full((3, 54), -1, np.int32)], axis=1)
    a, b = R.sparse_mla_reference(p), R.sparse_mla_reference(q)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("dtype,d_qk,extra", [("fp8", 576, None), ("bf16", 576, None),
                                               ("fp8", 1088, "bf16"), ("bf16", 1088, "fp8")])
def test_no_sink_equals_sdpa(dtype, d_qk, extra):
    p = S.small_problem(seed=31, T=3, h=5, d_qk=d_qk, topk=128, dtype=dtype, sink="none",
                        invalid=0.0, extra_dtype=extra, num_pages=3)
    o, _ = R.sparse_mla_reference(p)
    assert close(o, sdpa_reference(p), 1e-12)


def test_neginf_sink_equals_no_sink():
    p = S.small_problem(seed=32, T=2, h=3, sink="neginf", invalid=0.2)
    q = copy.copy(p)
    q.attn_sink = None
    a, b = R.sparse_mla_reference(p), R.sparse_mla_reference(q)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# --------------------------------------------------------------------------- closed forms
def test_zero_query_gives_mean_with_sink_weight():
    p = S.small_problem(seed=41, T=2, h=4, topk=128, sink="normal", invalid=0.3,
                        extra_dtype="bf16", num_pages=3)
    p.q_bits = np.zeros_like(p.q_bits)
    o, lse = R.sparse_mla_reference(p)
    rows, erows = torch_rows(p.kv).numpy(), torch_rows(p.extra).numpy()
    for t in range(p.T):
        v = np.concatenate([rows[valid_entries(p.kv, p.indices[t])],
                            erows[valid_entries(p.extra, p.extra_indices[t])]])
        n = len(v)
        for h in range(p.h):
            sig = float(p.attn_sink[h])
            expect = v[:, : p.d_v].sum(axis=0) / (n + math.exp(sig))
            assert close(o[t, h], expect, 1e-12)
            assert abs(lse[t, h] - math.log(n + math.exp(sig))) < 1e-12


def test_single_valid_row_is_logistic():
    p = S.small_problem(seed=42, T=3, h=4, sink="normal", invalid=0.0)
    for t in range(p.T):
        keep = t * 5 % p.topk
        p.indices[t, np.arange(p.topk) != keep] = -1
    o, lse = R.sparse_mla_reference(p)
    rows = torch_rows(p.kv).numpy()
    q = torch_q(p).numpy()
    for t in range(p.T):
        r = rows[int(p.indices[t, t * 5 % p.topk])]
        for h in range(p.h):
            z = p.sm_scale * float(np.dot(q[t, h], r))
            sig = float(p.attn_sink[h])
            w = 1.0 / (1.0 + math.exp(sig - z))
            assert close(o[t, h], w * r[: p.d_v], 1e-12)
            assert abs(lse[t, h] - np.logaddexp(z, sig)) < 1e-12


def test_all_invalid_rows():
    p = S.small_problem(seed=43, T=2, h=3, sink="normal", invalid=1.0, out_of_range=5)
    o, lse = R.sparse_mla_reference(p)
    assert np.all(o == 0.0)
    assert np.array_equal(lse, np.broadcast_to(p.attn_sink.astype(np.float64), lse.shape))
    p.attn_sink = None
    o, lse = R.sparse_mla_reference(p)
    assert np.all(o == 0.0) and np.all(np.isneginf(lse)) and not np.isnan(o).any()


def _hand_problem(case) -> S.Problem:
    d_qk, d_v, pbs = 576, 512, 64
    slots = case["num_pages"] * pbs
    if case["dtype"] == "bf16":
        x = np.zeros((slots, d_qk), np.float32)
        for s, row in case["rows"].items():
            for d, val in row.items():
                x[int(s), int(d)] = val
        payload = S.to_bf16_bits(x).view(np.uint8).reshape(slots, 2 * d_qk)
        pool = S.pack_pool(payload, None, "bf16", d_qk)
    else:
        codes = np.zeros((slots, d_qk), np.uint8)
        scales = np.ones((slots, d_qk // 64), np.float32)
        for s, row in case["rows"].items():
            for d, (code, val) in row.items():
                assert R.e4m3fn_value(code) == val
                codes[int(s), int(d)] = code
        for s, sc in case.get("scales", {}).items():
            scales[int(s)] = sc
        pool = S.pack_pool(codes, scales, "fp8", d_qk, "footer")
    q = np.zeros((1, 1, d_qk), np.float32)
    for d, val in case["q"].items():
        q[0, 0, int(d)] = val
    sink = None if case["sink"] is None else np.array([case["sink"]], np.float32)
    idx = np.array([case["indices"]], np.int32)
    return S.Problem(case["name"], 1, 1, d_qk, d_v, S.to_bf16_bits(q), pool, idx,
                     case["sm_scale"], sink)


def _num(x):
    if isinstance(x, (int, float)):
        return float(x)
    e = math.e
    return {"ln3": math.log(3), "ln2": math.log(2), "e/(e+1)": e / (e + 1),
            "1/(e+1)": 1 / (e + 1), "ln(e+1)": math.log(e + 1), "1+ln2": 1 + math.log(2)}[x]


with open(GOLDEN) as f:
    HAND = json.load(f)["cases"]


@pytest.mark.parametrize("case", HAND, ids=lambda c: c["name"])
def test_hand_derived_cases(case):
    p = _hand_problem(case)
    o, lse = R.sparse_mla_reference(p)
    expect = np.zeros(p.d_v)
    for d, val in case["expect_o"].items():
        expect[int(d)] = _num(val)
    assert close(o[0, 0], expect, 1e-15)
    assert abs(lse[0, 0] - _num(case["expect_lse"])) < 1e-15


# --------------------------------------------------------------------------- invariants
def test_permutation_invariance():
    p = S.small_problem(seed=51, T=2, h=4, topk=128, num_pages=3, invalid=0.3,
                        extra_dtype="bf16")
    base = R.sparse_mla_reference(p)
    rng = np.random.default_rng(0)
    q = copy.deepcopy(p)
    for t in range(p.T):
        q.indices[t] = q.indices[t, rng.permutation(p.topk)]
        q.extra_indices[t] = q.extra_indices[t, rng.permutation(p.topk_extra)]
    perm = R.sparse_mla_reference(q)
    assert close(base[0], perm[0], 1e-13) and close(base[1], perm[1], 1e-13)


def test_head_prefix_independence():
    p = S.small_problem(seed=52, T=2, h=7, sink="normal", invalid=0.2)
    o, lse = R.sparse_mla_reference(p)
    for hp in (1, 3, 6):
        q = copy.deepcopy(p)
        q.h, q.q_bits, q.attn_sink = hp, p.q_bits[:, :hp].copy(), p.attn_sink[:hp].copy()
        o2, lse2 = R.sparse_mla_reference(q)
        assert close(o[:, :hp], o2, 1e-14) and close(lse[:, :hp], lse2, 1e-14)


def test_dual_cache_equals_concatenated_pool():
    p = S.small_problem(seed=53, T=2, h=3, dtype="fp8", extra_dtype="fp8", invalid=0.2,
                        extra_pages=2, topk_extra=64)
    pm, sm = S.pool_payload(p.kv)
    pe, se = S.pool_payload(p.extra)
    single = S.pack_pool(np.concatenate([pm, pe]), np.concatenate([sm, se]), "fp8", p.d_qk)
    q = copy.deepcopy(p)
    shifted = np.where(p.extra_indices >= 0, p.extra_indices + p.kv.num_slots, -1)
    q.kv, q.extra, q.extra_indices = single, None, None
    q.indices = np.concatenate([p.indices, shifted.astype(np.int32)], axis=1)
    a, b = R.sparse_mla_reference(p), R.sparse_mla_reference(q)
    assert close(a[0], b[0], 1e-14) and close(a[1], b[1], 1e-14)


def test_invalid_entries_equal_compaction():
    p = S.small_problem(seed=54, T=3, h=2, invalid=0.4, out_of_range=4)
    o, lse = R.sparse_mla_reference(p)
    for t in range(p.T):
        q = copy.deepcopy(p)
        keep = valid_entries(p.kv, p.indices[t])
        q.T, q.q_bits = 1, p.q_bits[t : t + 1]
        q.indices = np.array([keep], np.int32)
        o2, lse2 = R.sparse_mla_reference(q)
        assert np.array_equal(o[t], o2[0]) and np.array_equal(lse[t], lse2[0])


@pytest.mark.parametrize("layout,row_pad,page_pad", [("footer", 0, 0), ("separate", 0, 0),
                                                     ("inline", 64, 128), ("footer", 16, 64)])
def test_byte_layout_invariance(layout, row_pad, page_pad):
    p = S.small_problem(seed=55, T=2, h=3, layout="inline", invalid=0.2)
    q = copy.deepcopy(p)
    q.kv = S.relayout(p.kv, layout, row_pad, page_pad)
    a, b = R.sparse_mla_reference(p), R.sparse_mla_reference(q)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_power_of_two_fp8_equals_bf16_pool():
    rng = np.random.default_rng(56)
    p = S.small_problem(seed=56, T=2, h=3, invalid=0.2)
    payload, _ = S.pool_payload(p.kv)
    scales = np.exp2(rng.integers(-4, 5, size=(p.kv.num_slots, 9))).astype(np.float32)
    p.kv = S.pack_pool(payload, scales, "fp8", 576)
    vals = torch_rows(p.kv).numpy().astype(np.float32)  # exact: e4m3 * 2^k fits bf16
    bf = S.to_bf16_bits(vals)
    assert np.array_equal(R.bf16_to_f64(bf), torch_rows(p.kv).numpy())
    q = copy.deepcopy(p)
    q.kv = S.pack_pool(bf.view(np.uint8).reshape(p.kv.num_slots, -1), None, "bf16", 576)
    a, b = R.sparse_mla_reference(p), R.sparse_mla_reference(q)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_scale_covariance():
    p = S.small_problem(seed=57, T=2, h=3, invalid=0.2)
    payload, scales = S.pool_payload(p.kv)
    o, lse = R.sparse_mla_reference(p)
    for k in (-3, 2):
        c = 2.0 ** k
        q = copy.deepcopy(p)
        q.kv = S.pack_pool(payload, scales * np.float32(c), "fp8", 576)
        q.sm_scale = p.sm_scale / c
        o2, lse2 = R.sparse_mla_reference(q)
        assert np.array_equal(o2, o * c) and np.array_equal(lse2, lse)


# --------------------------------------------------------------------------- parallel harness
@pytest.mark.parametrize("workers,order", [(3, "sorted"), (4, "shuffled"), (7, "subset")])
def test_parallel_oracle_equals_serial_bitwise(workers, order):
    """The block-parallel harness returns the serial oracle's rows, in the order of the token
    list, bit for bit: uneven blocks (np.array_split of 7 or 11 tokens), a shuffled list and
    a subset with a repeated token. Both sides run with one BLAS thread, so the per-token
    arithmetic is the same code on the same thread count."""
    from threadpoolctl import threadpool_limits
    p = S.small_problem(seed=61, T=11, h=5, topk=96, dtype="fp8", sink="normal",
                        invalid=0.2, extra_dtype="bf16", topk_extra=40, extra_pages=2)
    rng = np.random.default_rng(62)
    toks = {"sorted": np.arange(p.T), "shuffled": rng.permutation(p.T),
            "subset": np.array([9, 2, 2, 0, 10, 5, 7])}[order]
    with threadpool_limits(1):
        o_ref, lse_ref = R.sparse_mla_reference(p, toks)
    o, lse, used = R.sparse_mla_reference_parallel(p, toks, workers=workers)
    assert used == min(workers, len(toks))
    assert o.shape == o_ref.shape and np.array_equal(o, o_ref)
    assert np.array_equal(lse, lse_ref)
    # each row is its own token's result, not a neighbour's
    o1, _ = R.sparse_mla_reference(p, toks[-1:])
    assert np.array_equal(o[-1], o1[0])


# --------------------------------------------------------------------------- planted mistakes
def _pins_pass() -> bool:
    """A quick subset of the pins above; True iff every one passes."""
    try:
        for case in (BRUTE_CASES[0], BRUTE_CASES[3], BRUTE_CASES[5], BRUTE_CASES[12]):
            p = S.small_problem(**case)
            o, lse = R.sparse_mla_reference(p)
            bo, blse = brute_force(p)
            if not (close(o, bo, 1e-12) and close(lse, blse, 1e-12)):
                return False
        p = S.small_problem(seed=31, T=2, h=3, topk=64, dtype="fp8", sink="none",
                            invalid=0.0, extra_dtype="bf16")
        if not close(R.sparse_mla_reference(p)[0], sdpa_reference(p), 1e-12):
            return False
        for case in HAND:
            p = _hand_problem(case)
            o, lse = R.sparse_mla_reference(p)
            expect = np.zeros(p.d_v)
            for d, val in case["expect_o"].items():
                expect[int(d)] = _num(val)
            if not (close(o[0, 0], expect, 1e-15) and abs(lse[0, 0] - _num(
                    case["expect_lse"])) < 1e-15):
                return False
    except (IndexError, ValueError, FloatingPointError):
        return False
    return True


def _attend_sink_sign(q, rows, sink, sm_scale, d_v):
    return _ORIG_ATTEND(q, rows, -sink, sm_scale, d_v)


def _attend_no_sink(q, rows, sink, sm_scale, d_v):
    return _ORIG_ATTEND(q, rows, np.full_like(sink, -np.inf), sm_scale, d_v)


def _attend_sink_as_row(q, rows, sink, sm_scale, d_v):
    # mistake: the sink also contributes a value row (first latent row)
    o, lse = _ORIG_ATTEND(q, rows, sink, sm_scale, d_v)
    if rows.shape[0]:
        o = o + (np.exp(sink - lse))[:, None] * rows[0, :d_v][None, :]
    return o, lse


def _attend_no_scale(q, rows, sink, sm_scale, d_v):
    return _ORIG_ATTEND(q, rows, sink, 1.0, d_v)


_ORIG_ATTEND = R.attend

MUTATIONS = {
    "scale_group_shifted": ("_scale_group", lambda d: (d // 64 + 1) % 9),
    "scale_group_by_32": ("_scale_group", lambda d: np.minimum(d // 32, 8)),
    "value_is_last_dims": ("_value_part", lambda rows, d_v: rows[:, -d_v:]),
    "page_offset_swapped": ("_slot_location",
                            lambda pool, s: (s % pool.page_block_size, s // pool.page_block_size)),
    "valid_bound_off_by_one": ("valid_mask",
                               lambda pool, s: (np.asarray(s) >= 0) &
                               (np.asarray(s) <= pool.num_slots)),
    "negatives_kept": ("valid_mask", lambda pool, s: np.asarray(s) < pool.num_slots),
    "sink_sign": ("attend", _attend_sink_sign),
    "sink_dropped": ("attend", _attend_no_sink),
    "sink_has_value": ("attend", _attend_sink_as_row),
    "scale_dropped": ("attend", _attend_no_scale),
    "length_ignored": ("live_entries", lambda row, lengths, t: np.asarray(row, np.int64)),
    "length_off_by_one": ("live_entries", lambda row, lengths, t: np.asarray(row, np.int64)[
        : (len(row) if lengths is None else max(int(lengths[t]), 0) + 1)]),
    "length_not_clamped_below": ("live_entries", lambda row, lengths, t: np.asarray(
        row, np.int64)[: (len(row) if lengths is None else int(lengths[t]))]),
    "bf16_bytes_swapped": ("bf16_to_f64", lambda b: _ORIG_BF16(
        ((np.asarray(b, np.uint16) >> 8) | (np.asarray(b, np.uint16) << 8)).astype(np.uint16))),
}
_ORIG_BF16 = R.bf16_to_f64


def test_unmutated_oracle_passes_quick_pins():
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(R, attr, fn)
    with np.errstate(all="ignore"):
        assert not _pins_pass(), f"planted mistake {name} was not caught"
