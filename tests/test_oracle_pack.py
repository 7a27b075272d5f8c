"""Pins for the CPU oracle of the fp8 packing step (oracle/pack.py).

* the e4m3fn rounding against torch's float8_e4m3fn cast (a library routine) on random
  values, on every midpoint between adjacent codes and on signed zeros;
* hand-derived codes and scales of one row (tests/golden/pack_cases.json);
* properties: each group's largest magnitude lands on +-448, the round trip through an
  independent byte decoder (oracle/brute.py) stays within half an e4m3fn step, and slots
  outside the pool are left alone;
* planted mistakes in the oracle each fail at least one of these pins.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import oracle.pack as PK
from oracle import brute
from oracle.reference import e4m3fn_table
from workloads import synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack_cases.json")


def torch_e4m3(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def midpoints() -> np.ndarray:
    tab = e4m3fn_table()
    fin = np.unique(tab[~np.isnan(tab)])
    mids = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)
    return mids[np.abs(mids) <= 448]


rows = S.draw_pack_rows


# below this group maximum 448 / amax overflows fp32 and the multiplier is clamped
TINY = 448.0 / float(np.finfo(np.float32).max)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------- rounding
def test_nearest_even_matches_torch():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(-448, 448, 400), rng.uniform(-0.02, 0.02, 200),
                        midpoints(), -midpoints(), [0.0, -0.0, 448.0, -448.0, 1e-30, -1e-30]])
    v = v.astype(np.float32)
    assert np.array_equal(PK.e4m3fn_nearest_even(v), torch_e4m3(v))


# --------------------------------------------------------------------------- golden
def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["groups"]


def test_golden_row():
    x = np.zeros(576, np.float32)
    for g in _golden():
        for d, val in g["values"].items():
            x[int(d)] = val
    codes, scales = PK.quantize_row(S.to_bf16_bits(x))
    expect_scale = {"2^-6": np.float32(2.0 ** -6), "0": np.float32(0.0),
                    "fl32(1/448)": np.float32(1.0) / np.float32(448.0)}
    for gi, g in enumerate(_golden()):
        for d, c in g["codes"].items():
            assert codes[int(d)] == int(c, 16), (d, hex(codes[int(d)]), c)
        assert scales[gi] == expect_scale[g["scale"]], (gi, scales[gi])
    assert np.all(codes[192:] == 0) and np.all(scales[3:] == 0)


# --------------------------------------------------------------------------- properties
def test_group_max_lands_on_448():
    r = rows(5, 6)
    for i in range(r.shape[0]):
        codes, scales = PK.quantize_row(r[i])
        x = bf16_values(r[i])
        for g in range(9):
            xs = x[64 * g:64 * g + 64]
            amax = float(np.max(np.abs(xs)))
            if amax == 0:
                assert scales[g] == 0
                continue
            if amax < TINY:  # the multiplier is clamped there (row 2's group 3)
                continue
            j = int(np.argmax(np.abs(xs)))
            assert codes[64 * g + j] == (0xFE if xs[j] < 0 else 0x7E)
            assert abs(448.0 * float(scales[g]) - amax) <= amax * 2.0 ** -23


def _fp8_pool(layout: str, num_pages: int = 3, d_qk: int = 576, seed: int = 9):
    return S.draw_pool(np.random.default_rng(seed), "fp8", d_qk, num_pages, layout)


@pytest.mark.parametrize("layout,d_qk", [("inline", 576), ("footer", 576), ("separate", 1088)])
def test_round_trip_within_half_step(layout, d_qk):
    pool = _fp8_pool(layout, d_qk=d_qk)
    r = rows(11, 10, d_qk)
    slots = np.array([5, 64, 130, 0, 191, 77, 78, 12, 150, 33])
    PK.pack_kv_reference(r, slots, pool)
    for i, s in enumerate(slots):
        got = np.array(brute._row(pool, int(s)))  # independent byte decoder
        x = bf16_values(r[i]).astype(np.float64)
        _, scales = PK.quantize_row(r[i])
        sc = np.repeat(scales.astype(np.float64), 64)
        # half an e4m3fn step: 2^-4 relative for normal codes, 2^-10 * scale below 2^-6
        bound = np.maximum(np.abs(x) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 2.0 ** -20)
        ok = np.abs(got - x) <= bound
        amax = np.repeat(np.abs(x).reshape(-1, 64).max(axis=1), 64)
        assert np.all(ok | (amax < TINY)), (layout, i)


@pytest.mark.parametrize("layout", ["inline", "separate"])
def test_skipped_slots_leave_the_pool_alone(layout):
    pool = _fp8_pool(layout)
    before_d, before_s = pool.data.copy(), pool.scales.copy()
    r = rows(13, 5)
    slots = np.array([-1, pool.num_pages * 64, 2**31 - 1, 7, -7])
    PK.pack_kv_reference(r, slots, pool)
    # only slot 7 (page 0, offset 7) changes: its payload, and its scales
    changed = np.flatnonzero(pool.data != before_d)
    base = pool.data_offset + 7 * pool.row_stride
    assert changed.size and changed.min() >= base and changed.max() < base + pool.row_stride
    if pool.scales is not pool.data:
        sch = np.flatnonzero(pool.scales != before_s)
        sbase = pool.scale_offset + 7 * pool.scale_row_stride
        assert sch.size and sch.min() >= sbase and sch.max() < sbase + 4 * 9


# --------------------------------------------------------------------------- planted mistakes
def _pins_pass() -> bool:
    try:
        test_nearest_even_matches_torch()
        test_golden_row()
        test_group_max_lands_on_448()
        test_round_trip_within_half_step("inline", 576)
    except AssertionError:
        return False
    return True


def _ties_away_from_zero(v):
    # mistake: a value halfway between two codes takes the one of larger magnitude
    out = _ORIG_NEAREST(v).astype(np.int64)
    tab = e4m3fn_table()
    vv = np.asarray(v, np.float64)
    mid = np.isin(np.abs(vv), midpoints().astype(np.float64))
    return np.where(mid & (np.abs(tab[out]) < np.abs(vv)), out + 1, out).astype(np.uint8)


def _no_signed_zero(v):
    out = _ORIG_NEAREST(v)
    return np.where(out == 0x80, 0, out).astype(np.uint8)


_ORIG_NEAREST = PK.e4m3fn_nearest_even

MUTATIONS = {
    "max_240": ("E4M3_MAX", 240.0),
    "group_32": ("GROUP", 32),
    "ties_away_from_zero": ("e4m3fn_nearest_even", _ties_away_from_zero),
    "zero_sign_dropped": ("e4m3fn_nearest_even", _no_signed_zero),
}


def test_unmutated_pack_oracle_passes_pins():
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_pack_mistake_is_caught(name, monkeypatch):
    attr, val = MUTATIONS[name]
    monkeypatch.setattr(PK, attr, val)
    with np.errstate(all="ignore"):
        assert not _pins_pass(), f"planted mistake {name} was not caught"
