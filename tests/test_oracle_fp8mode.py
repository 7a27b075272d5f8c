"""Pins for the CPU oracle of the fp8 compute mode (oracle/fp8mode.py).

* a special case that reduces to the exact oracle: q rows already on the e4m3fn grid of
  their own scale (a power of two, largest magnitude 448 times it) round to themselves, so
  the fp8-mode result equals oracle.reference bit for bit;
* the rounding of q against torch's float8_e4m3fn cast of the scaled values (a library
  routine), and each head's largest magnitude landing on +-448;
* the rounding error bound |q' - q| <= max(2^-4 |q|, qs 2^-10) element by element;
* planted mistakes in the oracle each fail at least one of these pins.
"""
from __future__ import annotations

import copy

import numpy as np
import pytest
import torch

import oracle.fp8mode as F
from oracle.reference import bf16_to_f64, e4m3fn_table, sparse_mla_reference
from workloads import synth as S


def _on_grid_problem(seed):
    """q rows whose values are e4m3fn values times 2^-k_h, with one element per head at
    448 * 2^-k_h (so amax / 448 = 2^-k_h exactly)."""
    p = S.small_problem(seed=seed, T=3, h=5, topk=128, dtype="fp8", invalid=0.1, num_pages=4)
    rng = np.random.default_rng(seed)
    tab = e4m3fn_table()
    finite = np.flatnonzero(~np.isnan(tab) & (np.abs(tab) <= 448))
    codes = rng.choice(finite, size=(p.T, p.h, p.d_qk))
    codes[:, :, 0] = 0x7E  # 448
    k = rng.integers(2, 9, size=(p.T, p.h, 1))
    q = (tab[codes] * np.exp2(-k.astype(np.float64))).astype(np.float32)
    p.q_bits = S.to_bf16_bits(q)
    assert np.array_equal(bf16_to_f64(p.q_bits), q.astype(np.float64))  # exact in bf16
    return p


def test_on_grid_q_equals_exact_oracle():
    p = _on_grid_problem(41)
    a = F.sparse_mla_reference_fp8q(p)
    b = sparse_mla_reference(p)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_q_codes_match_torch_and_max_lands_on_448():
    p = S.small_problem(seed=42, T=4, h=7, topk=64, dtype="fp8")
    codes, qs = F.quantize_q_rows(p.q_bits)
    x = bf16_to_f64(p.q_bits).astype(np.float32)
    amax = np.abs(x).max(axis=-1, keepdims=True)
    inv = (np.float32(448) / amax).astype(np.float32)
    v = np.clip((x * inv).astype(np.float32), -448, 448)
    t = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, t)
    j = np.abs(x).argmax(axis=-1)
    top = np.take_along_axis(codes, j[..., None], axis=-1)[..., 0]
    assert np.all((top == 0x7E) | (top == 0xFE))
    assert np.array_equal(qs, (amax / np.float32(448)).astype(np.float32))


def test_q_rounding_error_bound():
    p = S.small_problem(seed=43, T=3, h=9, topk=64, dtype="fp8")
    q = bf16_to_f64(p.q_bits)
    qd = F.dequantized_q(p.q_bits)
    _, qs = F.quantize_q_rows(p.q_bits)
    bound = np.maximum(np.abs(q) * 2.0 ** -4, qs.astype(np.float64) * 2.0 ** -10) * (1 + 2 ** -20)
    assert np.all(np.abs(qd - q) <= bound)
    assert not np.array_equal(qd, q)  # the mode really rounds


# --------------------------------------------------------------------------- planted mistakes
def _pins_pass() -> bool:
    try:
        test_on_grid_q_equals_exact_oracle()
        test_q_codes_match_torch_and_max_lands_on_448()
        test_q_rounding_error_bound()
    except AssertionError:
        return False
    return True


_ORIG_Q = F.quantize_q_rows


def _per_token_amax(q_bits):
    # mistake: one scale per token (over all heads) instead of per (token, head)
    x = bf16_to_f64(q_bits).astype(np.float32)
    amax = np.max(np.abs(x), axis=(-2, -1), keepdims=True) * np.ones(x.shape[:-1] + (1,), np.float32)
    qs = (amax / np.float32(448)).astype(np.float32)
    v = np.clip((x * (np.float32(448) / amax)).astype(np.float32), -448, 448)
    return F.e4m3fn_nearest_even(v), qs


def _scale_240(q_bits):
    codes, qs = _ORIG_Q(q_bits)
    return codes, (qs * np.float32(448 / 240)).astype(np.float32)


MUTATIONS = {"per_token_amax": _per_token_amax, "scale_240": _scale_240}


def test_unmutated_fp8mode_oracle_passes_pins():
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_fp8mode_mistake_is_caught(name, monkeypatch):
    monkeypatch.setattr(F, "quantize_q_rows", MUTATIONS[name])
    with np.errstate(all="ignore"):
        assert not _pins_pass(), name
