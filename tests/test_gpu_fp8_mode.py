"""GPU parity of the fp8 compute mode (compute_mode = 1), through the C ABI.

The mode is an approximation: q is rounded to e4m3fn per (token, head). It runs on the
narrow kernel's fp8 instance when a token's list spans two or more tiles of 64 (every head
count, 32 heads per work item) and on the fp8qk kernel for a single tile; the test hook
SMLA_TEST_PREFILL_KERNEL=wide keeps every shape on the fp8qk kernel. Its oracle
(oracle/fp8mode.py) is the exact attention with that rounded q, and the kernel is held to
the bf16 mode's gate against it (max 2e-2, mean 2e-3): the fp8 rows enter the fp8 MFMA
exactly, and P and the output are bf16 as in the bf16 mode. lse is checked against
1e-5 (1 + |lse|) plus 2^-16 sm_scale max_j sum_d |q'_d r_jd| for the logit sums (the fp8
MFMA's accumulation was measured at about 2^-19 of that sum on a single-row case) plus
n 2^-24 for the fp32 sum of the n exponentials.

Against the exact oracle the rounding of q costs accuracy: an element of q moves by up to
max(2^-4 |q_d|, qs 2^-10). On the large prefill (2048 keys per token) the result still
meets the 2e-2 / 2e-3 gate against the exact oracle, which is asserted there; on few-key
cases it does not (max up to 5e-2, mean up to 7e-3 measured), so those are checked against
the fp8-mode oracle only. The bf16 mode stays the default.
"""
from __future__ import annotations

import copy

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

MAX_TOL, MEAN_TOL = 2e-2, 2e-3


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_top_mla_prefill_amd as smla
    return smla


def run_fp8(p, form="prefill"):
    smla = _gpu()
    from workloads.device import to_device
    d = to_device(p)
    o = d.new_out()
    L = torch.full((p.T, p.h), float("nan"), device="cuda")
    fn = smla.sparse_mla_forward if form == "forward" else smla.sparse_mla_prefill
    fn(d.q, d.kv, d.indices, d.sm_scale, out=o, lse=L, compute_mode=smla.SMLA_COMPUTE_FP8,
       **d.kwargs())
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), L.cpu().numpy()


def oracle(p, tokens=None):
    from oracle.fp8mode import sparse_mla_reference_fp8q
    return sparse_mla_reference_fp8q(p, tokens)


def exact_oracle(p, tokens=None):
    from oracle import sparse_mla_reference
    return sparse_mla_reference(p, tokens)


def lse_bound_fp8(p, tokens=None):
    from oracle.fp8mode import dequantized_q
    from oracle.reference import gather_token
    toks = np.arange(p.T) if tokens is None else np.asarray(tokens)
    out = np.zeros((len(toks), p.h))
    for i, t in enumerate(toks):
        rows = gather_token(p, int(t))
        q = np.abs(dequantized_q(p.q_bits[t]))
        if rows.shape[0]:
            # logit sums (the fp8 MFMA's accumulation: a single-row case measured 2^-19 of
            # sm_scale sum |q' r|; 2^-16 allowed), and the fp32 sum of n exponentials
            out[i] = (2.0 ** -16 * p.sm_scale * (q @ np.abs(rows).T).max(axis=1)
                      + rows.shape[0] * 2.0 ** -24)
    return out


def check(o, L, ro, rl, bound, what):
    diff = np.abs(o.astype(np.float64) - ro)
    assert not np.isnan(o).any(), what
    assert diff.max() <= MAX_TOL and diff.mean() <= MEAN_TOL, \
        f"{what}: max {diff.max():.3e} mean {diff.mean():.3e}"
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(L), np.isneginf(rl)), what
    err = np.abs(L - np.where(fin, rl, 0.0))
    tol = bound + 1e-5 * (1.0 + np.abs(rl))
    assert not (fin & (err > tol)).any(), f"{what}: lse err {err[fin].max():.3e}"


CASES = [
    # T, h, topk, sink, invalid, lengths
    (1, 1, 32, "normal", 0.0, False),
    (3, 16, 64, "none", 0.3, False),
    (2, 32, 100, "normal", 0.1, False),
    (4, 33, 256, "neginf", 0.2, False),
    (3, 64, 512, "normal", 0.1, True),
    (2, 128, 300, "normal", 1.0, False),
    (5, 80, 1000, "normal", 0.05, True),
]


@pytest.mark.parametrize("kernel", ["default", "fp8qk"])
@pytest.mark.parametrize("k", range(len(CASES)))
def test_fp8_mode_small(k, kernel, monkeypatch):
    from workloads import small_problem
    if kernel == "fp8qk":
        monkeypatch.setenv("SMLA_TEST_PREFILL_KERNEL", "wide")
    T, h, topk, sink, invalid, lengths = CASES[k]
    p = small_problem(seed=1800 + k, T=T, h=h, topk=topk, dtype="fp8", sink=sink,
                      invalid=invalid, out_of_range=2, num_pages=max(2, topk // 32),
                      lengths=lengths, layout=["inline", "footer", "separate"][k % 3])
    print(f"fp8 mode {CASES[k]} {kernel}", flush=True)
    o, L = run_fp8(p, "forward" if k % 2 else "prefill")
    ro, rl = oracle(p)
    check(o, L, ro, rl, lse_bound_fp8(p), f"fp8 mode {CASES[k]}")


def test_fp8_mode_head_prefix_bitwise():
    # q is quantised per head, so a head's result does not depend on the others.
    from workloads import small_problem
    p = small_problem(seed=1850, T=3, h=64, topk=256, dtype="fp8", invalid=0.2, num_pages=8)
    o, L = run_fp8(p)
    for hp in (40, 17, 1):
        q = copy.deepcopy(p)
        q.h, q.q_bits, q.attn_sink = hp, p.q_bits[:, :hp].copy(), p.attn_sink[:hp].copy()
        o2, L2 = run_fp8(q)
        assert np.array_equal(o[:, :hp], o2) and np.array_equal(L[:, :hp], L2), hp


def test_fp8_mode_large_prefill_sampled():
    from workloads import WORKLOADS
    p = WORKLOADS["prefill_large"]()
    o, L = run_fp8(p)
    rng = np.random.default_rng(19)
    toks = np.sort(rng.choice(p.T, size=48, replace=False))
    ro, rl = oracle(p, toks)
    check(o[toks], L[toks], ro, rl, lse_bound_fp8(p, toks), "fp8 mode prefill_large")
    eo, _ = exact_oracle(p, toks)
    diff = np.abs(o[toks].astype(np.float64) - eo)
    print(f"fp8 mode against the exact oracle: max {diff.max():.3e} mean {diff.mean():.3e}")
    assert diff.max() <= MAX_TOL and diff.mean() <= MEAN_TOL


def test_fp8_mode_tp2_prefill_sampled():
    from workloads import WORKLOADS
    p = WORKLOADS["prefill_tp2"]()
    o, L = run_fp8(p)
    rng = np.random.default_rng(21)
    toks = np.sort(rng.choice(p.T, size=256, replace=False))
    ro, rl = oracle(p, toks)
    check(o[toks], L[toks], ro, rl, lse_bound_fp8(p, toks), "fp8 mode prefill_tp2")


def test_fp8_mode_envelope_errors():
    smla = _gpu()
    from workloads import small_problem
    from workloads.device import to_device
    fp8 = smla.SMLA_COMPUTE_FP8
    p = small_problem(seed=1860, T=2, h=8, topk=64, dtype="bf16", num_pages=2)
    d = to_device(p)
    with pytest.raises(smla.SparseMLAError, match="compute_mode=1"):
        smla.sparse_mla_prefill(d.q, d.kv, d.indices, d.sm_scale, compute_mode=fp8)
    p = small_problem(seed=1861, T=2, h=8, topk=64, dtype="fp8", num_pages=2)
    d = to_device(p)
    with pytest.raises(smla.SparseMLAError, match="prefill and routed forms"):
        smla.sparse_mla_decode(d.q, d.kv, d.indices, d.sm_scale, compute_mode=fp8)
