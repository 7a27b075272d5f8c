"""GPU test of sparse_mla_decode_noalloc, the decode form whose split-K partials live in the
library's per-device scratch instead of a caller's workspace.

It runs the same plan and kernels as sparse_mla_decode, so its output must equal that entry
point's bit for bit (stricter than the 2e-2 / 2e-3 gate against the oracle, which it also
meets). Two calls in a row, the second with a smaller input, show that the scratch left by
one call does not leak into the next. Both calls split (their workspace size is non-zero),
so the scratch is really used.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_top_mla_prefill_amd as smla
    return smla


def _call_pair(smla, p):
    from workloads.device import to_device
    d = to_device(p)
    need = smla.sparse_mla_workspace_size(d.q, d.kv, d.indices, d.sm_scale, d.new_out(), True,
                                          **d.kwargs())
    assert need > 0, "the case must split, so that the scratch is used"
    ref_o, ref_l = d.new_out(), torch.empty(p.T, p.h, device="cuda")
    smla.sparse_mla_decode(d.q, d.kv, d.indices, d.sm_scale, out=ref_o, lse=ref_l,
                           **d.kwargs())
    o = torch.full_like(ref_o, float("nan"))
    lse = torch.full_like(ref_l, float("nan"))
    smla.sparse_mla_decode_noalloc(d.q, d.kv, d.indices, d.sm_scale, o, lse=lse,
                                   **d.kwargs())
    torch.cuda.synchronize()
    return o, lse, ref_o, ref_l


def test_noalloc_matches_decode_twice_shrinking():
    smla = _gpu()
    from oracle import sparse_mla_reference
    from workloads import small_problem
    big = small_problem(seed=4100, T=12, h=64, topk=1024, dtype="fp8", num_pages=20,
                        sink="normal", invalid=0.1)
    small = small_problem(seed=4101, T=3, h=20, topk=448, dtype="fp8", num_pages=8,
                          sink="normal", invalid=0.2, extra_dtype="bf16", topk_extra=64,
                          extra_pages=2)
    for name, p in (("first", big), ("second, smaller", small)):
        print(f"noalloc {name}: T={p.T} h={p.h} topk={p.topk}", flush=True)
        o, lse, ref_o, ref_l = _call_pair(smla, p)
        assert torch.equal(o, ref_o), name
        assert torch.equal(lse, ref_l), name
        ro, _ = sparse_mla_reference(p)
        err = np.abs(o.float().cpu().numpy().astype(np.float64) - ro)
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, (name, err.max(), err.mean())


def test_noalloc_needs_out_and_zero_tokens():
    smla = _gpu()
    from workloads import small_problem
    from workloads.device import to_device
    p = small_problem(seed=4102, T=2, h=8, topk=128, dtype="fp8", num_pages=4)
    d = to_device(p)
    with pytest.raises(TypeError):
        smla.sparse_mla_decode_noalloc(d.q, d.kv, d.indices, d.sm_scale, None)
    out = d.new_out()[:0]
    smla.sparse_mla_decode_noalloc(d.q[:0], d.kv, d.indices[:0], d.sm_scale, out)
