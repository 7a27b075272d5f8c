"""GPU parity of the packing kernel (sparse_mla_pack_kv) against the CPU oracle, through
the C ABI.

The packed bytes are integer results decided in fp32, by the same IEEE fp32 operations in
kernel and oracle: per group of 64 the scale fl32(amax / 448) and the multiplier
min(fl32(448 / amax), FLT_MAX), and per element the code nearest to clamp(fl32(x * m), +-448).
So the bar is bit-exact: the whole pool buffer after the kernel equals the oracle's,
untouched slots included.
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


def _slots(rng, num_slots: int, n: int) -> np.ndarray:
    """n distinct slots of the pool, with a few skipped entries (-1, past the end, huge)."""
    s = rng.permutation(num_slots)[:n].astype(np.int64)
    for j, bad in zip(rng.choice(n, size=min(n, 4), replace=False),
                      (-1, num_slots, 2**31 - 1, -(2**31))):
        s[j] = bad
    return s.astype(np.int32)


@pytest.mark.parametrize("layout,d_qk,n", [("inline", 576, 300), ("footer", 576, 257),
                                           ("separate", 1088, 130), ("inline", 1088, 64),
                                           ("separate", 576, 1), ("footer", 576, 512)])
def test_pack_bitwise(layout, d_qk, n):
    smla = _gpu()
    from oracle.pack import pack_kv_reference
    from workloads import synth as S
    from workloads.device import pool_to_device
    rng = np.random.default_rng(2000 + n + d_qk)
    pool = S.draw_pool(rng, "fp8", d_qk, 8, layout)
    rows = S.draw_pack_rows(3000 + n, n, d_qk)
    slots = _slots(rng, pool.num_slots, n)
    dev = pool_to_device(pool, "cuda")
    print(f"pack {layout} d_qk={d_qk} n={n}", flush=True)
    smla.sparse_mla_pack_kv(
        torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16).cuda(),
        torch.from_numpy(slots).cuda(), dev)
    torch.cuda.synchronize()
    pack_kv_reference(rows, slots, pool)
    assert np.array_equal(dev.data.cpu().numpy(), pool.data)
    if dev.scales is not None and dev.scales is not dev.data:
        assert np.array_equal(dev.scales.cpu().numpy(), pool.scales)


def test_pack_then_attend():
    # The packed pool is what the attention path reads: attention over the GPU-packed pool
    # matches the oracle's attention over the oracle-packed pool.
    smla = _gpu()
    from oracle import sparse_mla_reference
    from oracle.pack import pack_kv_reference
    from workloads import synth as S
    from workloads.device import to_device
    p = S.small_problem(seed=2100, T=4, h=64, topk=256, dtype="fp8", num_pages=8, invalid=0.1)
    # N(0,1) rows (no per-group spread), the magnitudes the attention tolerance is set for
    rows = S.draw_pack_rows(2101, p.kv.num_slots, 576, spread=0.0)
    slots = np.arange(p.kv.num_slots, dtype=np.int32)
    d = to_device(p)
    smla.sparse_mla_pack_kv(torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16).cuda(),
                            torch.from_numpy(slots).cuda(), d.kv)
    pack_kv_reference(rows, slots, p.kv)
    out = d.new_out()
    smla.sparse_mla_prefill(d.q, d.kv, d.indices, d.sm_scale, out=out, **d.kwargs())
    torch.cuda.synchronize()
    ref, _ = sparse_mla_reference(p)
    err = np.abs(out.float().cpu().numpy() - ref)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())


def test_pack_full_decode_pool_sampled():
    # The benchmark's pack: every slot of the decode workload's pool (32 x 18432 rows of
    # 576, fp8 inline), rows N(0,1) in bf16 from a seeded device generator, slots in a
    # random order. 256 sampled rows are checked bit-exactly against the oracle.
    smla = _gpu()
    from oracle.pack import quantize_row
    from workloads import synth as S
    from workloads.device import pool_to_device
    n = 32 * 18432
    pool = S.pack_pool(np.zeros((n, 576), np.uint8), np.ones((n, 9), np.float32), "fp8", 576)
    dev = pool_to_device(pool, "cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(2200)
    rows = torch.randn(n, 576, device="cuda", generator=g).to(torch.bfloat16)
    slots = torch.randperm(n, device="cuda", generator=g).to(torch.int32)
    smla.sparse_mla_pack_kv(rows, slots, dev)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2201)
    pick = rng.choice(n, size=256, replace=False)
    data = dev.data.cpu().numpy()
    sl = slots.cpu().numpy()
    rbits = rows[torch.from_numpy(pick).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
    for k, r in enumerate(pick):
        codes, scales = quantize_row(rbits[k])
        s = int(sl[r])
        base = pool.data_offset + (s // 64) * pool.page_stride + (s % 64) * pool.row_stride
        assert np.array_equal(data[base:base + 576], codes), r
        sbase = pool.scale_offset + (s // 64) * pool.scale_page_stride + (s % 64) * pool.scale_row_stride
        assert np.array_equal(data[sbase:sbase + 36].view("<f4"), scales), r


def test_pack_errors():
    smla = _gpu()
    from workloads import synth as S
    from workloads.device import pool_to_device
    bf = pool_to_device(S.draw_pool(np.random.default_rng(1), "bf16", 576, 2), "cuda")
    rows = torch.zeros(3, 576, dtype=torch.bfloat16, device="cuda")
    slots = torch.zeros(3, dtype=torch.int32, device="cuda")
    with pytest.raises(smla.SparseMLAError, match="packing writes fp8 pools only"):
        smla.sparse_mla_pack_kv(rows, slots, bf)
    f8 = pool_to_device(S.draw_pool(np.random.default_rng(2), "fp8", 576, 2), "cuda")
    smla.sparse_mla_pack_kv(rows[:0], slots[:0], f8)  # n = 0: a no-op
