"""C-ABI tests that need no GPU: the library loads and exports every declared symbol.

Every host-side validation path fails with the documented status and message before any
HIP call, so these run on a machine without a GPU. The envelope query matches what the
entry points accept. No test here launches a kernel.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from sparse_top_mla_prefill_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_mla.h")

FAKE = 0x7F0000000000  # an aligned fake device address; validation never dereferences it


def declared_functions() -> list[str]:
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char \*)\s*(sparse_mla_\w+)\s*\(", text,
                                 re.M)))


def test_header_declares_the_bound_functions():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version():
    assert B.sparse_mla_abi_version() == 2


def test_supported_configs():
    cfgs = B.sparse_mla_supported_configs()
    assert len(cfgs) == 12
    geos = {(c["d_qk"], c["d_v"]) for c in cfgs}
    assert geos == {(576, 512), (1088, 1024)}
    for c in cfgs:
        assert (c["min_h"], c["max_h"], c["topk_multiple"], c["page_block_size"],
                c["decode_max_tokens"]) == (1, 128, 1, 64, 64)
        assert c["kv_dtype"] in (0, 1) and c["extra_kv_dtype"] in (-1, 0, 1)
    count = ctypes.c_int(0)
    assert B.LIB.sparse_mla_supported_configs(None, 0, ctypes.byref(count)) == 0
    assert count.value == 12
    assert B.LIB.sparse_mla_supported_configs(None, 3, ctypes.byref(count)) == B.SMLA_ERR_INVALID


def _pool(dtype=B.SMLA_FP8_E4M3_G64, d_qk=576, num_pages=16):
    c = B.smla_cache()
    c.data = FAKE
    c.dtype = dtype
    c.page_block_size = 64
    c.num_pages = num_pages
    if dtype == B.SMLA_FP8_E4M3_G64:
        c.row_stride = ((d_qk + 4 * (d_qk // 64) + 63) // 64) * 64
        c.scales = FAKE + d_qk
        c.scale_row_stride = c.row_stride
    else:
        c.row_stride = 2 * d_qk
    c.page_stride = 64 * c.row_stride
    c.scale_page_stride = c.page_stride
    return c


def good_args(T=4, h=16, topk=128, d_qk=576, d_v=512, topk_extra=0, extra_dtype=None):
    a = B.smla_args()
    a.T, a.h, a.d_qk, a.d_v = T, h, d_qk, d_v
    a.q = FAKE
    a.q_stride_h = d_qk
    a.q_stride_t = h * d_qk
    a.kv = _pool(d_qk=d_qk)
    a.indices = FAKE
    a.topk = topk
    a.indices_stride = topk
    if topk_extra:
        a.extra = _pool(dtype=extra_dtype, d_qk=d_qk)
        a.extra_indices = FAKE
        a.topk_extra = topk_extra
        a.extra_indices_stride = topk_extra
    a.attn_sink = FAKE
    a.sm_scale = 1.0 / 24
    a.out = FAKE
    a.out_stride_h = d_v
    a.out_stride_t = h * d_v
    a.lse = FAKE
    a.lse_stride_t = h
    return a


def ws_status(a, decode=False):
    n = ctypes.c_size_t(0)
    rc = B.LIB.sparse_mla_workspace_size(ctypes.byref(a), int(decode), ctypes.byref(n))
    return rc, n.value, B.LIB.sparse_mla_last_error().decode()


def test_valid_args_pass_validation():
    for decode in (False, True):
        rc, n, msg = ws_status(good_args(), decode)
        assert rc == B.SMLA_OK, msg
    assert ws_status(good_args(), False)[1] == 0
    assert ws_status(good_args(T=32, h=64, topk=512), True)[1] > 0


def test_decode_plan_keeps_decode_kernel_within_one_round():
    # The decode form takes the decode kernel (16 heads per workgroup, chunks of at most 4
    # tiles of 64) while its work items, T x ceil(h / 16) x chunks, fit one round of
    # workgroups (256 CUs without a device); larger plans take the wide kernels' split model,
    # whose chunk count differs here. Read from the workspace sizes: partials of 512 bf16 and
    # (m, l) per (token, head, chunk), heads padded to 16 in the decode kernel.
    def ws16(T, h, nc):
        rows = T * -(-h // 16) * 16 * nc
        return -(-rows * 512 * 2 // 256) * 256 + rows * 8

    assert ws_status(good_args(T=4, h=128, topk=2048), True)[1] == ws16(4, 128, 8)
    assert ws_status(good_args(T=32, h=64, topk=512), True)[1] == ws16(32, 64, 2)
    for T, h, topk in ((64, 128, 2048), (48, 64, 512), (24, 128, 512)):
        n = ws_status(good_args(T=T, h=h, topk=topk), True)[1]
        assert n > 0 and n != ws16(T, h, -(-topk // 256)), (T, h, topk, n)


def mutate(**changes):
    a = good_args(**changes.pop("base", {}))
    for k, v in changes.items():
        obj = a
        parts = k.split(".")
        for p in parts[:-1]:
            obj = getattr(obj, p)
        setattr(obj, parts[-1], v)
    return a


FAILURES = [
    # (mutation, expected status, message fragment)
    (dict(h=0), B.SMLA_ERR_UNSUPPORTED, "num_heads=0 outside [1,128]"),
    (dict(h=200), B.SMLA_ERR_UNSUPPORTED, "num_heads=200 outside [1,128]"),
    (dict(topk=0), B.SMLA_ERR_UNSUPPORTED, "topk=0 must be >= 1"),
    (dict(topk=-64), B.SMLA_ERR_UNSUPPORTED, "topk=-64 must be >= 1"),
    (dict(topk=(1 << 24) + 1, indices_stride=(1 << 24) + 1), B.SMLA_ERR_UNSUPPORTED,
     "topk + topk_extra = 16777217 exceeds 16777216"),
    (dict(topk_length=FAKE + 2), B.SMLA_ERR_INVALID, "topk_length / extra_topk_length must be"),
    (dict(base=dict(topk_extra=64, extra_dtype=B.SMLA_BF16), extra_topk_length=FAKE + 1),
     B.SMLA_ERR_INVALID, "4-byte aligned"),
    (dict(d_qk=512, d_v=512), B.SMLA_ERR_UNSUPPORTED, "(576, 512), (1088, 1024)"),
    (dict(d_v=1024), B.SMLA_ERR_UNSUPPORTED, "(d_qk, d_v)=(576, 1024)"),
    (dict(T=-1), B.SMLA_ERR_INVALID, "T=-1"),
    (dict(sm_scale=0.0), B.SMLA_ERR_INVALID, "sm_scale"),
    (dict(sm_scale=float("nan")), B.SMLA_ERR_INVALID, "sm_scale"),
    (dict(q=None), B.SMLA_ERR_INVALID, "q is NULL"),
    (dict(q=FAKE + 2), B.SMLA_ERR_INVALID, "q must be 16-byte aligned"),
    (dict(q_stride_h=577), B.SMLA_ERR_INVALID, "multiples of 8"),
    (dict(indices=None), B.SMLA_ERR_INVALID, "indices is NULL"),
    (dict(indices_stride=64), B.SMLA_ERR_INVALID, "indices_stride=64 must be >= topk=128"),
    (dict(out=None), B.SMLA_ERR_INVALID, "out is NULL"),
    (dict(out=FAKE + 2), B.SMLA_ERR_INVALID, "out must be 8-byte aligned"),
    (dict(lse_stride_t=3), B.SMLA_ERR_INVALID, "lse_stride_t=3 must be >= num_heads=16"),
    (dict(**{"kv.page_block_size": 32}), B.SMLA_ERR_UNSUPPORTED,
     "kv page_block_size=32 is not supported (supported: 64)"),
    (dict(**{"kv.dtype": 7}), B.SMLA_ERR_UNSUPPORTED, "kv dtype=7"),
    (dict(**{"kv.data": None}), B.SMLA_ERR_INVALID, "kv data is NULL"),
    (dict(**{"kv.data": FAKE + 8}), B.SMLA_ERR_INVALID, "kv data is not 16-byte aligned"),
    (dict(**{"kv.num_pages": 0}), B.SMLA_ERR_INVALID, "kv num_pages=0"),
    (dict(**{"kv.row_stride": 1024}), B.SMLA_ERR_INVALID, "kv page_stride=40960"),
    (dict(**{"kv.row_stride": 520}), B.SMLA_ERR_INVALID, "kv row_stride=520"),
    (dict(**{"kv.page_stride": 640 * 63}), B.SMLA_ERR_INVALID,
     "page_stride=40320 must be a multiple of 16 and >= page_block_size * row_stride = 40960"),
    (dict(**{"kv.scales": None}), B.SMLA_ERR_INVALID, "kv scales is NULL"),
    (dict(**{"kv.scales": FAKE + 2}), B.SMLA_ERR_INVALID, "kv scales is not 4-byte aligned"),
    (dict(**{"kv.scale_row_stride": 32}), B.SMLA_ERR_INVALID, "scale_row_stride=32"),
    (dict(**{"kv.scale_page_stride": 640}), B.SMLA_ERR_INVALID, "scale_page_stride=640"),
    (dict(base=dict(topk_extra=64, extra_dtype=B.SMLA_BF16),
          **{"extra.page_block_size": 16}), B.SMLA_ERR_UNSUPPORTED,
     "extra page_block_size=16"),
    (dict(base=dict(topk_extra=64, extra_dtype=B.SMLA_BF16), extra_indices=None),
     B.SMLA_ERR_INVALID, "extra_indices is NULL"),
    (dict(base=dict(topk_extra=64, extra_dtype=B.SMLA_BF16), topk_extra=-1),
     B.SMLA_ERR_UNSUPPORTED, "topk_extra=-1 must be >= 0"),
    (dict(base=dict(topk_extra=64, extra_dtype=B.SMLA_BF16), extra_indices_stride=63),
     B.SMLA_ERR_INVALID, "extra_indices_stride=63 must be >= topk_extra=64"),
]


@pytest.mark.parametrize("mutation,status,fragment", FAILURES,
                         ids=[str(i) for i in range(len(FAILURES))])
def test_validation_failures(mutation, status, fragment):
    for decode, form in ((0, "prefill"), (1, "decode"), (2, "forward")):
        rc, _, msg = ws_status(mutate(**dict(mutation)), decode)
        assert rc == status, msg
        assert fragment in msg, msg
        if rc != B.SMLA_ERR_INVALID or "sparse-MLA:" not in msg:
            assert msg.startswith(f"Unsupported sparse-MLA {form} configuration: num_heads="), msg


def test_message_prefix_lists_the_call_shape():
    a = mutate(topk=320, indices_stride=320, h=200)
    rc, _, msg = ws_status(a)
    assert rc == B.SMLA_ERR_UNSUPPORTED
    assert msg.startswith("Unsupported sparse-MLA prefill configuration: num_heads=200 topk=320 "
                          "page_block_size=64 topk_extra=0 extra_page_block_size=0 d_qk=576 "
                          "d_v=512: num_heads=200 outside [1,128]")


def _chunks(a, form):
    """Index chunks per token of a form's plan, read back from its workspace size. The wide
    kernels' partials are [T][chunks][h][d_v] bf16 plus [T][chunks][h][2] fp32; the decode
    kernel's are the same per (token, group of 16 heads) with the heads padded to 16."""
    rc, n, msg = ws_status(a, form)
    assert rc == B.SMLA_OK, msg
    if n == 0:
        return 1
    per_chunk_row = a.d_v * 2  # bf16 O / l of one (token, chunk, head)
    for nc in range(2, 257):
        for rows in (a.T * nc * a.h, a.T * nc * 16 * -(-a.h // 16)):
            if -(-rows * per_chunk_row // 256) * 256 + rows * 8 == n:
                return nc
    raise AssertionError(f"workspace {n} matches no chunk count")


def test_decode_split_choices():
    # The decode kernel (fp8 pools at d_qk 576) holds a chunk of up to 4 index tiles in LDS
    # and takes the fewest chunks that fit, up to 8 (up to 2048 keys per token).
    for (T, h, topk), want in [((32, 64, 512), 2), ((24, 16, 2048), 8), ((1, 64, 128), 1),
                               ((64, 16, 128), 1), ((1, 64, 2048), 8), ((5, 100, 300), 2),
                               ((3, 8, 1000), 4)]:
        a = good_args(T=T, h=h, topk=topk)
        assert _chunks(a, 1) == want, (T, h, topk)
    # Past 8 chunks the plan is the wide kernels' (one tile per chunk here).
    assert _chunks(good_args(T=1, h=64, topk=4096), 1) == 64


def test_wide_decode_split_choices(monkeypatch):
    # Chunk counts the wide kernels' split model picks (the decode kernel switched off by its
    # test hook, as for bf16 pools and d_qk 1088):
    #   - the decode workload's shape: 8 chunks of one 64-key tile (256 work items);
    #   - 24 tokens of 32 index tiles: 8 chunks of 4 tiles (192 items), not 11 chunks of 3,
    #     whose 264 items would need a second round on 8 CUs;
    #   - two tiles per token: no split (the combine pass costs what the split saves);
    #   - one token of 32 tiles: one tile per chunk.
    monkeypatch.setenv("SMLA_TEST_DECODE_KERNEL", "wide")
    for (T, h, topk), want in [((32, 64, 512), 8), ((24, 16, 2048), 8), ((1, 64, 128), 1),
                               ((64, 16, 128), 1), ((1, 64, 2048), 32)]:
        a = good_args(T=T, h=h, topk=topk)
        assert _chunks(a, 1) == want, (T, h, topk)
    bf = good_args(T=32, h=64, topk=512)
    bf.kv = _pool(dtype=B.SMLA_BF16)
    monkeypatch.delenv("SMLA_TEST_DECODE_KERNEL")
    assert _chunks(bf, 1) == 8  # bf16 pools always take the wide kernels


@pytest.mark.parametrize("hook", [None, "wide"])
def test_decode_chunks_never_empty(hook, monkeypatch):
    if hook:
        monkeypatch.setenv("SMLA_TEST_DECODE_KERNEL", hook)
    for T in (1, 2, 3, 5, 8, 17, 24, 31, 48, 64):
        for h in (8, 32, 64, 100, 128):
            for topk in (128, 300, 512, 2048):
                a = good_args(T=T, h=h, topk=topk)
                nc = _chunks(a, 1)
                tiles = -(-topk // 64)
                assert 1 <= nc <= tiles
                assert -(-tiles // -(-tiles // nc)) == nc  # no empty chunk


def test_forward_routes_by_rows():
    # up to 64 rows the routed form plans like the decode form; above, like prefill
    for T in (1, 24, 64):
        a = good_args(T=T, h=64, topk=512)
        assert ws_status(a, 2)[:2] == ws_status(a, 1)[:2]
    for T in (65, 1000):
        a = good_args(T=T, h=64, topk=512)
        rc, n, msg = ws_status(a, 2)
        assert (rc, n) == (B.SMLA_OK, 0), msg
        assert ws_status(a, 1)[0] == B.SMLA_ERR_UNSUPPORTED
    rc, _, msg = ws_status(good_args(), 3)
    assert rc == B.SMLA_ERR_INVALID and "form=3" in msg


def test_decode_row_limit():
    rc, _, msg = ws_status(good_args(T=65), True)
    assert rc == B.SMLA_ERR_UNSUPPORTED and "exceeds the decode limit of 64" in msg
    assert ws_status(good_args(T=65), False)[0] == B.SMLA_OK
    assert ws_status(good_args(T=64), True)[0] == B.SMLA_OK


def test_zero_tokens_is_a_noop_without_device():
    a = good_args(T=0)
    a.q = a.out = a.indices = a.lse = None
    for fn in (B.LIB.sparse_mla_prefill, B.LIB.sparse_mla_decode, B.LIB.sparse_mla_forward):
        assert fn(ctypes.byref(a), None) == B.SMLA_OK
    assert ws_status(a, True)[:2] == (B.SMLA_OK, 0)


def test_decode_workspace_is_checked_before_the_device():
    a = good_args(T=8, h=64, topk=512)
    rc, need, _ = ws_status(a, True)
    assert rc == 0 and need > 0
    a.workspace, a.workspace_bytes = FAKE, need - 1
    assert B.LIB.sparse_mla_decode(ctypes.byref(a), None) == B.SMLA_ERR_WORKSPACE
    assert "smaller than" in B.sparse_mla_last_error()
    a.workspace, a.workspace_bytes = FAKE + 16, need
    assert B.LIB.sparse_mla_decode(ctypes.byref(a), None) == B.SMLA_ERR_WORKSPACE
    assert "256-byte aligned" in B.sparse_mla_last_error()


@pytest.mark.parametrize("cfg", B.sparse_mla_supported_configs(),
                         ids=lambda c: f"{c['d_qk']}-{c['kv_dtype']}-{c['extra_kv_dtype']}")
def test_envelope_matches_acceptance(cfg):
    """Every advertised envelope is accepted at its corners and rejected just outside."""
    d_qk, d_v = cfg["d_qk"], cfg["d_v"]
    ex = cfg["extra_kv_dtype"]
    for h in (cfg["min_h"], 7, 64, cfg["max_h"]):
        for topk in (1, 37, 64, 192, 500, 2048):
            a = good_args(T=3, h=h, topk=topk, d_qk=d_qk, d_v=d_v,
                          topk_extra=64 if ex >= 0 else 0, extra_dtype=max(ex, 0))
            a.kv = _pool(dtype=cfg["kv_dtype"], d_qk=d_qk)
            for decode in (False, True):
                rc, _, msg = ws_status(a, decode)
                assert rc == B.SMLA_OK, msg
    for bad in (dict(h=cfg["max_h"] + 1), dict(h=cfg["min_h"] - 1), dict(topk=0)):
        a = good_args(d_qk=d_qk, d_v=d_v, **{k: v for k, v in bad.items()})
        a.indices_stride = max(a.indices_stride, a.topk)
        assert ws_status(a)[0] == B.SMLA_ERR_UNSUPPORTED
    a = good_args(d_qk=d_qk, d_v=d_v, T=cfg["decode_max_tokens"] + 1)
    assert ws_status(a, True)[0] == B.SMLA_ERR_UNSUPPORTED


def test_ragged_widths_and_live_counts_are_accepted():
    # any positive width, a ragged extra width, and aligned live-count arrays
    for topk, topk_extra in ((1, 0), (500, 0), (37, 21), (64, 1)):
        a = good_args(T=5, h=64, topk=topk, topk_extra=topk_extra, extra_dtype=B.SMLA_BF16)
        a.topk_length = FAKE
        a.extra_topk_length = FAKE + 64
        for decode in (False, True):
            rc, n, msg = ws_status(a, decode)
            assert rc == B.SMLA_OK, msg
            tiles = -(-topk // 64) + -(-topk_extra // 64)  # a ragged tail is a whole tile
            assert n == 0 or (decode and tiles > 1), (topk, topk_extra, n)
            if decode and topk == 500:
                assert n > 0  # 8 tiles (the last one partial): split
    # without an extra list, extra_topk_length is ignored (even a misaligned value)
    a = good_args(T=5, topk=100)
    a.extra_topk_length = FAKE + 1
    assert ws_status(a)[0] == B.SMLA_OK


def test_binding_rejects_wrong_sink_length():
    import torch
    q = torch.zeros(2, 4, 576, dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="num_heads=4"):
        B._make_args(q, B.KVPool(B.SMLA_BF16, 1, 64 * 1152, 1152,
                                 torch.zeros(8, dtype=torch.uint8)),
                     torch.zeros(2, 64, dtype=torch.int32), 0.1,
                     torch.zeros(2, 4, 512, dtype=torch.bfloat16),
                     attn_sink=torch.zeros(5, dtype=torch.float32))


def _pack_args(n=10, d_qk=576):
    a = B.smla_pack_args()
    a.n, a.d_qk = n, d_qk
    a.rows = FAKE
    a.rows_stride = d_qk
    a.slots = FAKE
    a.kv = _pool(d_qk=d_qk)
    return a


PACK_FAILURES = [
    (dict(n=-1), B.SMLA_ERR_INVALID, "n is negative"),
    (dict(d_qk=512), B.SMLA_ERR_UNSUPPORTED, "d_qk=512 is not supported"),
    (dict(**{"kv.dtype": B.SMLA_BF16}), B.SMLA_ERR_UNSUPPORTED, "fp8 pools only"),
    (dict(rows=None), B.SMLA_ERR_INVALID, "rows must be non-NULL"),
    (dict(rows=FAKE + 8), B.SMLA_ERR_INVALID, "16-byte aligned"),
    (dict(rows_stride=570), B.SMLA_ERR_INVALID, "rows_stride=570"),
    (dict(rows_stride=580), B.SMLA_ERR_INVALID, "rows_stride=580"),
    (dict(slots=None), B.SMLA_ERR_INVALID, "slots must be non-NULL"),
    (dict(**{"kv.scales": None}), B.SMLA_ERR_INVALID, "kv scales is NULL"),
    (dict(**{"kv.row_stride": 520}), B.SMLA_ERR_INVALID, "kv row_stride=520"),
]


@pytest.mark.parametrize("mutation,status,fragment", PACK_FAILURES,
                         ids=[str(i) for i in range(len(PACK_FAILURES))])
def test_pack_validation_failures(mutation, status, fragment):
    a = _pack_args()
    for k, v in mutation.items():
        obj = a
        parts = k.split(".")
        for p in parts[:-1]:
            obj = getattr(obj, p)
        setattr(obj, parts[-1], v)
    rc = B.LIB.sparse_mla_pack_kv(ctypes.byref(a), None)
    msg = B.sparse_mla_last_error()
    assert rc == status, msg
    assert fragment in msg and msg.startswith("sparse-MLA pack (n="), msg


def test_pack_zero_rows_is_a_noop_without_device():
    a = _pack_args(n=0)
    a.rows = a.slots = None
    assert B.LIB.sparse_mla_pack_kv(ctypes.byref(a), None) == B.SMLA_OK


def test_compute_mode_validation():
    # fp8 mode: prefill and routed forms, d_qk 576, fp8 main pool, no extra cache
    a = good_args(T=4, h=64, topk=256)
    a.compute_mode = B.SMLA_COMPUTE_FP8
    assert ws_status(a, 0)[:2] == (B.SMLA_OK, 0)
    assert ws_status(a, 2)[:2] == (B.SMLA_OK, 0)  # the routed form does not split in fp8 mode
    rc, _, msg = ws_status(a, 1)
    assert rc == B.SMLA_ERR_UNSUPPORTED and "prefill and routed forms" in msg
    for bad in (dict(d_qk=1088, d_v=1024), dict(topk_extra=64, extra_dtype=B.SMLA_BF16)):
        b = good_args(T=4, h=64, topk=256, **bad)
        b.compute_mode = B.SMLA_COMPUTE_FP8
        rc, _, msg = ws_status(b, 0)
        assert rc == B.SMLA_ERR_UNSUPPORTED and "fp8 main pool with no extra cache" in msg, msg
    b = good_args(T=4, h=64, topk=256)
    b.kv = _pool(dtype=B.SMLA_BF16)
    b.compute_mode = B.SMLA_COMPUTE_FP8
    assert ws_status(b, 0)[0] == B.SMLA_ERR_UNSUPPORTED
    b.compute_mode = 2
    rc, _, msg = ws_status(b, 0)
    assert rc == B.SMLA_ERR_INVALID and "compute_mode=2" in msg


def test_noalloc_decode_validates_before_the_device():
    """sparse_mla_decode_noalloc validates like the decode form, ignores any workspace the
    caller passes, and (with no GPU here) stops at the device check after validation."""
    a = good_args(T=0)
    a.q = a.out = a.indices = a.lse = None
    assert B.LIB.sparse_mla_decode_noalloc(ctypes.byref(a), None) == B.SMLA_OK
    a = good_args(T=65)
    assert B.LIB.sparse_mla_decode_noalloc(ctypes.byref(a), None) == B.SMLA_ERR_UNSUPPORTED
    assert "exceeds the decode limit of 64" in B.sparse_mla_last_error()
    a = good_args(T=8, h=64, topk=512)
    a.workspace, a.workspace_bytes = None, 0  # no workspace: the scratch stands in for it
    rc = B.LIB.sparse_mla_decode_noalloc(ctypes.byref(a), None)
    assert rc in (B.SMLA_ERR_DEVICE, B.SMLA_OK), B.sparse_mla_last_error()
