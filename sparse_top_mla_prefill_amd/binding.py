"""ctypes binding of libsparse_mla (argument marshalling only).

Every entry point of ``include/sparse_mla.h`` has a function of the same name here. The
functions take torch tensors for device memory and the current HIP stream, check dtypes,
devices and shapes, fill the C argument struct and call the library. All arithmetic runs in
the library's HIP kernels. If the library is missing or fails to load, importing this
module raises: nothing here computes a fallback.
"""
from __future__ import annotations

import contextlib
import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_mla.so")

SMLA_BF16 = 0
SMLA_FP8_E4M3_G64 = 1
SMLA_COMPUTE_BF16, SMLA_COMPUTE_FP8 = 0, 1
SMLA_OK, SMLA_ERR_INVALID, SMLA_ERR_UNSUPPORTED, SMLA_ERR_WORKSPACE, SMLA_ERR_DEVICE = range(5)
STATUS_NAMES = {0: "SMLA_OK", 1: "SMLA_ERR_INVALID", 2: "SMLA_ERR_UNSUPPORTED",
                3: "SMLA_ERR_WORKSPACE", 4: "SMLA_ERR_DEVICE"}

EXPORTS = ("sparse_mla_prefill", "sparse_mla_decode", "sparse_mla_forward",
           "sparse_mla_decode_noalloc", "sparse_mla_workspace_size",
           "sparse_mla_supported_configs", "sparse_mla_pack_kv", "sparse_mla_last_error",
           "sparse_mla_abi_version")


class smla_cache(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("page_block_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("page_stride", ctypes.c_int64),
        ("row_stride", ctypes.c_int64),
        ("scale_page_stride", ctypes.c_int64),
        ("scale_row_stride", ctypes.c_int64),
    ]


class smla_args(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32),
        ("h", ctypes.c_int32),
        ("d_qk", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("q_stride_t", ctypes.c_int64),
        ("q_stride_h", ctypes.c_int64),
        ("kv", smla_cache),
        ("indices", ctypes.c_void_p),
        ("topk", ctypes.c_int32),
        ("indices_stride", ctypes.c_int64),
        ("extra", smla_cache),
        ("extra_indices", ctypes.c_void_p),
        ("topk_extra", ctypes.c_int32),
        ("extra_indices_stride", ctypes.c_int64),
        ("attn_sink", ctypes.c_void_p),
        ("sm_scale", ctypes.c_float),
        ("out", ctypes.c_void_p),
        ("out_stride_t", ctypes.c_int64),
        ("out_stride_h", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
        ("lse_stride_t", ctypes.c_int64),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("topk_length", ctypes.c_void_p),
        ("extra_topk_length", ctypes.c_void_p),
        ("compute_mode", ctypes.c_int32),
    ]


class smla_pack_args(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int64),
        ("d_qk", ctypes.c_int32),
        ("rows", ctypes.c_void_p),
        ("rows_stride", ctypes.c_int64),
        ("slots", ctypes.c_void_p),
        ("kv", smla_cache),
    ]


class smla_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "d_qk", "d_v", "kv_dtype", "extra_kv_dtype", "min_h", "max_h", "topk_multiple",
        "page_block_size", "decode_max_tokens")]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python sparse_top_mla_prefill_amd/build.py` "
            "(the GPU path has no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name in ("sparse_mla_prefill", "sparse_mla_decode", "sparse_mla_forward",
                 "sparse_mla_decode_noalloc"):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.POINTER(smla_args), ctypes.c_void_p]
        fn.restype = ctypes.c_int
    lib.sparse_mla_workspace_size.argtypes = [ctypes.POINTER(smla_args), ctypes.c_int,
                                              ctypes.POINTER(ctypes.c_size_t)]
    lib.sparse_mla_workspace_size.restype = ctypes.c_int
    lib.sparse_mla_supported_configs.argtypes = [ctypes.POINTER(smla_config), ctypes.c_int,
                                                 ctypes.POINTER(ctypes.c_int)]
    lib.sparse_mla_supported_configs.restype = ctypes.c_int
    lib.sparse_mla_pack_kv.argtypes = [ctypes.POINTER(smla_pack_args), ctypes.c_void_p]
    lib.sparse_mla_pack_kv.restype = ctypes.c_int
    lib.sparse_mla_last_error.argtypes = []
    lib.sparse_mla_last_error.restype = ctypes.c_char_p
    lib.sparse_mla_abi_version.argtypes = []
    lib.sparse_mla_abi_version.restype = ctypes.c_int
    return lib


LIB = _load()


class SparseMLAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


def _check(status: int) -> None:
    if status != SMLA_OK:
        raise SparseMLAError(status, LIB.sparse_mla_last_error().decode())


# --------------------------------------------------------------------------- pools
@dataclasses.dataclass
class KVPool:
    """A paged latent KV pool in device memory plus its descriptor (see smla_cache).

    ``data`` and ``scales`` are uint8 device tensors (``scales`` may be ``data``);
    ``data_offset`` / ``scale_offset`` are byte offsets of slot 0's payload and scales.
    """

    dtype: int
    num_pages: int
    page_stride: int
    row_stride: int
    data: torch.Tensor
    data_offset: int = 0
    scales: Optional[torch.Tensor] = None
    scale_offset: int = 0
    scale_page_stride: int = 0
    scale_row_stride: int = 0
    page_block_size: int = 64

    def to_c(self) -> smla_cache:
        if self.data.dtype != torch.uint8 or not self.data.is_cuda:
            raise TypeError("KVPool.data must be a uint8 device tensor")
        c = smla_cache()
        c.data = self.data.data_ptr() + self.data_offset
        if self.dtype == SMLA_FP8_E4M3_G64:
            if self.scales is None or not self.scales.is_cuda:
                raise TypeError("an fp8 KVPool needs a device scales tensor")
            c.scales = self.scales.data_ptr() + self.scale_offset
        else:
            c.scales = None
        c.dtype = self.dtype
        c.page_block_size = self.page_block_size
        c.num_pages = self.num_pages
        c.page_stride = self.page_stride
        c.row_stride = self.row_stride
        c.scale_page_stride = self.scale_page_stride
        c.scale_row_stride = self.scale_row_stride
        return c


def _stream_handle(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _row_stride(x: torch.Tensor) -> int:
    return x.stride(0) if x.dim() >= 1 and x.shape[0] > 1 else x.shape[-1]


def _lengths_ptr(name: str, x, T: int):
    if x is None:
        return None
    if x.dtype != torch.int32 or x.dim() != 1 or x.shape[0] != T or (T > 1 and x.stride(0) != 1):
        raise TypeError(f"{name} must be a dense int32 tensor of T={T} entries")
    if x.numel() and not x.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    return x.data_ptr() if x.numel() else None


def _make_args(q, kv: KVPool, indices, sm_scale, out, lse=None, extra: Optional[KVPool] = None,
               extra_indices=None, attn_sink=None, workspace=None, topk_length=None,
               extra_topk_length=None, compute_mode=SMLA_COMPUTE_BF16) -> smla_args:
    if q.dtype != torch.bfloat16 or q.dim() != 3 or q.stride(2) != 1:
        raise TypeError("q must be bf16 [T, h, d_qk] with a dense last dimension")
    T, h, d_qk = q.shape
    if indices.dtype != torch.int32 or indices.dim() != 2 or indices.shape[0] != T \
            or indices.stride(1) != 1:
        raise TypeError("indices must be int32 [T, topk] with a dense last dimension")
    if out.dtype != torch.bfloat16 or out.dim() != 3 or out.shape[:2] != (T, h) \
            or out.stride(2) != 1:
        raise TypeError("out must be bf16 [T, h, d_v] with a dense last dimension")
    if attn_sink is not None:
        if attn_sink.dtype != torch.float32 or attn_sink.numel() != h \
                or (attn_sink.dim() == 1 and attn_sink.stride(0) != 1):
            raise TypeError(f"attn_sink must be a dense float32 tensor of num_heads={h} entries")
        if not attn_sink.is_cuda:
            raise TypeError("attn_sink must be a device tensor")
    a = smla_args()
    a.T, a.h, a.d_qk, a.d_v = T, h, d_qk, out.shape[2]
    a.q = q.data_ptr() if q.numel() else None
    a.q_stride_t, a.q_stride_h = q.stride(0), q.stride(1)
    a.kv = kv.to_c()
    a.indices = indices.data_ptr() if indices.numel() else None
    a.topk = indices.shape[1]
    a.indices_stride = indices.stride(0) if T > 1 else indices.shape[1]
    if extra is not None and extra_indices is not None and extra_indices.shape[1] > 0:
        if extra_indices.dtype != torch.int32 or extra_indices.dim() != 2 \
                or extra_indices.shape[0] != T or extra_indices.stride(1) != 1:
            raise TypeError("extra_indices must be int32 [T, topk_extra]")
        a.extra = extra.to_c()
        a.extra_indices = extra_indices.data_ptr() if extra_indices.numel() else None
        a.topk_extra = extra_indices.shape[1]
        a.extra_indices_stride = extra_indices.stride(0) if T > 1 else extra_indices.shape[1]
    if attn_sink is not None:
        a.attn_sink = attn_sink.data_ptr()
    a.sm_scale = float(sm_scale)
    a.out = out.data_ptr() if out.numel() else None
    a.out_stride_t, a.out_stride_h = out.stride(0), out.stride(1)
    if lse is not None:
        if lse.dtype != torch.float32 or lse.dim() != 2 or lse.shape != (T, h) \
                or lse.stride(1) != 1:
            raise TypeError("lse must be float32 [T, h] with a dense last dimension")
        a.lse = lse.data_ptr() if lse.numel() else None
        a.lse_stride_t = lse.stride(0) if T > 1 else h
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    a.compute_mode = int(compute_mode)
    a.topk_length = _lengths_ptr("topk_length", topk_length, T)
    if a.topk_extra > 0:
        a.extra_topk_length = _lengths_ptr("extra_topk_length", extra_topk_length, T)
    for name, t in (("q", q), ("indices", indices), ("out", out)):
        if t.numel() and not t.is_cuda:
            raise TypeError(f"{name} must be a device tensor")
    return a


FORM_PREFILL, FORM_DECODE, FORM_FORWARD = 0, 1, 2


def sparse_mla_workspace_size(q, kv: KVPool, indices, sm_scale, out, form, **kw) -> int:
    """Workspace bytes of a form: 0 / False prefill, 1 / True decode, 2 forward."""
    a = _make_args(q, kv, indices, sm_scale, out, **kw)
    n = ctypes.c_size_t(0)
    _check(LIB.sparse_mla_workspace_size(ctypes.byref(a), int(form), ctypes.byref(n)))
    return int(n.value)


def _on_stream(stream):
    """Context in which buffers that the binding allocates for a call belong to the stream
    the call's kernels run on. The caching allocator then hands their memory to another
    allocation only in that stream's order, so a workspace dropped when the call returns
    cannot be reused while those kernels still read or write it."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _new_out(q, out):
    if out is not None:
        return out
    d_v = {576: 512, 1088: 1024}.get(q.shape[-1], q.shape[-1])
    return torch.empty(q.shape[0], q.shape[1], d_v, dtype=torch.bfloat16, device=q.device)


def _run(fn, form, q, kv, indices, sm_scale, out, lse, extra, extra_indices, attn_sink,
         workspace, stream, topk_length=None, extra_topk_length=None,
         compute_mode=SMLA_COMPUTE_BF16):
    kw = dict(lse=lse, extra=extra, extra_indices=extra_indices, attn_sink=attn_sink,
              topk_length=topk_length, extra_topk_length=extra_topk_length,
              compute_mode=compute_mode)
    with _on_stream(stream):
        out = _new_out(q, out)
        if form != FORM_PREFILL and workspace is None:
            nbytes = sparse_mla_workspace_size(q, kv, indices, sm_scale, out, form, **kw)
            if nbytes:
                workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        a = _make_args(q, kv, indices, sm_scale, out, workspace=workspace, **kw)
        _check(fn(ctypes.byref(a), _stream_handle(stream)))
    return out


def sparse_mla_prefill(q, kv: KVPool, indices, sm_scale: float, out=None, lse=None,
                       extra: Optional[KVPool] = None, extra_indices=None, attn_sink=None,
                       stream=None, topk_length=None, extra_topk_length=None,
                       compute_mode=SMLA_COMPUTE_BF16) -> torch.Tensor:
    """out[t, h] = softmax-with-sink attention of q[t, h] over the token's gathered rows.

    ``topk_length`` / ``extra_topk_length``: optional int32 [T] live counts per index row.
    ``compute_mode``: SMLA_COMPUTE_BF16 (default) or SMLA_COMPUTE_FP8 (see the header)."""
    return _run(LIB.sparse_mla_prefill, FORM_PREFILL, q, kv, indices, sm_scale, out, lse, extra,
                extra_indices, attn_sink, None, stream, topk_length, extra_topk_length,
                compute_mode)


def sparse_mla_decode(q, kv: KVPool, indices, sm_scale: float, out=None, lse=None,
                      extra: Optional[KVPool] = None, extra_indices=None, attn_sink=None,
                      workspace=None, stream=None, topk_length=None,
                      extra_topk_length=None, compute_mode=SMLA_COMPUTE_BF16) -> torch.Tensor:
    """Decode form (T <= 64): the same function, split over index chunks.

    ``stream``: the torch stream to run on (default: the current stream). An ``out`` or
    workspace that this function allocates belongs to that stream."""
    return _run(LIB.sparse_mla_decode, FORM_DECODE, q, kv, indices, sm_scale, out, lse, extra,
                extra_indices, attn_sink, workspace, stream, topk_length, extra_topk_length,
                compute_mode)


def sparse_mla_decode_noalloc(q, kv: KVPool, indices, sm_scale: float, out, lse=None,
                              extra: Optional[KVPool] = None, extra_indices=None,
                              attn_sink=None, stream=None, topk_length=None,
                              extra_topk_length=None) -> torch.Tensor:
    """Decode form whose split-K partials live in the library's per-device scratch: the
    call allocates nothing, so ``out`` (and ``lse``, if wanted) must be given. Calls that
    overlap in time on one device race on that scratch."""
    if out is None:
        raise TypeError("sparse_mla_decode_noalloc allocates nothing: pass out")
    a = _make_args(q, kv, indices, sm_scale, out, lse=lse, extra=extra,
                   extra_indices=extra_indices, attn_sink=attn_sink, topk_length=topk_length,
                   extra_topk_length=extra_topk_length)
    _check(LIB.sparse_mla_decode_noalloc(ctypes.byref(a), _stream_handle(stream)))
    return out


def sparse_mla_forward(q, kv: KVPool, indices, sm_scale: float, out=None, lse=None,
                       extra: Optional[KVPool] = None, extra_indices=None, attn_sink=None,
                       workspace=None, stream=None, topk_length=None,
                       extra_topk_length=None, compute_mode=SMLA_COMPUTE_BF16) -> torch.Tensor:
    """Routed form (any T): the decode form's split plan up to 64 rows, else prefill."""
    return _run(LIB.sparse_mla_forward, FORM_FORWARD, q, kv, indices, sm_scale, out, lse, extra,
                extra_indices, attn_sink, workspace, stream, topk_length, extra_topk_length,
                compute_mode)


def sparse_mla_pack_kv(rows, slots, kv: KVPool, stream=None) -> None:
    """Write bf16 rows [n, d_qk] into their slots of the fp8 pool ``kv`` (see the header)."""
    if rows.dtype != torch.bfloat16 or rows.dim() != 2 or rows.stride(1) != 1:
        raise TypeError("rows must be bf16 [n, d_qk] with a dense last dimension")
    n, d_qk = rows.shape
    if slots.dtype != torch.int32 or slots.dim() != 1 or slots.shape[0] != n \
            or (n > 1 and slots.stride(0) != 1):
        raise TypeError(f"slots must be a dense int32 tensor of n={n} entries")
    if n and not (rows.is_cuda and slots.is_cuda):
        raise TypeError("rows and slots must be device tensors")
    a = smla_pack_args()
    a.n, a.d_qk = n, d_qk
    a.rows = rows.data_ptr() if n else None
    a.rows_stride = rows.stride(0) if n > 1 else d_qk
    a.slots = slots.data_ptr() if n else None
    a.kv = kv.to_c()
    _check(LIB.sparse_mla_pack_kv(ctypes.byref(a), _stream_handle(stream)))


def sparse_mla_supported_configs() -> list[dict]:
    count = ctypes.c_int(0)
    _check(LIB.sparse_mla_supported_configs(None, 0, ctypes.byref(count)))
    arr = (smla_config * count.value)()
    _check(LIB.sparse_mla_supported_configs(arr, count.value, ctypes.byref(count)))
    return [{n: getattr(c, n) for n, _ in smla_config._fields_} for c in arr]


def sparse_mla_last_error() -> str:
    return LIB.sparse_mla_last_error().decode()


def sparse_mla_abi_version() -> int:
    return int(LIB.sparse_mla_abi_version())
