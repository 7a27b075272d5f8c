"""Upload a generated Problem to device memory in the library's descriptor form.

Plumbing only: copies bytes and fills descriptor fields; no attention arithmetic.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from sparse_top_mla_prefill_amd.binding import SMLA_BF16, SMLA_FP8_E4M3_G64, KVPool

from .synth import Pool, Problem


@dataclasses.dataclass
class DeviceProblem:
    q: torch.Tensor
    kv: KVPool
    indices: torch.Tensor
    sm_scale: float
    attn_sink: Optional[torch.Tensor]
    extra: Optional[KVPool]
    extra_indices: Optional[torch.Tensor]
    d_v: int
    topk_length: Optional[torch.Tensor] = None
    extra_topk_length: Optional[torch.Tensor] = None

    def kwargs(self) -> dict:
        kw = dict(extra=self.extra, extra_indices=self.extra_indices, attn_sink=self.attn_sink)
        if self.topk_length is not None:
            kw["topk_length"] = self.topk_length
        if self.extra_topk_length is not None:
            kw["extra_topk_length"] = self.extra_topk_length
        return kw

    def new_out(self) -> torch.Tensor:
        T, h, _ = self.q.shape
        return torch.empty(T, h, self.d_v, dtype=torch.bfloat16, device=self.q.device)


def pool_to_device(pool: Pool, device) -> KVPool:
    data = torch.from_numpy(np.ascontiguousarray(pool.data)).to(device)
    scales, soff = None, 0
    if pool.dtype == "fp8":
        if pool.scales is pool.data:
            scales, soff = data, pool.scale_offset
        else:
            scales = torch.from_numpy(np.ascontiguousarray(pool.scales)).to(device)
            soff = pool.scale_offset
    return KVPool(dtype=SMLA_BF16 if pool.dtype == "bf16" else SMLA_FP8_E4M3_G64,
                  num_pages=pool.num_pages, page_stride=pool.page_stride,
                  row_stride=pool.row_stride, data=data, data_offset=pool.data_offset,
                  scales=scales, scale_offset=soff, scale_page_stride=pool.scale_page_stride,
                  scale_row_stride=pool.scale_row_stride, page_block_size=pool.page_block_size)


def to_device(p: Problem, device="cuda") -> DeviceProblem:
    q = torch.from_numpy(np.ascontiguousarray(p.q_bits).view(np.int16)).view(torch.bfloat16)
    sink = None if p.attn_sink is None else torch.from_numpy(p.attn_sink.astype(np.float32))
    extra = eidx = None
    if p.extra is not None:
        extra = pool_to_device(p.extra, device)
        eidx = torch.from_numpy(np.ascontiguousarray(p.extra_indices)).to(device)
    def _lens(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(device)

    return DeviceProblem(q=q.to(device), kv=pool_to_device(p.kv, device),
                         indices=torch.from_numpy(np.ascontiguousarray(p.indices)).to(device),
                         sm_scale=float(p.sm_scale),
                         attn_sink=None if sink is None else sink.to(device),
                         extra=extra, extra_indices=eidx, d_v=p.d_v,
                         topk_length=_lens(p.topk_length),
                         extra_topk_length=_lens(p.extra_topk_length))
