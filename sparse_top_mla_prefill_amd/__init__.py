"""Sparse top-k MLA attention over a paged latent KV pool, for AMD MI355X (gfx950).

The compute path is libsparse_mla.so (hand-written HIP kernels behind a C ABI, see
include/sparse_mla.h); ``binding`` marshals torch tensors into its calls.
"""
from .binding import (  # noqa: F401
    SMLA_BF16,
    SMLA_COMPUTE_BF16,
    SMLA_COMPUTE_FP8,
    SMLA_FP8_E4M3_G64,
    KVPool,
    SparseMLAError,
    sparse_mla_abi_version,
    sparse_mla_decode,
    sparse_mla_decode_noalloc,
    sparse_mla_forward,
    sparse_mla_last_error,
    sparse_mla_pack_kv,
    sparse_mla_prefill,
    sparse_mla_supported_configs,
    sparse_mla_workspace_size,
)
