"""CPU oracle for sparse top-k MLA attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this package.
The GPU library neither imports nor links anything from here.
"""
from .reference import (  # noqa: F401
    attend,
    bf16_to_f64,
    decode_rows,
    e4m3fn_table,
    e4m3fn_value,
    gather_token,
    sparse_mla_reference,
    sparse_mla_reference_parallel,
    valid_mask,
)
