"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check."""
from .synth import (  # noqa: F401
    GEOMETRIES,
    PAGE_BLOCK_SIZE,
    WORKLOADS,
    Pool,
    Problem,
    distinct,
    draw_pool,
    pack_pool,
    pool_payload,
    relayout,
    small_problem,
    to_bf16_bits,
    to_e4m3_bytes,
)
