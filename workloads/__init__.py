"""Seeded synthetic inputs for proxy-query token eviction (no compaction arithmetic here)."""
from .gen import (  # noqa: F401
    Workload,
    spec,
    custom,
    unit_keys,
    unit_values,
    unit_queries,
    bias_row,
    block_tables,
    build_contiguous,
    build_paged,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    c4_budget,
    score_rows,
    row_positions,
    device_normal_bf16,
)
