"""Seeded synthetic inputs for paged MLA decode.

This package only draws random numbers and lays them out in the cache formats
(page pool, block table, sequence lengths, BF16 rows, 656-byte FP8 records).
It holds none of the attention arithmetic: both the CPU oracle (test side)
and the HIP library consume what it produces.
"""
from .gen import (  # noqa: F401
    Workload,
    WORKLOAD_SPECS,
    make_workload,
    make_sparse_workload,
    draw_indices,
    dense_as_sparse,
    PrefillWorkload,
    PREFILL_SPECS,
    make_prefill_workload,
    named_prefill,
    named_workload,
    poison_unused,
    permute_pages,
    quantize_fp8_records,
)
