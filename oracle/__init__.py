"""CPU fp64 oracle for paged MLA decode.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and its
Python binding) imports, links or runs anything in this package; only the
test suite, the smoke check and the benchmark's CPU-baseline leg do.
"""
from .mla_oracle import (  # noqa: F401
    PAGE,
    D_QK,
    D_V,
    FP8_RECORD,
    bf16_bits_to_f64,
    e4m3fn_to_f64,
    decode_fp8_records,
    decode_kv_rows,
    gather_sequence,
    attend,
    combine_partials,
    mla_decode,
    mla_decode_sparse,
    mla_sparse_prefill,
    mla_decode_workload,
)
