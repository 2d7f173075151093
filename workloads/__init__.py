"""Seeded synthetic inputs for masked paged attention.

This package only draws random numbers and lays them out in the operator's
layouts (packed / padded query rows, paged key/value cache with a random block
permutation, block tables, host length arrays, ALiBi slopes, explicit compressed
mask tiles).  It holds none of
the attention arithmetic: both the HIP path's tests/benchmark and the fp64 oracle
read the tensors it returns.
"""

from .gen import (  # noqa: F401
    FP16,
    BF16,
    PrefillCase,
    MLACase,
    alibi_slopes,
    compressed_tile,
    make_prefill,
    make_prefill_config,
    make_mla,
    make_mla_config,
    make_mla_int8,
    pad_prefill_case,
    PREFILL_CONFIGS,
    MLA_CONFIGS,
)
