"""Seeded synthetic inputs for the paged-attention path.

This package is the only code shared by the CPU oracle and the HIP path's
tests and benchmark.  It draws random numbers and lays out the scheduler's
metadata (block tables, slot mappings, packed query boundaries); it holds
none of the attention arithmetic and none of the cache-write logic.
"""

from .generate import (  # noqa: F401
    CONFIG_NAMES,
    Case,
    bf16_bits_from_f32,
    build_case,
    make_config,
    prefix_kv_rows,
)
