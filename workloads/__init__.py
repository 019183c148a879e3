"""Seeded synthetic workloads for paged-attention decode.

This package is the only code shared by the CPU oracle and the HIP path.
It draws random numbers and arranges them into the shapes the method
consumes (a physical block pool, per-sequence block tables, context lengths,
queries and the new tokens' K/V).  It contains none of the method's
arithmetic: no block-table resolution, no gather, no attention.
"""

from .synth import (  # noqa: F401
    CONFIG_NAMES,
    AppendBatch,
    Workload,
    bf16_round_bits,
    config_spec,
    make_append_batch,
    make_workload,
    storage_dtype,
)
