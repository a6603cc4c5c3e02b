"""Seeded synthetic workloads for the paged KV-cache write and paged decode attention.

This package only draws inputs: sequence lengths, block placements, q/K/V contents,
the write-side ``slot_mapping`` a scheduler would hand over, and the pool layout of
each workload.  It holds none of the method's arithmetic (no slot decoding, no
address translation inside a kernel, no attention).  Both the CPU oracle and the
GPU path consume what it produces.
"""

from .gen import (  # noqa: F401
    BLOCK_SIZE,
    CONFIG_NAMES,
    VarlenStep,
    Workload,
    alibi_variant,
    custom,
    dtype_nbytes,
    fp8_variant,
    make_config,
    nan_bits,
    varlen_config,
    varlen_variant,
)
