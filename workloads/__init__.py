"""Seeded synthetic inputs for paged decode attention.

This package only *draws* inputs (random values, context lengths, block
placement) and stores them in the byte formats the cache uses (fp32, bf16,
FP8 E4M3 codes with per-token scales).  It holds none of the attention
arithmetic: both the CPU oracle and the GPU path consume what it returns.
"""

from .synthetic import (  # noqa: F401
    BLOCK_SIZE,
    Inputs,
    Spec,
    NAMED_SPECS,
    make_device_workload,
    make_inputs,
    named_spec,
)
from .chunks import (  # noqa: F401
    CHUNK_SPECS,
    ChunkInputs,
    chunk_queries,
    make_chunk_inputs,
)
from .kivi import KiviInputs, kivi_state, make_kivi_inputs  # noqa: F401
