"""Seeded synthetic inputs for the paged decode and chunked-prefill steps.

This package is shared by the oracle side (tests) and the GPU side (binding
tests, bench).  It draws random numbers and lays out arrays; it holds none of
the attention arithmetic, none of the cache-write/copy semantics and no block
manager.  Block placement is expressed as a list of block-manager operations
(``ops``) that each side replays through its own block manager.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    PREFILL_CONFIGS,
    PrefillWorkload,
    Workload,
    bf16_bits_from_f32,
    make_workload,
    make_custom,
    make_prefill_custom,
    make_prefill_workload,
)
