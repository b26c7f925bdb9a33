"""Seeded synthetic inputs for paged attention.

This package holds no attention arithmetic: it draws sequence lengths, places
logical KV blocks in a shuffled physical pool, fills the pool and the queries
with bf16 values, and poisons every cache slot that no sequence owns with NaN.
Both the oracle tests and the GPU path consume what it returns.
"""

from .synth import (  # noqa: F401
    Batch,
    WORKLOADS,
    build_batch,
    make_workload,
    repermute_pool,
    workload_lengths,
)
