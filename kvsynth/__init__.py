"""Seeded synthetic KV caches shared by the tests, the smoke check and the
benchmark.

This package holds input generation only -- shapes, value distributions and
the placement of structured (tie) groups.  It contains none of the codec's
arithmetic and imports neither the codec nor the oracle.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    decode_queries,
    layer_kv,
    stream_tokens,
    uniform_with_ties,
    slice_index,
)
