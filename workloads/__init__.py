"""Seeded synthetic workloads shared by the tests, the oracle checks and bench.py."""

from .gen import (  # noqa: F401
    Workload,
    bf16_rne_bits,
    build,
    to_fp8,
    tiny,
    batch_decode,
    long_context,
    verify,
    padded,
    merge_inputs,
    GatherWorkload,
    context_gather,
    long_context_gather,
    STANDARD,
)
