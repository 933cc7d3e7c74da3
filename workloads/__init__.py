"""Seeded synthetic workloads for paged prefix-reuse attention.

This module only draws inputs: lengths, block placements, block tables, slot
mappings, N(0,1) values rounded to 16-bit payloads, and the K scales a caller of a
quantised pool might pick from example tokens.  It holds none of the
attention arithmetic.  Both the fp64 oracle (through the tests) and the HIP path
(through the tests and the benchmark) consume what it returns.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    Workload,
    make,
    make_config,
    make_custom,
    round_to_bits,
    blocks_for,
    channel_scales,
)
