"""Seeded synthetic inputs shared by the tests, the oracle checks and the benchmark.

Holds input generation only (counter-based SplitMix64 + an N(0,1) bf16 table,
the five workloads and their planted needles/chains); none of the method's
arithmetic lives here.
"""
from . import splitmix, workloads, native  # noqa: F401
