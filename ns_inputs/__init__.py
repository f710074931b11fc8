"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This package draws random matrices and nothing else: it holds none of the
Newton–Schulz arithmetic, and it is the only code that both the oracle-side
tests and the HIP-side callers use.
"""

from .generators import (  # noqa: F401
    GROUPED_SETS,
    WORKLOADS,
    Workload,
    gaussian,
    make_grouped_set,
    make_workload,
    workload_names,
)
