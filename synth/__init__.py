"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This package only draws random numbers and lays them out in the paged-pool
format; it holds none of the attention method's arithmetic (no scoring,
selection, softmax or combine), so that both the HIP library and the fp64
oracle can be fed the very same bytes without sharing any of the method.
"""

from .inputs import (  # noqa: F401
    WORKLOADS,
    WORKLOAD_SEEDS,
    Case,
    generate,
    host_view,
    workload,
)
