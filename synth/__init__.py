"""Seeded synthetic workloads shared by the oracle tests, the GPU parity
tests and the benchmark.  Holds shapes and random draws only."""
from .configs import HEADLINE, WORKLOADS, Workload  # noqa: F401
from . import gen  # noqa: F401
