"""Seeded synthetic workloads for the EP dispatch/combine path.

This package holds only input generation (routing, weights, activations,
expert outputs) and the workload table.  It contains none of the method's
arithmetic, and both the oracle-side tests and the GPU path consume its
output.
"""
from .gen import WORKLOADS, Workload, generate, workload  # noqa: F401
