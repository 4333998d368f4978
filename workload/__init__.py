"""Synthetic workloads for the H2O hot path: configurations and seeded inputs.

Shared by the GPU path's harness and the CPU oracle; holds none of the method's
arithmetic.
"""
from .configs import WORKLOADS, BY_INDEX, Workload, budget_from_percent, get, scaled  # noqa: F401
from . import synth  # noqa: F401
