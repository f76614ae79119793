"""Seeded synthetic workloads shared by the oracle, the tests and the benchmark.

This package holds shapes, method constants and random input generation only.
It contains none of the attention method's arithmetic, so the CPU oracle and the
GPU path can both consume it without sharing any computation.
"""
from .configs import Workload, CONFIGS, get_config, small_workload  # noqa: F401
from .generator import make_inputs, perturb, positional_features  # noqa: F401
