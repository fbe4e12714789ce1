"""Seeded synthetic workloads shared by the tests, the benchmark and the oracle
checks.  Holds no attention arithmetic."""

from .synthetic import CONFIGS, Workload, make_config, make_tree, make_workload  # noqa: F401
