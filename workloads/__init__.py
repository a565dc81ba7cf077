"""Synthetic workloads (shapes and seeded inputs) for the sparse attention step."""
from .configs import ALL, BY_NAME, Workload  # noqa: F401
