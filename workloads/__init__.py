"""Seeded synthetic workloads shared by the tests, the benchmark and the smoke check."""

from .synthetic import (  # noqa: F401
    WORKLOADS,
    Workload,
    activations,
    gate_up,
    outlier_channels,
    random_matrix,
    round_bf16,
    weights,
)
