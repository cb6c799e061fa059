"""Seeded synthetic workloads shared by the tests, the benchmark and the smoke check."""

from .synthetic import (  # noqa: F401
    KV_WORKLOADS,
    WORKLOADS,
    KvWorkload,
    Workload,
    activations,
    device_activations,
    device_gate_up,
    device_weights,
    gate_up,
    kv_key_channels,
    kv_slot_mapping,
    kv_tokens,
    outlier_channels,
    random_matrix,
    random_nvfp4_bytes,
    round_bf16,
    weights,
)
