"""Seeded synthetic workloads: the only code shared by the oracle harness and the GPU path.

Nothing in this package computes a step of the attention method. It draws Q/K/V, plants
stripe keys and a local band, rounds to bf16 and names the five workload shapes.
"""
from .stripes import (  # noqa: F401
    Workload,
    WORKLOADS,
    bf16_bits_to_f32,
    bf16_round_bits,
    generate,
    generate_for,
)
