"""Seeded synthetic workloads (inputs only; no estimator or attention arithmetic)."""
from .gen import (WORKLOADS, Rope, Workload, apply_rope, bf16_bits_to_f32, f32_to_bf16_bits,
                  make_qkv, random_mask, rope_axes, rope_freqs, rope_positions, rope_tables, to_f64)

__all__ = ["WORKLOADS", "Rope", "Workload", "apply_rope", "bf16_bits_to_f32", "f32_to_bf16_bits",
           "make_qkv", "random_mask", "rope_axes", "rope_freqs", "rope_positions", "rope_tables", "to_f64"]
