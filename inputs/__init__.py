"""Seeded synthetic inputs for the decode workloads (no recurrence arithmetic here)."""
from .synthetic import (GDN, KDA, RWKV6, VARIANT_NAMES, WORKLOADS, DecodeInputs,  # noqa: F401
                        bf16_bits_to_f32, f32_to_bf16_bits, make_inputs, tile_inputs)
