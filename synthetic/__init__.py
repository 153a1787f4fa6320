"""Seeded synthetic inputs (trits, fp16/bf16 bit patterns) for the MoE block."""
from .layers import (CONFIGS, PQ2_0, PTQ1_0, LayerConfig, LayerGen, bank_byte_sizes,
                     bf16_bits, f16_bits)

__all__ = ["CONFIGS", "PQ2_0", "PTQ1_0", "LayerConfig", "LayerGen", "bank_byte_sizes",
           "bf16_bits", "f16_bits"]
