"""Seeded inputs of the k=1 draft head: fp16 weights and biases, bf16 hidden
states and next-token embeddings.  The drafter's weights are not published
(Scion-35B-A3B card, "Shipped Components"); these are random with the usual
fan-in scaling.  Only numbers are drawn here."""
from __future__ import annotations

import numpy as np

from .layers import bf16_bits, f16_bits

_SEED = 0x5C1C


def _rng(*key):
    return np.random.default_rng(np.random.SeedSequence(_SEED, spawn_key=tuple(key)))


def head_weights(h: int, m: int, seed: int = 0):
    """fp16 bits: W1 [m, 2h] ~ N(0, 1/2h), b1 [m] ~ N(0, 0.02^2), W2 [h, m] ~ N(0, 1/m), b2 [h]."""
    w1 = f16_bits(_rng(seed, h, m, 0).normal(0.0, 1.0 / np.sqrt(2 * h), size=(m, 2 * h)))
    b1 = f16_bits(_rng(seed, h, m, 1).normal(0.0, 0.02, size=m))
    w2 = f16_bits(_rng(seed, h, m, 2).normal(0.0, 1.0 / np.sqrt(m), size=(h, m)))
    b2 = f16_bits(_rng(seed, h, m, 3).normal(0.0, 0.02, size=h))
    return w1, b1, w2, b2


def head_inputs(T: int, h: int, seed: int = 0):
    """bf16 bits: hidden states [T, h] ~ N(0, 1) and next-token embeddings [T, h] ~ N(0, 1)."""
    return (bf16_bits(_rng(seed, T, h, 10).normal(size=(T, h))),
            bf16_bits(_rng(seed, T, h, 11).normal(size=(T, h))))
