"""Oracle k=1 draft head (test infrastructure only; see the package docstring).

The 35B-A3B release ships a 50 MB k=1 drafter: an fp16 head of fc1, gelu and
fc2 over the model's own hidden state and the next token's embedding
(Scion-35B-A3B card, "Shipped Components" and "Highlights").  Plainest reading,
evaluated in float64:

    x = [hidden ; embedding]             the two vectors concatenated, hidden first
    y = W2 gelu(W1 x + b1) + b2          gelu(v) = v Phi(v) = v (1 + erf(v / sqrt 2)) / 2
    W1 [m x 2h], W2 [h x m] fp16; b1 [m], b2 [h] fp16 or absent

With h = 2048 (the 35B-A3B-class model width used here) and m = 4096 the head
holds 25.2 M fp16 weights, the card's 50 MB.
"""
from __future__ import annotations

import math

import numpy as np

from .moe import bf16_to_f64, f16_to_f64


def gelu(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return 0.5 * v * (1.0 + erf(v / math.sqrt(2.0)))


def head(hidden_bits, emb_bits, w1_bits, b1_bits, w2_bits, b2_bits) -> np.ndarray:
    """bf16 hidden [T, h] and embedding [T, h], fp16 W1 [m, 2h], b1 [m] or None,
    W2 [h, m], b2 [h] or None (bit patterns) -> y float64 [T, h]."""
    x = np.concatenate([bf16_to_f64(hidden_bits), bf16_to_f64(emb_bits)], axis=1)
    a = x @ f16_to_f64(w1_bits).T
    if b1_bits is not None:
        a = a + f16_to_f64(b1_bits)
    y = gelu(a) @ f16_to_f64(w2_bits).T
    if b2_bits is not None:
        y = y + f16_to_f64(b2_bits)
    return y
