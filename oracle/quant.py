"""Oracle ternary quantizer for 128-weight groups (test infrastructure only; see
the package docstring).

The pages name two ways of turning a group of weights into ternary codes and one
scale, without spelling them out: one-shot absmean and the deployed ternary
Lloyd quantizer over groups of 128, which they report as the better of the two
(project README, "What the experiments established"; the Scion-35B-A3B
discussion thread, its list of findings; the Scion-35B-A3B card, "Highlights").
This module takes the plainest reading of each:

  absmean   s = mean |w| over the group; t = sign(w) where 2|w| > s, else 0.
            This is clamp(round(w / s), -1, 1) with a tie |w| = s/2 rounded to
            the even value 0, decided without forming w / s.
  lloyd     Start from the absmean codes, then alternate
                s = mean |w| over the weights whose code is not 0
                t = sign(w) where 2|w| > s, else 0
            until the codes repeat (at most 32 rounds).  Each half-step is the
            exact minimiser of the squared error for the other half held fixed.

Precision: the codes are integers decided by floating point, so this oracle
takes those decisions in the kernel's precision, float32, with every sum over a
group taken in one fixed order (a balanced tree over adjacent pairs: weights
2m and 2m+1, then the pair sums 2m and 2m+1, and so on).  The stored scale is
s rounded to binary16 (nearest, ties to even; values beyond the largest finite
binary16 saturate to it).  A group of zeros gets scale 0 and codes 0.  Inputs
are bfloat16 bit patterns and must be finite.
"""
from __future__ import annotations

import numpy as np

from . import codec

GROUP = 128
MAX_ROUNDS = 32
ABSMEAN = 0
LLOYD = 1
F16_MAX_BITS = 0x7BFF


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def tree_sum_f32(v: np.ndarray) -> np.ndarray:
    """float32 sums over the last axis (a power of two long) as a balanced tree
    over adjacent pairs."""
    v = np.asarray(v, dtype=np.float32)
    while v.shape[-1] > 1:
        v = v[..., 0::2] + v[..., 1::2]
    return v[..., 0]


def codes_for(w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """t = sign(w) where 2|w| > s, else 0 (float32, exact comparison)."""
    a2 = np.float32(2) * np.abs(w)
    return np.where(a2 > s[..., None], np.sign(w), np.float32(0)).astype(np.int8)


def mean_of_nonzero(w: np.ndarray, t: np.ndarray) -> np.ndarray:
    """float32 mean |w| over the weights with t != 0 (0 where there are none)."""
    a = np.where(t != 0, np.abs(w), np.float32(0)).astype(np.float32)
    total = tree_sum_f32(a)
    count = np.count_nonzero(t, axis=-1).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(count > 0, total / np.maximum(count, np.float32(1)), np.float32(0)).astype(np.float32)


def scale_bits(s: np.ndarray) -> np.ndarray:
    """binary16 bit patterns of the float32 scales, nearest-even, saturating."""
    h = np.asarray(s, dtype=np.float32).astype(np.float16)
    bits = h.view(np.uint16).copy()
    bits[np.isinf(h)] = F16_MAX_BITS
    return bits


def quantize_groups(w_bits: np.ndarray, method: int, history: list | None = None):
    """bfloat16 weights (n multiple of 128) -> (trits int8 [n], binary16 scale
    bits [n / 128], float32 scales before rounding, rounds taken per group).

    history: if a list, receives (codes, scales) after every round (absmean
    start included), for the tests."""
    w = bf16_to_f32(np.asarray(w_bits).reshape(-1, GROUP))
    s = tree_sum_f32(np.abs(w)) / np.float32(GROUP)
    t = codes_for(w, s)
    rounds = np.zeros(w.shape[0], dtype=np.int32)
    if history is not None:
        history.append((t.copy(), s.copy()))
    if method == LLOYD:
        active = np.ones(w.shape[0], dtype=bool)
        for _ in range(MAX_ROUNDS):
            if not active.any():
                break
            s_new = mean_of_nonzero(w, t)
            t_new = codes_for(w, s_new)
            s = np.where(active, s_new, s)
            changed = np.any(t_new != t, axis=1) & active
            rounds += active
            t = np.where(active[:, None], t_new, t)
            active = changed
            if history is not None:
                history.append((t.copy(), s.copy()))
        # the stored scale belongs to the final codes
        s = mean_of_nonzero(w, t)
    elif method != ABSMEAN:
        raise ValueError(f"unknown method {method}")
    return t.reshape(-1), scale_bits(s), s, rounds


def quantize(fmt: int, w_bits: np.ndarray, method: int) -> np.ndarray:
    """The container bytes (row-major group order) of the quantized weights."""
    t, sb, _, _ = quantize_groups(w_bits, method)
    return codec.pack(fmt, t, sb)
