"""Seeded dense bfloat16 weight matrices, the input of the ternary quantizer.

The pages quantize trained expert weights (project README, "What the
experiments established": OLMoE experts, groups of 128) and publish none, so
these stand in for them: Student-t entries with 5 degrees of freedom (heavier
tails than a Gaussian, as trained weights have) times a per-row log-normal
scale (median 0.02, sigma 0.25 in log space).  Only numbers are drawn here;
nothing of the quantizer's arithmetic.
"""
from __future__ import annotations

import numpy as np

from .layers import bf16_bits

_SEED = 0x5C1A
ROW_MEDIAN = 0.02
ROW_SIGMA = 0.25
T_DOF = 5


def weights_bf16(rows: int, cols: int, seed: int = 0) -> np.ndarray:
    """[rows x cols] bfloat16 bit patterns (uint16), host memory."""
    rng = np.random.default_rng(np.random.SeedSequence(_SEED, spawn_key=(seed, rows, cols)))
    scale = ROW_MEDIAN * np.exp(ROW_SIGMA * rng.standard_normal(rows))
    w = rng.standard_t(T_DOF, size=(rows, cols)) * scale[:, None]
    return bf16_bits(w)


def weights_bf16_device(rows: int, cols: int, seed: int = 0, device="cuda"):
    """The same distribution drawn on the device with torch's generator (for
    sizes the host generator would take minutes on): an int16 tensor of
    bfloat16 bit patterns, [rows x cols].  Student-t as normal / sqrt(chi2/5)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_SEED * 1_000_003 + seed)
    scale = ROW_MEDIAN * torch.exp(ROW_SIGMA * torch.randn(rows, 1, generator=g, device=device))
    out = torch.empty(rows, cols, dtype=torch.bfloat16, device=device)
    step = max(1, (1 << 26) // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        z = torch.randn(r1 - r0, cols, generator=g, device=device)
        chi2 = torch.zeros_like(z)
        for _ in range(T_DOF):
            chi2 += torch.randn(r1 - r0, cols, generator=g, device=device) ** 2
        out[r0:r1] = (z / torch.sqrt(chi2 / T_DOF) * scale[r0:r1]).to(torch.bfloat16)
    return out.view(torch.int16)
