"""Seeded synthetic MoE-block inputs shared by the HIP path's tests/bench and the oracle.

This module only draws numbers. It holds none of the method's arithmetic: no
container packing, no routing, no matmul. It returns raw trits in {-1, 0, +1}
(int8), IEEE binary16 bit patterns (uint16) for fp16 tensors and bfloat16 bit
patterns (uint16) for activations. Each consumer packs the trits into its own
containers with its own codec.

Shapes follow the layers the release cards describe:
  * the OLMoE-1B-7B proxy (Scion project README, "What the experiments established"),
  * the 35B-A3B release (Scion-35B-A3B card, "Model Overview": 256 experts, top-8),
  * the FlashNext release (Scion-FlashNext-176B-A6B card, "Model Overview":
    512 experts, top-10 routed + 1 shared, PTQ1_0 experts).
The dimensions d, f, r and the distributions are those of the five synthetic
layer configurations below; the pages publish no weights.

Every tensor comes from its own counter-addressed stream:
SeedSequence(0x5C10 + config index, spawn_key=(kind, ...)). A stream never
depends on the order in which other tensors were drawn, so an expert or an
activation set can be regenerated alone.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple

import numpy as np

PQ2_0 = 142    # format ids used by the fork for its containers
PTQ1_0 = 143   # (Scion-35B-A3B card "Quickstart"; FlashNext card "About the Hub's quant chip")

# stream kinds (fixed order: x, W_r, dW_r, codes, scales, A, B, outliers, format map, zipf,
# ternary-coded dW_r, A, B)
_K_X, _K_WR, _K_DWR, _K_CODES, _K_SCALES, _K_A, _K_B, _K_OUTL, _K_FMT, _K_ZIPF = range(10)
_K_DWR_Q, _K_A_Q, _K_B_Q = 10, 11, 12
_K_DU, _K_DV = 13, 14
# group-scale spread of the ternary-coded router delta and correction: a
# ternary code set with P(+-1) = 0.3 each and scale |N(0, sigma)| has about the
# magnitude of the dense N(0, 0.002) delta and N(0, 0.01) factors
_Q_SIGMA = {_K_DWR_Q: 0.003, _K_A_Q: 0.015, _K_B_Q: 0.015}

# Zipf popularity enters through a constant "massive activation" channel 0 of x
# and router column 0 = tau * ln p_e.  tau was chosen once so the hottest expert
# takes roughly 40x the mean load at T=4096 (checked by a CPU test).
ZIPF_TAU = 3.0
ZIPF_S = 1.1


@dataclass(frozen=True)
class LayerConfig:
    name: str
    index: int            # seed index
    d_model: int
    n_experts: int        # routed experts E
    d_ff: int             # expert ffn dim f
    top_k: int
    n_shared: int         # always-on shared experts S (0 or 1)
    rank: int             # correction rank r
    fmt: str              # "pq2_0" | "ptq1_0" | "mixed"
    decode_tokens: Tuple[int, ...] = ()
    prefill_tokens: Tuple[int, ...] = ()
    zipf: bool = False
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0

    @property
    def n_banks(self) -> int:
        return self.n_experts + self.n_shared


CONFIGS = {
    # C0 tiny block: correctness only
    "tiny": LayerConfig("tiny", 0, 256, 8, 128, 2, 0, 16, "pq2_0", decode_tokens=(16,)),
    # C1 OLMoE-shaped layer
    "olmoe": LayerConfig("olmoe", 1, 2048, 64, 1024, 8, 0, 512, "pq2_0",
                         decode_tokens=(1, 8, 64)),
    # C2 35B-A3B-class layer
    "a3b35": LayerConfig("a3b35", 2, 2048, 128, 768, 8, 0, 512, "pq2_0",
                         decode_tokens=(1, 2, 4, 8, 16, 32), prefill_tokens=(4096,)),
    # C3 Flash-Next-shaped layer, PTQ1_0 experts and one shared expert
    "flashnext": LayerConfig("flashnext", 3, 3072, 512, 512, 10, 1, 512, "ptq1_0",
                             decode_tokens=(1, 2, 4, 8, 16, 32, 64), prefill_tokens=(4096,)),
    # C4 skewed-routing stress at Flash-Next shape, mixed containers
    "skewed": LayerConfig("skewed", 4, 3072, 512, 512, 10, 1, 512, "mixed",
                          prefill_tokens=(16384,), zipf=True, outlier_frac=0.01,
                          outlier_scale=50.0),
}


def f16_bits(a: np.ndarray) -> np.ndarray:
    """Round float64 to IEEE binary16 (round-to-nearest-even) and return the bits."""
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float16)).view(np.uint16)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float64 -> float32 -> bfloat16 (both round-to-nearest-even); return bits."""
    b = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32)).view(np.uint32)
    b = b.astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


_TRIT_LUT = np.array([-1, -1, -1, 0, 0, 0, 0, 1, 1, 1], dtype=np.int8)  # P(0)=0.4, P(+-1)=0.3


class LayerGen:
    """Deterministic generator for one layer configuration."""

    def __init__(self, cfg: LayerConfig):
        self.cfg = cfg
        self._entropy = 0x5C10 + cfg.index
        self._zipf_cache = None

    # -- streams -----------------------------------------------------------
    def rng(self, *key: int) -> np.random.Generator:
        return np.random.default_rng(np.random.SeedSequence(self._entropy, spawn_key=tuple(key)))

    # -- Zipf popularity (skewed config only) ------------------------------
    def zipf_ranks(self) -> np.ndarray:
        """rank_e in 1..E of each routed expert (1 = most popular)."""
        if self._zipf_cache is None:
            E = self.cfg.n_experts
            order = self.rng(_K_ZIPF).permutation(E)
            ranks = np.empty(E, dtype=np.int64)
            ranks[order] = np.arange(1, E + 1)
            self._zipf_cache = ranks
        return self._zipf_cache

    # -- dense fp16 tensors -------------------------------------------------
    def router_bits(self) -> np.ndarray:
        c = self.cfg
        w = self.rng(_K_WR).normal(0.0, 0.02, size=(c.n_experts, c.d_model))
        if c.zipf:
            p = self.zipf_ranks().astype(np.float64) ** (-ZIPF_S)
            p /= p.sum()
            w[:, 0] = ZIPF_TAU * np.log(p)
        return f16_bits(w)

    def delta_bits(self) -> np.ndarray:
        c = self.cfg
        return f16_bits(self.rng(_K_DWR).normal(0.0, 0.002, size=(c.n_experts, c.d_model)))

    def corr_a_bits(self) -> np.ndarray:
        c = self.cfg
        return f16_bits(self.rng(_K_A).normal(0.0, 0.01, size=(c.rank, c.d_model)))

    def corr_b_bits(self) -> np.ndarray:
        c = self.cfg
        return f16_bits(self.rng(_K_B).normal(0.0, 0.01, size=(c.d_model, c.rank)))

    def delta_factor_bits(self, rank: int):
        """(U [E, rank], V [rank, d]) fp16 bits of a factorised router delta;
        entries N(0, 0.02), so U V has a spread of about 0.02^2 sqrt(rank)
        (0.009 at rank 512, half the router weights')."""
        c = self.cfg
        u = self.rng(_K_DU, rank).normal(0.0, 0.02, size=(c.n_experts, rank))
        v = self.rng(_K_DV, rank).normal(0.0, 0.02, size=(rank, c.d_model))
        return f16_bits(u), f16_bits(v)

    # -- ternary-coded router delta and correction -----------------------------
    def _ternary(self, kind: int, rows: int, cols: int):
        u = self.rng(kind, 0).integers(0, 10, size=(rows, cols), dtype=np.uint8)
        s = np.abs(self.rng(kind, 1).normal(0.0, _Q_SIGMA[kind], size=(rows, cols // 128)))
        return _TRIT_LUT[u], f16_bits(s)

    def delta_q_parts(self):
        """(trits int8 [E, d], scale bits uint16 [E, d/128]) of a ternary-coded router delta."""
        c = self.cfg
        return self._ternary(_K_DWR_Q, c.n_experts, c.d_model)

    def corr_a_q_parts(self):
        """(trits [r, d], scale bits [r, d/128]) of a ternary-coded correction A."""
        c = self.cfg
        return self._ternary(_K_A_Q, c.rank, c.d_model)

    def corr_b_q_parts(self):
        """(trits [d, r], scale bits [d, r/128]) of a ternary-coded correction B."""
        c = self.cfg
        return self._ternary(_K_B_Q, c.d_model, c.rank)

    # -- expert banks -------------------------------------------------------
    def formats(self) -> np.ndarray:
        """uint8[E+S] container id per bank (routed experts first, then shared)."""
        c = self.cfg
        if c.fmt == "pq2_0":
            return np.full(c.n_banks, PQ2_0, dtype=np.uint8)
        if c.fmt == "ptq1_0":
            return np.full(c.n_banks, PTQ1_0, dtype=np.uint8)
        r = self.rng(_K_FMT).random(c.n_experts)
        f = np.where(r < 0.5, PQ2_0, PTQ1_0).astype(np.uint8)
        if c.zipf:
            ranks = self.zipf_ranks()
            f[ranks == 1] = PQ2_0
            f[ranks == 2] = PTQ1_0
        shared = np.full(c.n_shared, PTQ1_0, dtype=np.uint8)
        return np.concatenate([f, shared])

    def matrix_shapes(self):
        """(rows, cols) of gate, up, down; groups of 128 run along cols."""
        c = self.cfg
        return [(c.d_ff, c.d_model), (c.d_ff, c.d_model), (c.d_model, c.d_ff)]

    def expert_trits(self, e: int):
        """[gate, up, down] int8 trit matrices of bank e."""
        out = []
        for m, (rows, cols) in enumerate(self.matrix_shapes()):
            u = self.rng(_K_CODES, e, m).integers(0, 10, size=(rows, cols), dtype=np.uint8)
            out.append(_TRIT_LUT[u])
        return out

    def expert_scales(self, e: int):
        """[gate, up, down] uint16 fp16-bit scale matrices [rows, cols/128] of bank e."""
        out = []
        for m, (rows, cols) in enumerate(self.matrix_shapes()):
            s = np.abs(self.rng(_K_SCALES, e, m).normal(0.0, 0.02, size=(rows, cols // 128)))
            out.append(f16_bits(s))
        return out

    # -- activations ----------------------------------------------------------
    def tokens(self, n_tokens: int, set_index: int = 0) -> np.ndarray:
        """bf16 bits [T, d]: N(0,1); skewed config adds 1% x50 outliers and channel 0 = 1."""
        c = self.cfg
        x = self.rng(_K_X, set_index, n_tokens).normal(0.0, 1.0, size=(n_tokens, c.d_model))
        if c.outlier_frac > 0:
            mask = self.rng(_K_OUTL, set_index, n_tokens).random((n_tokens, c.d_model)) < c.outlier_frac
            x = np.where(mask, x * c.outlier_scale, x)
        if c.zipf:
            x[:, 0] = 1.0
        return bf16_bits(x)


def bank_byte_sizes(cfg: LayerConfig, formats: np.ndarray) -> np.ndarray:
    """Bytes of each bank's [gate | up | down] containers: 34 B (PQ2_0) or 28 B
    (PTQ1_0) per 128 weights.  Only the block sizes the cards print are used here."""
    per_block = np.where(formats == PQ2_0, 34, 28).astype(np.int64)
    n_blocks = 3 * cfg.d_ff * cfg.d_model // 128
    return per_block * n_blocks
