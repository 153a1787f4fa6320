"""Shared set-up for the GPU parity tests: one synthetic layer, packed twice.

The oracle side packs each bank with the oracle codec (oracle.moe.LazyBanks);
the product side packs with the library's moe_pack and uploads.  Both start
from the same seeded trits and scale bits (synthetic.LayerGen), and a test
checks the two packings agree byte for byte.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import moe as omoe
from synthetic import CONFIGS, LayerConfig, LayerGen

_DEVICE_CACHE = {}


class Layer:
    def __init__(self, cfg, zero_banks=False, formats=None, key=None):
        self.cfg = CONFIGS[cfg] if isinstance(cfg, str) else cfg
        self.gen = LayerGen(self.cfg)
        self.formats = self.gen.formats() if formats is None else np.asarray(formats, np.uint8)
        self.zero_banks = zero_banks
        self.router = self.gen.router_bits()
        self.delta = self.gen.delta_bits()
        self.corr_a = self.gen.corr_a_bits()
        self.corr_b = self.gen.corr_b_bits()
        c = self.cfg
        self.key = key or (c.name, c.index, zero_banks, self.formats.tobytes())
        self.oracle_banks = omoe.LazyBanks(self.source, self.formats, c.d_model, c.d_ff, c.n_experts,
                                           c.n_shared)

    def source(self, e):
        trits, scales = self.gen.expert_trits(e), self.gen.expert_scales(e)
        if self.zero_banks:
            trits = [np.zeros_like(t) for t in trits]
        return trits, scales

    # ---- product side ----------------------------------------------------------
    def device(self):
        """ExpertBanks on cuda:0, packed by the library (cached per layer key)."""
        if self.key not in _DEVICE_CACHE:
            import ternary_quantized_moe_amd as tq
            c = self.cfg
            data, offsets = tq.build_banks(self.source, c.n_banks, self.formats, c.d_model, c.d_ff)
            _DEVICE_CACHE[self.key] = (tq.ExpertBanks(data, offsets, self.formats, c.d_model, c.d_ff,
                                                      c.n_experts, c.n_shared), data, offsets)
        return _DEVICE_CACHE[self.key][0]

    def host_bytes(self):
        self.device()
        return _DEVICE_CACHE[self.key][1], _DEVICE_CACHE[self.key][2]

    def tensors(self, x_bits, use_delta=True, use_corr=True, corr_b=None):
        import torch
        dev = torch.device("cuda:0")
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
        b = self.corr_b if corr_b is None else corr_b
        return dict(x=t(x_bits), router=t(self.router), delta=t(self.delta) if use_delta else None,
                    a=t(self.corr_a) if use_corr else None, b=t(b) if use_corr else None)


def row_metric(y_gpu_bits, y_ref):
    """max_j |y_gpu - y_ref| / ||y_ref||_2 per token row."""
    y = omoe.bf16_to_f64(y_gpu_bits)
    num = np.abs(y - y_ref).max(axis=1)
    den = np.linalg.norm(y_ref, axis=1)
    return num / np.maximum(den, 1e-300)


def logit_bound(x, w):
    """gamma[t, e] = 8 sqrt(d) 2^-24 sum_j |w[e, j] x[t, j]| (probabilistic fp32 bound)."""
    d = x.shape[1]
    return 8.0 * math.sqrt(d) * 2.0 ** -24 * (np.abs(x) @ np.abs(w).T)
