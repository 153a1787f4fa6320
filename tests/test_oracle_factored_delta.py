"""Pins of the oracle's factorised router delta, dW_r = U V (FlashNext card,
"Weight Representation": rank-512 F16 factors), against the dense delta it
stands for, a closed form and an exact invariance."""
import numpy as np
import pytest

from oracle import moe
from synthetic import CONFIGS, f16_bits

from test_oracle_forward import build_layer, run

TINY = CONFIGS["tiny"]


def _factors(E, d, rd, seed):
    rng = np.random.default_rng(seed)
    return f16_bits(rng.normal(scale=0.05, size=(E, rd))), f16_bits(rng.normal(scale=0.05, size=(rd, d)))


def test_selection_factors_equal_the_dense_delta():
    """U = [I 0] picks the first E rows of V: U V is exactly those rows."""
    L = build_layer(TINY)
    E, d = TINY.n_experts, TINY.d_model
    rd = E + 8
    u = np.zeros((E, rd), np.uint16)
    u[np.arange(E), np.arange(E)] = 0x3C00                       # fp16 1.0
    _, v = _factors(E, d, rd, 1)
    v[:E] = L["dwr"]
    dense = run(L)
    fact = run(L, delta_bits=None, delta_factors=(u, v))
    assert np.array_equal(fact.logits, dense.logits)
    assert np.array_equal(fact.idx, dense.idx)
    assert np.array_equal(fact.y, dense.y)


def test_rank_one_delta_closed_form():
    """rd = 1: the delta adds u_e (v . x) to logit e, summed here by a loop."""
    L = build_layer(TINY, n_tokens=3)
    E, d = TINY.n_experts, TINY.d_model
    u, v = _factors(E, d, 1, 2)
    base = run(L, delta_bits=None).logits
    got = run(L, delta_bits=None, delta_factors=(u, v)).logits
    x = moe.bf16_to_f64(L["x"])
    uf, vf = moe.f16_to_f64(u)[:, 0], moe.f16_to_f64(v)[0]
    for t in range(3):
        dot = 0.0
        for j in range(d):
            dot += vf[j] * x[t, j]
        for e in range(E):
            assert abs(got[t, e] - (base[t, e] + uf[e] * dot)) <= 1e-12 * (1 + abs(base[t, e]))


def test_factor_rescaling_leaves_the_block_unchanged():
    """(2U)(V/2) = U V exactly: powers of two rescale fp16 (away from its
    subnormals, so magnitudes here are at least 0.01) and float64 exactly."""
    L = build_layer(TINY)
    E, d = TINY.n_experts, TINY.d_model
    rng = np.random.default_rng(3)
    mag = lambda shape: rng.uniform(0.01, 0.1, size=shape) * rng.choice([-1.0, 1.0], size=shape)
    u, v = f16_bits(mag((E, 16))), f16_bits(mag((16, d)))
    u2 = f16_bits(moe.f16_to_f64(u) * 2)
    v2 = f16_bits(moe.f16_to_f64(v) / 2)
    a = run(L, delta_bits=None, delta_factors=(u, v))
    b = run(L, delta_bits=None, delta_factors=(u2, v2))
    assert np.array_equal(a.logits, b.logits) and np.array_equal(a.y, b.y)


def test_dense_and_factored_delta_together_is_an_error():
    L = build_layer(TINY)
    u, v = _factors(TINY.n_experts, TINY.d_model, 8, 4)
    with pytest.raises(ValueError):
        run(L, delta_factors=(u, v))
