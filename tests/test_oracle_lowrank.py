"""Pins of the oracle's stand-alone rank-r branch (oracle.moe.lowrank_apply)."""
import numpy as np

from oracle import moe as omoe
from synthetic import bf16_bits, f16_bits


def _inputs(T=3, d=8, r=4, seed=0):
    rng = np.random.default_rng(seed)
    return (bf16_bits(rng.standard_normal((T, d))), bf16_bits(rng.standard_normal((T, d))),
            f16_bits(rng.standard_normal((r, d)) * 0.5), f16_bits(rng.standard_normal((d, r)) * 0.5))


def test_zero_factors_leave_y():
    x, y, a, b = _inputs()
    assert np.array_equal(omoe.lowrank_apply(x, y, np.zeros_like(a), b), omoe.bf16_to_f64(y))
    assert np.array_equal(omoe.lowrank_apply(x, y, a, np.zeros_like(b)), omoe.bf16_to_f64(y))
    assert np.array_equal(omoe.lowrank_apply(x, None, a, np.zeros_like(b)), np.zeros((3, 8)))


def test_one_hot_input_is_a_column_product():
    x, y, a, b = _inputs(T=1, d=6, r=3, seed=1)
    j = 4
    xj = bf16_bits(np.eye(1, 6, j))
    A, B = omoe.f16_to_f64(a), omoe.f16_to_f64(b)
    want = [omoe.bf16_to_f64(y)[0, i] + sum(B[i, c] * A[c, j] for c in range(3)) for i in range(6)]
    assert np.allclose(omoe.lowrank_apply(xj, y, a, b)[0], want, rtol=0, atol=1e-14)


def test_branch_is_linear_in_b_and_x():
    x, y, a, b = _inputs(seed=2)
    base = omoe.lowrank_apply(x, None, a, b)
    assert np.array_equal(omoe.lowrank_apply(x, None, a, b ^ 0x8000), -base)          # -B
    assert np.array_equal(omoe.lowrank_apply(x ^ 0x8000, None, a, b), -base)          # -x
    b2 = (omoe.f16_to_f64(b) * 2).astype(np.float16).view(np.uint16)
    assert np.allclose(omoe.lowrank_apply(x, None, a, b2), 2 * base, rtol=1e-15, atol=0)
