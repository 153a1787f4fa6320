"""Pins of the oracle draft head (oracle/mtp.py)."""
import numpy as np
from scipy import stats

from oracle import mtp
from synthetic import bf16_bits, f16_bits


def test_gelu_closed_forms():
    # gelu(v) = v Phi(v): Phi from an independent routine
    v = np.array([-3.0, -1.0, -0.25, 0.0, 0.5, 1.0, 2.5])
    assert np.allclose(mtp.gelu(v), v * stats.norm.cdf(v), rtol=0, atol=1e-15)
    assert abs(mtp.gelu(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15   # Phi(1)
    # gelu(v) - gelu(-v) = v exactly in real arithmetic; gelu'(0) = 1/2; large |v| limits
    w = np.linspace(-6, 6, 97)
    assert np.allclose(mtp.gelu(w) - mtp.gelu(-w), w, atol=1e-14)
    eps = 1e-6
    assert abs((mtp.gelu(np.array([eps]))[0] - mtp.gelu(np.array([-eps]))[0]) / (2 * eps) - 0.5) < 1e-9
    assert abs(mtp.gelu(np.array([40.0]))[0] - 40.0) < 1e-12 and abs(mtp.gelu(np.array([-40.0]))[0]) < 1e-12


def _head_inputs(T=3, h=8, m=16, seed=0):
    rng = np.random.default_rng(seed)
    return (bf16_bits(rng.standard_normal((T, h))), bf16_bits(rng.standard_normal((T, h))),
            f16_bits(rng.standard_normal((m, 2 * h)) * 0.3), f16_bits(rng.standard_normal(m) * 0.1),
            f16_bits(rng.standard_normal((h, m)) * 0.3), f16_bits(rng.standard_normal(h) * 0.1))


def test_head_structure():
    hid, emb, w1, b1, w2, b2 = _head_inputs()
    y = mtp.head(hid, emb, w1, b1, w2, b2)
    # W2 = 0 leaves the bias
    z = mtp.head(hid, emb, w1, b1, np.zeros_like(w2), b2)
    assert np.array_equal(z, np.tile(mtp.f16_to_f64(b2), (3, 1)))
    # the output is linear in (W2, b2): negating both (the fp16 sign bit) negates y
    assert np.array_equal(mtp.head(hid, emb, w1, b1, w2 ^ 0x8000, b2 ^ 0x8000), -y)
    # concatenation order: swapping hidden and embedding equals swapping W1's column halves
    h = hid.shape[1]
    w1s = np.concatenate([w1[:, h:], w1[:, :h]], axis=1)
    assert np.allclose(mtp.head(emb, hid, w1s, b1, w2, b2), y, rtol=0, atol=1e-12)
    # absent biases equal zero biases
    assert np.array_equal(mtp.head(hid, emb, w1, None, w2, None),
                          mtp.head(hid, emb, w1, np.zeros_like(b1), w2, np.zeros_like(b2)))


def test_head_brute_force_one_token():
    hid, emb, w1, b1, w2, b2 = _head_inputs(T=1, h=4, m=6, seed=3)
    x = np.concatenate([mtp.bf16_to_f64(hid[0]), mtp.bf16_to_f64(emb[0])])
    W1, W2 = mtp.f16_to_f64(w1), mtp.f16_to_f64(w2)
    want = []
    for i in range(4):
        acc = mtp.f16_to_f64(b2)[i]
        for j in range(6):
            a = sum(W1[j, k] * x[k] for k in range(8)) + mtp.f16_to_f64(b1)[j]
            acc += W2[i, j] * a * stats.norm.cdf(a)
        want.append(acc)
    assert np.allclose(mtp.head(hid, emb, w1, b1, w2, b2)[0], want, rtol=1e-13, atol=1e-13)
