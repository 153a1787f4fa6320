"""Pins of the oracle quantizer (oracle/quant.py) against what the mathematics fixes.

- Closed forms on iid N(0, 1) weights: the population relative error of the
  absmean rule (s = E|w| = sqrt(2/pi), threshold s/2) and of the Lloyd fixed
  point (threshold tau solving tau = phi(tau) / (2 (1 - Phi(tau)))), both by
  numerical integration here; 128-weight groups land within sampling noise.
  (The pages report 0.517 and 0.442 on real OLMoE experts; Gaussian weights
  are not those, so only the ordering and the closed forms are pinned.)
- Lloyd never increases a group's squared error, and ends on a fixed point.
- The code rule equals clamp(round(w / s), -1, 1) with ties to even.
- Special groups: zeros, exact ties, a single nonzero, saturation.
- Packing: the container decodes to scale * code.
"""
import math

import numpy as np
import pytest
from scipy import integrate, optimize, stats

from oracle import codec, quant


def bf16_bits(x):
    """float64 -> bfloat16 bits (round to nearest even through float32)."""
    f = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (f + 0x7FFF + ((f >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def gaussian_groups(n_groups, seed=0):
    rng = np.random.default_rng(seed)
    return bf16_bits(rng.standard_normal(n_groups * 128))


def rel_error(w_bits, t, s_bits):
    w = quant.bf16_to_f32(w_bits).astype(np.float64)
    s = codec.f16_to_f64(s_bits)
    what = np.repeat(s, 128) * t.astype(np.float64)
    return math.sqrt(np.sum((w - what) ** 2) / np.sum(w ** 2))


def population_rel_error(tau, s):
    """sqrt(E[(w - s t)^2]) for w ~ N(0,1), t = sign(w) [|w| > tau] (E[w^2] = 1)."""
    inner, _ = integrate.quad(lambda w: w * w * stats.norm.pdf(w), 0, tau)
    outer, _ = integrate.quad(lambda w: (w - s) ** 2 * stats.norm.pdf(w), tau, np.inf)
    return math.sqrt(2 * (inner + outer))


def test_absmean_matches_gaussian_closed_form():
    s = math.sqrt(2 / math.pi)
    want = population_rel_error(s / 2, s)
    w = gaussian_groups(4096)
    t, sb, _, _ = quant.quantize_groups(w, quant.ABSMEAN)
    got = rel_error(w, t, sb)
    assert abs(got - want) < 0.005


def test_lloyd_matches_gaussian_fixed_point():
    # fixed point of the population iteration: tau = s(tau) / 2, s(tau) = E[|w| | |w| > tau]
    f = lambda tau: tau - stats.norm.pdf(tau) / (2 * stats.norm.sf(tau))
    tau = optimize.brentq(f, 0.1, 2.0)
    s = 2 * tau
    want = population_rel_error(tau, s)
    w = gaussian_groups(4096, seed=1)
    t, sb, _, rounds = quant.quantize_groups(w, quant.LLOYD)
    got = rel_error(w, t, sb)
    assert abs(got - want) < 0.006
    # Lloyd beats absmean, as the pages report for real experts
    ta, sba, _, _ = quant.quantize_groups(w, quant.ABSMEAN)
    assert got < rel_error(w, ta, sba) - 0.05
    assert rounds.max() < quant.MAX_ROUNDS  # every group converged


def test_lloyd_error_never_increases_and_ends_on_fixed_point():
    w = gaussian_groups(512, seed=2)
    hist = []
    t, sb, s, _ = quant.quantize_groups(w, quant.LLOYD, history=hist)
    wf = quant.bf16_to_f32(w.reshape(-1, 128)).astype(np.float64)

    def sse(t_, s_):  # per group, float64, the exact error of that round's codes and scale
        return np.sum((wf - s_[:, None].astype(np.float64) * t_.astype(np.float64)) ** 2, axis=1)

    errs = [sse(tt, ss) for tt, ss in hist]
    for a, b in zip(errs, errs[1:]):
        assert np.all(b <= a * (1 + 1e-6) + 1e-12)
    t2 = t.reshape(-1, 128)
    # fixed point: the scale is the mean |w| of the nonzeros, the codes follow the scale
    assert np.array_equal(quant.codes_for(quant.bf16_to_f32(w.reshape(-1, 128)), s), t2)
    assert np.array_equal(quant.mean_of_nonzero(quant.bf16_to_f32(w.reshape(-1, 128)), t2), s)


def test_code_rule_is_round_to_nearest_even_of_w_over_s():
    w = gaussian_groups(256, seed=3)
    wf = quant.bf16_to_f32(w.reshape(-1, 128)).astype(np.float64)
    for method in (quant.ABSMEAN, quant.LLOYD):
        t, _, s, _ = quant.quantize_groups(w, method)
        ref = np.clip(np.round(wf / s[:, None].astype(np.float64)), -1, 1)  # numpy rounds ties to even
        assert np.array_equal(t.reshape(-1, 128), ref.astype(np.int8))


def test_special_groups():
    g_zero = np.zeros(128)
    g_tie = np.concatenate([np.full(64, 1.0), np.full(64, -3.0)])  # mean 2: |w| = 1 is a tie -> 0
    g_one = np.zeros(128)
    g_one[5] = -0.75  # mean 0.75/128: only the nonzero survives, Lloyd scale = 0.75
    g_big = np.full(128, 3.0e5)  # beyond binary16: the scale saturates
    w = bf16_bits(np.concatenate([g_zero, g_tie, g_one, g_big]))
    for method in (quant.ABSMEAN, quant.LLOYD):
        t, sb, s, _ = quant.quantize_groups(w, method)
        t = t.reshape(-1, 128)
        assert np.all(t[0] == 0) and sb[0] == 0
        assert np.all(t[1, :64] == 0) and np.all(t[1, 64:] == -1)
        assert np.count_nonzero(t[2]) == 1 and t[2, 5] == -1
        assert np.all(t[3] == 1) and sb[3] == quant.F16_MAX_BITS
    _, sb, s, _ = quant.quantize_groups(w, quant.ABSMEAN)
    assert s[1] == 2.0 and s[2] == np.float32(0.75 / 128)
    _, sb, s, _ = quant.quantize_groups(w, quant.LLOYD)
    assert s[1] == 3.0 and s[2] == 0.75  # the mean over the nonzeros


@pytest.mark.parametrize("fmt", [codec.PQ2_0, codec.PTQ1_0])
@pytest.mark.parametrize("method", [quant.ABSMEAN, quant.LLOYD])
def test_container_decodes_to_scale_times_code(fmt, method):
    w = gaussian_groups(64, seed=4)
    data = quant.quantize(fmt, w, method)
    assert data.size == 64 * codec.block_bytes(fmt)
    t, sb, _, _ = quant.quantize_groups(w, method)
    assert np.array_equal(codec.decode(fmt, data, w.size), np.repeat(codec.f16_to_f64(sb), 128) * t)


# --- the float32 decisions against the rule taken exactly --------------------
# The oracle decides codes in float32 with a fixed summation tree (its reading
# of the pages, which fix no precision).  Here the same rules are evaluated in
# float64 from the exact bfloat16 inputs: a group sum of 128 terms has a
# float32 relative error of at most 7 ulp-halves (seven tree levels, u = 2^-24)
# and the division one more, so a float32 decision can differ from the exact
# one only for weights whose 2|w| lies within 8u s of the exact scale s.  Away
# from that band the codes (and for Lloyd the round count) must be identical,
# and the stored binary16 scale must equal the exact scale's rounding unless
# that scale lies within the same band of a binary16 rounding boundary.
U = 2.0 ** -24
BAND = 8 * U


def exact_groups(w_bits, method):
    """Per group: codes (int8) and exact scale from the rules in float64, the
    rounds taken, and whether every decision was clear of the near-tie band."""
    w = quant.bf16_to_f32(np.asarray(w_bits).reshape(-1, 128)).astype(np.float64)
    a = np.abs(w)
    out_t, out_s, out_r, clear = [], [], [], []
    for g in range(w.shape[0]):
        s = math.fsum(a[g]) / 128.0
        ok = True

        def decide(s):
            nonlocal ok
            if s > 0 and np.any(np.abs(2 * a[g] - s) <= BAND * s):
                ok = False
            return np.where(2 * a[g] > s, np.sign(w[g]), 0.0).astype(np.int8)

        t = decide(s)
        rounds = 0
        if method == quant.LLOYD:
            for _ in range(32):  # the reading's cap of 32 rounds, restated here
                nz = t != 0
                s_new = math.fsum(a[g][nz]) / nz.sum() if nz.any() else 0.0
                t_new = decide(s_new)
                rounds += 1
                s = s_new
                if np.array_equal(t_new, t):
                    break
                t = t_new
            nz = t != 0
            s = math.fsum(a[g][nz]) / nz.sum() if nz.any() else 0.0
        out_t.append(t)
        out_s.append(s)
        out_r.append(rounds)
        clear.append(ok)
    return np.array(out_t), np.array(out_s), np.array(out_r), np.array(clear)


def f16_bits_of(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("method", [quant.ABSMEAN, quant.LLOYD])
def test_float32_decisions_equal_the_exact_rule_away_from_ties(method):
    rng = np.random.default_rng(11)
    n = 768
    w = np.concatenate([rng.standard_normal(n * 64), rng.laplace(size=n * 32), 0.01 * rng.standard_t(3, size=n * 32)])
    w_bits = bf16_bits(w)
    t32, s_bits, _, rounds32 = quant.quantize_groups(w_bits, method)
    t64, s64, rounds64, clear = exact_groups(w_bits, method)
    t32 = t32.reshape(-1, 128)
    assert clear.mean() > 0.9, clear.mean()
    assert np.array_equal(t32[clear], t64[clear])
    if method == quant.LLOYD:
        assert np.array_equal(rounds32[clear], rounds64[clear])
    # the binary16 scale, where the exact scale is clear of a rounding boundary
    lo, hi = f16_bits_of(s64 * (1 - BAND)), f16_bits_of(s64 * (1 + BAND))
    firm = clear & (lo == hi)
    assert firm.mean() > 0.9
    assert np.array_equal(s_bits[firm], f16_bits_of(s64)[firm])
