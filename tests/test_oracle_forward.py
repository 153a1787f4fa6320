"""Pins for the oracle's forward pass (CPU only).

Each pin fixes part of the oracle by something other than its own code: library
routines (stable sorts, scipy's softmax and expit), brute force without grouping,
closed forms built by selection rather than summation, and invariants the
definition implies (zero codes, zero correction, relabelling, scale linearity,
token independence).
"""
import numpy as np
import pytest
from scipy.special import expit, softmax

from oracle import codec, moe
from synthetic import CONFIGS, PQ2_0, PTQ1_0, LayerConfig, LayerGen, f16_bits


def build_layer(cfg, fmt_override=None, zero_banks=False, n_tokens=16, set_index=0):
    g = LayerGen(cfg)
    formats = g.formats() if fmt_override is None else fmt_override
    parts = []
    for e in range(cfg.n_banks):
        trits = g.expert_trits(e)
        if zero_banks:
            trits = [np.zeros_like(t) for t in trits]
        parts.append((trits, g.expert_scales(e)))
    banks = moe.pack_banks(parts, formats, cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.n_shared)
    return dict(x=g.tokens(n_tokens, set_index), wr=g.router_bits(), dwr=g.delta_bits(),
                a=g.corr_a_bits(), b=g.corr_b_bits(), banks=banks, k=cfg.top_k, gen=g,
                parts=parts)


SMALL_SHARED = LayerConfig("small_shared", 11, 256, 12, 128, 3, 1, 32, "mixed")
TINY = CONFIGS["tiny"]


def run(L, **kw):
    args = dict(x_bits=L["x"], router_bits=L["wr"], delta_bits=L["dwr"], banks=L["banks"],
                a_bits=L["a"], b_bits=L["b"], top_k=L["k"])
    args.update(kw)
    return moe.forward(**args)


# ---- routing pieces against library routines ------------------------------------
def test_topk_matches_stable_argsort_with_ties():
    rng = np.random.default_rng(3)
    l = rng.normal(size=(40, 17)).round(1)          # many exact ties
    l[0, :] = 0.0
    l[1, 3], l[1, 5] = -0.0, 0.0                    # -0.0 ties +0.0
    for k in (1, 4, 17):
        got = moe.select_topk(l, k)
        ref = np.argsort(-l, axis=1, kind="stable")[:, :k]
        assert np.array_equal(got, ref)
    assert list(moe.select_topk(l[:1], 3)[0]) == [0, 1, 2]


def test_gate_weights_are_renormalised_full_softmax():
    rng = np.random.default_rng(4)
    l = rng.normal(scale=3, size=(25, 9))
    idx = moe.select_topk(l, 3)
    p = softmax(l, axis=1)
    sel = np.take_along_axis(p, idx, axis=1)
    assert np.allclose(moe.gate_weights(l, idx), sel / sel.sum(axis=1, keepdims=True), rtol=1e-13)


def test_grouping_matches_stable_sort_by_expert():
    rng = np.random.default_rng(5)
    l = rng.normal(size=(33, 7))
    idx = moe.select_topk(l, 3)
    counts, offsets, perm = moe.grouping(idx, 7)
    assert np.array_equal(counts, np.bincount(idx.reshape(-1), minlength=7))
    assert offsets[0] == 0 and offsets[-1] == 33 * 3
    assert np.array_equal(perm, np.argsort(idx.reshape(-1), kind="stable"))


def test_silu_matches_expit():
    g = np.linspace(-30, 30, 1001)
    assert np.allclose(moe.silu(g), g * expit(g), rtol=1e-14, atol=1e-300)


# ---- brute force (no grouping) ---------------------------------------------------
@pytest.mark.parametrize("cfg", [TINY, SMALL_SHARED])
def test_bruteforce_equals_grouped(cfg):
    L = build_layer(cfg)
    r = run(L)
    y_bf = moe.forward_bruteforce(L["x"], L["wr"], L["dwr"], L["banks"], L["a"], L["b"], L["k"])
    assert np.allclose(r.y, y_bf, rtol=1e-12, atol=1e-13)
    assert not np.allclose(r.y, 0)


# ---- closed form by selection: d = f = 128, one expert, k = 1, x = e_j -----------
def test_closed_form_single_expert_unit_input():
    cfg = LayerConfig("unit", 12, 128, 1, 128, 1, 0, 4, "pq2_0")
    g = LayerGen(cfg)
    trits, scales = g.expert_trits(0), g.expert_scales(0)
    for fmt in (PQ2_0, PTQ1_0):
        banks = moe.pack_banks([(trits, scales)], np.array([fmt], np.uint8), 128, 128, 1, 0)
        j = 37
        x = np.zeros((1, 128), dtype=np.uint16)
        x[0, j] = 0x3F80                               # bf16 1.0
        a = np.zeros((4, 128), dtype=np.uint16)
        b = np.zeros((128, 4), dtype=np.uint16)
        a[2, j] = 0x4000                               # fp16 2.0: z_2 = 2
        b[90, 2] = 0x3800                              # fp16 0.5: y_90 += 0.5 * z_2
        r = moe.forward(x, g.router_bits(), None, banks, a, b, 1)
        sg = scales[0].view(np.float16).astype(np.float64)
        su = scales[1].view(np.float16).astype(np.float64)
        sd = scales[2].view(np.float16).astype(np.float64)
        expect = np.zeros(128)
        for i in range(128):                            # gate/up row i reads column j only
            gi = sg[i, j // 128] * trits[0][i, j]
            ui = su[i, j // 128] * trits[1][i, j]
            hi = gi * expit(gi) * ui
            for n in range(128):
                expect[n] += sd[n, i // 128] * trits[2][n, i] * hi
        expect[90] += 0.5 * 2.0
        assert r.w[0, 0] == 1.0
        assert np.allclose(r.y[0], expect, rtol=1e-13, atol=1e-15)


# ---- invariants -------------------------------------------------------------------
def test_zero_codes_leave_only_the_correction():
    L = build_layer(SMALL_SHARED, zero_banks=True)
    r = run(L)
    x = moe.bf16_to_f64(L["x"])
    a, b = moe.f16_to_f64(L["a"]), moe.f16_to_f64(L["b"])
    assert np.allclose(r.y, (x @ a.T) @ b.T, rtol=1e-13, atol=1e-15)
    # the scale of an all-zero group does not matter
    parts = [([t for t in tr], [np.full_like(s, 0xC400) for s in sc]) for tr, sc in L["parts"]]
    parts = [([np.zeros_like(t) for t in tr], sc) for tr, sc in parts]
    banks2 = moe.pack_banks(parts, L["banks"].formats, 256, 128, 12, 1)
    assert np.array_equal(run(L, banks=banks2).y, r.y)


def test_zero_correction_is_the_uncorrected_block():
    L = build_layer(SMALL_SHARED)
    r_none = run(L, a_bits=None, b_bits=None)
    r_zero = run(L, b_bits=np.zeros_like(L["b"]))
    assert np.array_equal(r_none.y, r_zero.y)
    assert not np.allclose(run(L).y, r_none.y)


def test_delta_cancelling_router_picks_lowest_experts_uniformly():
    L = build_layer(SMALL_SHARED)
    neg = L["wr"] ^ np.uint16(0x8000)               # dW_r = -W_r exactly
    r = run(L, delta_bits=neg)
    assert np.all(r.logits == 0.0)
    assert np.array_equal(r.idx, np.tile(np.arange(3), (16, 1)))
    assert np.all(r.w == 1.0 / 3.0)
    # and a zero delta equals no delta
    assert np.array_equal(run(L, delta_bits=np.zeros_like(L["dwr"])).y, run(L, delta_bits=None).y)


def test_top1_has_unit_weight():
    L = build_layer(SMALL_SHARED)
    r = run(L, top_k=1)
    assert np.all(r.w == 1.0)


def test_token_independence():
    L = build_layer(SMALL_SHARED, n_tokens=9)
    r = run(L)
    for t in (0, 4, 8):
        rt = run(L, x_bits=L["x"][t:t + 1])
        assert np.allclose(rt.y[0], r.y[t], rtol=1e-13, atol=1e-15)


def test_expert_relabelling_invariance():
    cfg = SMALL_SHARED
    L = build_layer(cfg)
    E = cfg.n_experts
    p = np.random.default_rng(6).permutation(E)     # new expert p[e] is old expert e
    inv = np.argsort(p)
    wr = L["wr"][inv]
    dwr = L["dwr"][inv]
    parts = [L["parts"][inv[e]] for e in range(E)] + L["parts"][E:]
    fmts = np.concatenate([L["banks"].formats[:E][inv], L["banks"].formats[E:]])
    banks = moe.pack_banks(parts, fmts, cfg.d_model, cfg.d_ff, E, cfg.n_shared)
    r0, r1 = run(L), run(L, router_bits=wr, delta_bits=dwr, banks=banks)
    assert np.array_equal(p[r0.idx], r1.idx)
    assert np.allclose(r0.y, r1.y, rtol=1e-12, atol=1e-14)


def test_doubling_down_scales_doubles_the_moe_part():
    L = build_layer(SMALL_SHARED)
    parts2 = []
    for tr, sc in L["parts"]:
        d2 = f16_bits(2.0 * sc[2].view(np.float16).astype(np.float64))
        parts2.append((tr, [sc[0], sc[1], d2]))
    banks2 = moe.pack_banks(parts2, L["banks"].formats, 256, 128, 12, 1)
    y1 = run(L, a_bits=None, b_bits=None).y
    y2 = run(L, a_bits=None, b_bits=None, banks=banks2).y
    assert np.allclose(y2, 2.0 * y1, rtol=1e-13, atol=1e-15)


def test_forced_routing_is_used():
    L = build_layer(TINY)
    r = run(L)
    forced = r.idx[:, ::-1].copy()
    rf = run(L, forced_idx=forced)
    assert np.array_equal(rf.idx, forced)
    assert np.allclose(rf.y, r.y, rtol=1e-12, atol=1e-14)  # same set, order only


# ---- the skewed workload really is skewed -----------------------------------------
def test_skewed_config_has_hot_experts():
    cfg = CONFIGS["skewed"]
    g = LayerGen(cfg)
    x = moe.bf16_to_f64(g.tokens(4096))
    l = moe.router_logits(x, moe.f16_to_f64(g.router_bits()), moe.f16_to_f64(g.delta_bits()))
    idx = np.argsort(-l, axis=1, kind="stable")[:, :cfg.top_k]
    load = np.bincount(idx.reshape(-1), minlength=cfg.n_experts)
    ratio = load.max() / load.mean()
    assert ratio > 20, ratio
    assert (load == 0).any()
    hottest = int(np.argmax(load))
    assert g.zipf_ranks()[hottest] == 1
    assert g.formats()[hottest] == PQ2_0


@pytest.mark.parametrize("cfg", [TINY, SMALL_SHARED])
def test_bank_subsets_add_up_to_the_block(cfg):
    """forward(..., banks_subset=P) over a partition P of the banks, plus the
    correction, equals the brute-force block (every expert on every token, then
    masked), which has no grouping and no subsets."""
    L = build_layer(cfg, n_tokens=24, set_index=3)
    ref = moe.forward_bruteforce(L["x"], L["wr"], L["dwr"], L["banks"], L["a"], L["b"], L["k"])
    nb = cfg.n_banks
    parts = [list(range(0, nb, 3)), list(range(1, nb, 3)), list(range(2, nb, 3))]
    y = moe.correction(moe.bf16_to_f64(L["x"]), moe.f16_to_f64(L["a"]), moe.f16_to_f64(L["b"]))
    for p in parts:
        y = y + run(L, banks_subset=p).y
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-13)
    # an empty subset contributes nothing and leaves out the correction
    assert not run(L, banks_subset=[]).y.any()


def test_threaded_oracle_equals_one_call():
    """tests/oracle_threads.py splits the banks over threads; the sum equals one
    serial oracle call."""
    from layer_fixtures import Layer
    from oracle_threads import forward_y
    L = Layer(SMALL_SHARED)
    c = L.cfg
    x = L.gen.tokens(40, 5)
    ref = moe.forward(x, L.router, L.delta, L.oracle_banks, L.corr_a, L.corr_b, c.top_k)
    y = forward_y(L, x, L.router, L.delta, L.corr_a, L.corr_b, c.top_k, ref.idx, threads=4)
    assert np.allclose(y, ref.y, rtol=1e-12, atol=1e-13)
