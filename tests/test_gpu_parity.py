"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Bars: bit-exact device decode, routing indices (decidable-tie rule: the GPU's
top-k equals the top-k of its own exported fp32 logits; each logit lies within
gamma = 8 sqrt(d) 2^-24 sum|w x| of the fp64 logit; tokens whose fp64 k/k+1
gap exceeds 2 gamma match the fp64 choice), counts/offsets/permutation, and
block outputs within max_j |dy_j| / ||y||_2 <= 2e-3 per token row.
"""
import sys

import numpy as np
import pytest

from layer_fixtures import Layer, logit_bound, row_metric
from oracle_threads import forward_y
from oracle import codec, moe as omoe
from synthetic import CONFIGS, PQ2_0, PTQ1_0, LayerConfig

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_quantized_moe_amd as tq
    tq.lib()
    return tq


def tq_mod():
    import ternary_quantized_moe_amd as tq
    return tq


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("fmt", [PQ2_0, PTQ1_0])
def test_unpack_device_bit_exact(fmt):
    tq = tq_mod()
    rng = np.random.default_rng(7 + fmt)
    n = 128 * 1037
    t = rng.integers(-1, 2, size=n).astype(np.int8)
    s = rng.normal(0, 1, n // 128).astype(np.float16)
    s[:4] = [0.0, -0.0, 6.0e-8, -65504.0]          # zero, negative zero, subnormal, extreme
    s_bits = s.view(np.uint16)
    data = codec.pack(fmt, t, s_bits)
    say(f"unpack_device fmt={fmt} n={n}")
    d_src = torch.from_numpy(data).cuda()
    dt, ds = tq.unpack_device(fmt, d_src, n)
    torch.cuda.synchronize()
    assert np.array_equal(dt.cpu().numpy(), t)
    assert np.array_equal(ds.cpu().numpy().view(np.uint16), s_bits)


@pytest.mark.parametrize("name", ["tiny", "skewed"])
def test_unpack_device_real_banks(name):
    tq = tq_mod()
    L = Layer(name)
    c = L.cfg
    for e in (0, c.n_banks - 1):
        fmt = int(L.formats[e])
        data = L.oracle_banks.container(e)
        n = 3 * c.d_model * c.d_ff
        say(f"unpack_device bank {e} of {name}")
        dt, ds = tq.unpack_device(fmt, torch.from_numpy(data).cuda(), n)
        torch.cuda.synchronize()
        trits, scales = L.source(e)
        assert np.array_equal(dt.cpu().numpy(), np.concatenate([a.reshape(-1) for a in trits]))
        assert np.array_equal(ds.cpu().numpy().view(np.uint16), np.concatenate([a.reshape(-1) for a in scales]))


def test_library_packing_equals_oracle_packing():
    """The device banks are the oracle's containers with each matrix in the
    tile-major block order ([row tile][group][row in tile], written here as a
    numpy reshape)."""
    tq = tq_mod()
    L = Layer("skewed")
    c = L.cfg
    data, offsets = L.host_bytes()
    shapes = [(c.d_ff, c.d_model), (c.d_ff, c.d_model), (c.d_model, c.d_ff)]
    for e in (0, 1, 250, 511, 512):
        ref = L.oracle_banks.container(e)
        fmt = int(L.formats[e])
        bb = tq.block_bytes(fmt)
        pos, mine = 0, data[offsets[e]:offsets[e] + ref.size]
        for rows, cols in shapes:
            n = rows * cols // 128 * bb
            G = cols // 128
            want = ref[pos:pos + n].reshape(rows // 16, 16, G, bb).transpose(0, 2, 1, 3).reshape(-1)
            assert np.array_equal(mine[pos:pos + n], want), e
            assert np.array_equal(tq.untile_container(fmt, mine[pos:pos + n], rows, cols), ref[pos:pos + n])
            pos += n


# ------------------------------------------------------------------ routing
def check_routing(L, x_bits, r, tokens, use_delta=True):
    """R1-R3 and grouping checks; returns the GPU indices (numpy)."""
    c = L.cfg
    k = c.top_k
    lg = r["logits"].cpu().numpy().astype(np.float64)
    idx = r["idx"].cpu().numpy().astype(np.int64)
    w = r["w"].cpu().numpy().astype(np.float64)
    # R1: indices are the top-k of the GPU's own logits (stable order: ties -> lower index)
    ref_idx = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    assert np.array_equal(idx, ref_idx)
    # grouping of the GPU indices is exact
    counts, offsets, perm = omoe.grouping(idx, c.n_experts)
    assert np.array_equal(r["counts"].cpu().numpy(), counts)
    assert np.array_equal(r["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(r["perm"].cpu().numpy(), perm)
    # R2 on the checked tokens
    x = omoe.bf16_to_f64(x_bits[tokens])
    wr = omoe.f16_to_f64(L.router) + (omoe.f16_to_f64(L.delta) if use_delta else 0.0)
    l64 = x @ wr.T
    gam = logit_bound(x, wr)
    assert np.all(np.abs(lg[tokens] - l64) <= gam)
    # R3: decidable tokens match the fp64 choice as a set
    srt = np.sort(l64, axis=1)[:, ::-1]
    gap = srt[:, k - 1] - (srt[:, k] if k < c.n_experts else -np.inf)
    decidable = gap > 2 * gam.max(axis=1)
    fp64_idx = np.argsort(-l64, axis=1, kind="stable")[:, :k]
    for j, t in enumerate(tokens):
        if decidable[j]:
            assert set(idx[t]) == set(fp64_idx[j]), t
    # gate weights: the softmax of the GPU's own fp32 logits at its indices, up to
    # fp32 exp/divide rounding ...
    w_own = omoe.gate_weights(lg, idx)
    assert np.all(np.abs(w - w_own) <= 1e-5 * w_own + 1e-9)
    # ... and within the propagated logit bound of the fp64 softmax:
    # |dw_i| <= w_i |dl_i - sum_j w_j dl_j| <= 2 w_i max_j |dl_j|
    w64 = omoe.gate_weights(l64, idx[tokens])
    bound = 2 * w64 * gam.max(axis=1, keepdims=True) + 1e-5 * w64 + 1e-9
    assert np.all(np.abs(w[tokens] - w64) <= bound)
    return idx, int((~decidable).sum())


# ("olmoe", 300): a large batch whose 96-token down units would not fit in LDS
# (f = 1024), so the down projection takes its own 64-token items
CASES = [("tiny", 16), ("olmoe", 1), ("olmoe", 8), ("olmoe", 64), ("olmoe", 300), ("a3b35", 1), ("a3b35", 32),
         ("a3b35", 4096), ("flashnext", 1), ("flashnext", 64), ("flashnext", 4096), ("skewed", 16384)]


def sample_tokens(T, n, seed=0):
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    return np.sort(np.concatenate([[0, T - 1], rng.choice(np.arange(1, T - 1), n - 2, replace=False)]))


# The large-batch expert kernels split each routed expert's run of slots in
# the permutation (and each shared expert's tokens) into work items: of ITEM
# positions for the gate/up projection, and for the down one the same items
# where their rows fit in shared memory, else items of HALF positions.
ITEM, HALF = 96, 64


def item_edge_tokens(counts, offsets, perm, T, k, n_shared, item=ITEM, half=HALF, hot=5):
    """Tokens where the large-batch expert kernels' work items begin and end.

    For the `hot` experts with the most slots: the first and last token of every
    gate/up and every down item; for every other expert with slots: its first
    and last token and the first token of its last item of either kind; for a
    shared expert: both sides of every item boundary of either kind."""
    counts = np.asarray(counts, np.int64)
    offsets = np.asarray(offsets, np.int64)

    def cuts(n):                      # offsets (within a run of n) where an item of either kind starts
        return sorted(set(range(0, n, item)) | set(range(0, n, half)))

    pos = set()
    for e in np.nonzero(counts)[0]:
        o, n = int(offsets[e]), int(counts[e])
        pos.update([o, o + n - 1, o + (n - 1) // item * item, o + (n - 1) // half * half])
    for e in np.argsort(-counts, kind="stable")[:hot]:
        o, n = int(offsets[e]), int(counts[e])
        for c in cuts(n):
            pos.update([o + c, o + max(c - 1, 0)])
        pos.add(o + n - 1)
    toks = {int(perm[p]) // k for p in pos}
    if n_shared:
        for c in cuts(T):
            toks.update([max(c - 1, 0), c])
        toks.add(T - 1)
    return np.array(sorted(toks), dtype=np.int64)


@pytest.mark.parametrize("name,T", CASES)
def test_forward_parity(name, T):
    """Every token is compared up to 4096 tokens.  At 16384 tokens (Zipf-skewed
    routing) the compared tokens are the edges of every work item and staged
    part of the five hottest experts (the hottest holds about 37x the mean
    load), the first and last token and last-item start of every expert, both
    sides of every shared expert item boundary, and 256 random tokens."""
    tq = tq_mod()
    L = Layer(name)
    c = L.cfg
    x_bits = L.gen.tokens(T, 1)
    say(f"forward parity {name} T={T}: packing banks")
    banks = L.device()
    d = L.tensors(x_bits)
    say(f"forward parity {name} T={T}: route + forward")
    r = tq.route(d["x"], d["router"], d["delta"], c.n_experts, c.top_k)
    y = tq.forward(d["x"], d["router"], d["delta"], banks, d["a"], d["b"], c.top_k)
    torch.cuda.synchronize()
    if T <= 4096:
        toks = np.arange(T)
    else:
        edges = item_edge_tokens(r["counts"].cpu().numpy(), r["offsets"].cpu().numpy(),
                                 r["perm"].cpu().numpy(), T, c.top_k, c.n_shared)
        toks = np.union1d(edges, sample_tokens(T, 256, seed=3))
        assert len(toks) >= 512
    idx, undecided = check_routing(L, x_bits, r, toks)
    say(f"  {len(toks)} tokens compared, {undecided} undecided (routing forced to the GPU's choice)")
    ref = forward_y(L, x_bits[toks], L.router, L.delta, L.corr_a, L.corr_b, c.top_k, idx[toks])
    y_bits = y.cpu().numpy().view(np.uint16)
    m = row_metric(y_bits[toks], ref)
    say(f"  max row metric {m.max():.3e}")
    assert m.max() <= TOL


SMALL_MIXED = LayerConfig("small_mixed", 21, 256, 24, 256, 3, 1, 32, "mixed")


def test_mixed_formats_with_shared_expert():
    tq = tq_mod()
    L = Layer(SMALL_MIXED)
    c = L.cfg
    assert set(L.formats[:-1]) == {PQ2_0, PTQ1_0}
    for T in (1, 5, 37, 300):
        x_bits = L.gen.tokens(T, 2)
        d = L.tensors(x_bits)
        say(f"mixed T={T}")
        r = tq.route(d["x"], d["router"], d["delta"], c.n_experts, c.top_k)
        y = tq.forward(d["x"], d["router"], d["delta"], L.device(), d["a"], d["b"], c.top_k)
        torch.cuda.synchronize()
        idx, _ = check_routing(L, x_bits, r, np.arange(T))
        ref = omoe.forward(x_bits, L.router, L.delta, L.oracle_banks, L.corr_a, L.corr_b, c.top_k,
                           forced_idx=idx)
        assert row_metric(y.cpu().numpy().view(np.uint16), ref.y).max() <= TOL


# Ragged shapes: d = 1152 (9 groups; the small-batch x-projection's last K slice
# is partial), E + r = 68 (a ragged last row tile), f = 384 (3 down groups),
# mixed formats with a shared expert; T = 37 and 64 take the 32-row combine
# blocks, the separate top-k launch and its z-fold blocks; T = 300 the prefill
# kernels, including the mixed-format down GEMM.
RAGGED = LayerConfig("ragged", 23, 1152, 44, 384, 3, 1, 24, "mixed")


@pytest.mark.parametrize("T", [1, 13, 37, 64, 300])
def test_ragged_shapes(T):
    tq = tq_mod()
    L = Layer(RAGGED)
    c = L.cfg
    x_bits = L.gen.tokens(T, 3)
    d = L.tensors(x_bits)
    say(f"ragged T={T}")
    r = tq.route(d["x"], d["router"], d["delta"], c.n_experts, c.top_k)
    y = tq.forward(d["x"], d["router"], d["delta"], L.device(), d["a"], d["b"], c.top_k)
    torch.cuda.synchronize()
    idx, _ = check_routing(L, x_bits, r, np.arange(T))
    ref = omoe.forward(x_bits, L.router, L.delta, L.oracle_banks, L.corr_a, L.corr_b, c.top_k,
                       forced_idx=idx)
    m = row_metric(y.cpu().numpy().view(np.uint16), ref.y)
    say(f"  max row metric {m.max():.3e}")
    assert m.max() <= TOL


MANY_EXPERTS = LayerConfig("many", 22, 256, 1000, 128, 9, 0, 16, "pq2_0")


@pytest.mark.parametrize("T", [20, 300])
def test_many_experts(T):
    """E = 1000 (> 512): the 16-logits-per-lane top-k, the grouping over up to
    1024 experts, and banks spread over a large buffer."""
    tq = tq_mod()
    L = Layer(MANY_EXPERTS)
    c = L.cfg
    x_bits = L.gen.tokens(T, 8)
    d = L.tensors(x_bits)
    say(f"many experts T={T}")
    r = tq.route(d["x"], d["router"], d["delta"], c.n_experts, c.top_k)
    y = tq.forward(d["x"], d["router"], d["delta"], L.device(), d["a"], d["b"], c.top_k)
    torch.cuda.synchronize()
    toks = np.arange(T)
    idx, _ = check_routing(L, x_bits, r, toks)
    ref = forward_y(L, x_bits, L.router, L.delta, L.corr_a, L.corr_b, c.top_k, idx)
    assert row_metric(y.cpu().numpy().view(np.uint16), ref).max() <= TOL


def run_fwd(L, x_bits, k=None, use_delta=True, use_corr=True, corr_b=None, banks=None):
    tq = tq_mod()
    d = L.tensors(x_bits, use_delta, use_corr, corr_b)
    y = tq.forward(d["x"], d["router"], d["delta"], banks or L.device(), d["a"], d["b"], k or L.cfg.top_k)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16)


def test_top1_and_all_experts():
    tq = tq_mod()
    L = Layer("tiny")
    x_bits = L.gen.tokens(16, 3)
    for k in (1, 8):
        say(f"tiny k={k}")
        d = L.tensors(x_bits)
        r = tq.route(d["x"], d["router"], d["delta"], 8, k)
        torch.cuda.synchronize()
        w = r["w"].cpu().numpy()
        if k == 1:
            assert np.all(w == 1.0)
        idx = r["idx"].cpu().numpy()
        y = run_fwd(L, x_bits, k=k)
        ref = omoe.forward(x_bits, L.router, L.delta, L.oracle_banks, L.corr_a, L.corr_b, k, forced_idx=idx)
        assert row_metric(y, ref.y).max() <= TOL


def test_zero_tokens_is_a_noop():
    tq = tq_mod()
    L = Layer("tiny")
    d = L.tensors(L.gen.tokens(0))
    y = tq.forward(d["x"], d["router"], d["delta"], L.device(), d["a"], d["b"], 2)
    torch.cuda.synchronize()
    assert y.shape[0] == 0


# 16 tokens take the small-batch kernels, 300 the large-batch (LDS-tiled) ones
@pytest.mark.parametrize("T", [16, 300])
def test_zero_codes_leave_only_the_correction(T):
    L = Layer("tiny", zero_banks=True)
    x_bits = L.gen.tokens(T, 4)
    y = run_fwd(L, x_bits)
    x = omoe.bf16_to_f64(x_bits)
    ref = omoe.correction(x, omoe.f16_to_f64(L.corr_a), omoe.f16_to_f64(L.corr_b))
    assert row_metric(y, ref).max() <= TOL
    # an all-zero group's scale does not matter: flip every scale's sign bit
    L2 = Layer("tiny", zero_banks=True, key=("tiny-zero-flipped",))
    L2.source = lambda e: ([np.zeros_like(t) for t in L.gen.expert_trits(e)],
                           [s ^ np.uint16(0x8000) for s in L.gen.expert_scales(e)])
    assert np.array_equal(run_fwd(L2, x_bits), y)


@pytest.mark.parametrize("T", [8, 300])
def test_zero_correction_equals_uncorrected_bit_exact(T):
    L = Layer("olmoe")
    x_bits = L.gen.tokens(T, 5)
    y_none = run_fwd(L, x_bits, use_corr=False)
    y_zero = run_fwd(L, x_bits, corr_b=np.zeros_like(L.corr_b))
    assert np.array_equal(y_none, y_zero)
    y_corr = run_fwd(L, x_bits)
    assert not np.array_equal(y_none, y_corr)
    assert not np.array_equal(run_fwd(L, x_bits, use_delta=False), y_corr)


@pytest.mark.parametrize("T", [16, 300])
def test_doubling_down_scales_doubles_output_bit_exact(T):
    L = Layer("tiny")
    x_bits = L.gen.tokens(T, 6)
    y1 = run_fwd(L, x_bits, use_corr=False)
    L2 = Layer("tiny", key=("tiny-down-doubled",))

    def doubled(e):
        trits, scales = L.gen.expert_trits(e), L.gen.expert_scales(e)
        d2 = (scales[2].view(np.float16).astype(np.float32) * 2).astype(np.float16).view(np.uint16)
        return trits, [scales[0], scales[1], d2]
    L2.source = doubled
    y2 = run_fwd(L2, x_bits, use_corr=False)
    f1 = omoe.bf16_to_f64(y1)
    f2 = omoe.bf16_to_f64(y2)
    assert np.array_equal(f2, 2 * f1)


@pytest.mark.parametrize("T", [64, 300])
def test_deterministic_and_token_independent(T):
    tq = tq_mod()
    L = Layer("olmoe")
    x_bits = L.gen.tokens(T, 7)
    y1 = run_fwd(L, x_bits)
    y2 = run_fwd(L, x_bits)
    assert np.array_equal(y1, y2)
    d = L.tensors(x_bits)
    r1 = tq.route(d["x"], d["router"], d["delta"], 64, 8)
    r2 = tq.route(d["x"], d["router"], d["delta"], 64, 8)
    torch.cuda.synchronize()
    for key in ("logits", "idx", "w", "counts", "offsets", "perm"):
        assert torch.equal(r1[key], r2[key]), key
    for t in (0, 31, T - 1):
        yt = run_fwd(L, x_bits[t:t + 1])
        ref = omoe.bf16_to_f64(y1[t:t + 1])
        m = np.abs(omoe.bf16_to_f64(yt) - ref).max() / np.linalg.norm(ref)
        assert m <= TOL
