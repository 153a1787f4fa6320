"""GPU tests of the forward pass with the router delta given as two low-rank
fp16 factors U, V (moe_ternary_forward_factored), through the C ABI.

The bars: with U = 0 the block equals bit for bit the block without a delta
(decode and large-batch paths); the routing that moe_route_factored exports
(the same kernels the forward pass runs) selects the top-k of its own fp32
logits, groups them exactly, keeps every logit within the fp32 bound of the
oracle's W_r x + U V x, and matches the oracle's choice wherever that bound
decides it; the block output of every token is within the block tolerance of
the oracle with the routing forced to the GPU's choice; a token's output does
not depend on its batch.
"""
import sys

import numpy as np
import pytest

from layer_fixtures import Layer, row_metric
from oracle_threads import forward_y
from oracle import moe as omoe
from synthetic import LayerConfig

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


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def bits(t):
    return t.cpu().numpy().view(np.uint16)


def factored_bound(x, wr, uf, vf):
    """gamma[t, e]: the fp32 bound 8 sqrt(K) 2^-24 sum |w x| of W_r x (K = d)
    plus that of U (V x) (K = d and rank, through |U| |V| |x|)."""
    d, rd = wr.shape[1], uf.shape[1]
    eps = 8 * 2.0 ** -24
    return eps * np.sqrt(d) * (np.abs(x) @ np.abs(wr).T) + \
        eps * (np.sqrt(d) + np.sqrt(rd)) * ((np.abs(x) @ np.abs(vf).T) @ np.abs(uf).T)


def check_factored_routing(L, x_bits, u, v, r):
    """R1-R3 on every token against the oracle's logits W_r x + U V x; returns
    the GPU's indices and the number of tokens the bound leaves undecided."""
    c = L.cfg
    k = c.top_k
    lg = r["logits"].cpu().numpy().astype(np.float64)
    idx = r["idx"].cpu().numpy().astype(np.int64)
    assert np.array_equal(idx, np.argsort(-lg, axis=1, kind="stable")[:, :k])       # R1
    counts, offsets, perm = omoe.grouping(idx, c.n_experts)
    assert np.array_equal(r["counts"].cpu().numpy(), counts)
    assert np.array_equal(r["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(r["perm"].cpu().numpy(), perm)
    x = omoe.bf16_to_f64(x_bits)
    wr, uf, vf = omoe.f16_to_f64(L.router), omoe.f16_to_f64(u), omoe.f16_to_f64(v)
    l64 = x @ (wr + uf @ vf).T
    gam = factored_bound(x, wr, uf, vf)
    assert np.all(np.abs(lg - l64) <= gam)                                              # R2
    undecided = 0
    for t in range(len(x)):                                                             # R3
        sel = np.zeros(c.n_experts, bool)
        sel[omoe.select_topk(l64[t:t + 1], k)[0]] = True
        if sel.all() or (l64[t, sel] - 2 * gam[t, sel]).min() > (l64[t, ~sel] + 2 * gam[t, ~sel]).max():
            assert set(idx[t]) == set(np.nonzero(sel)[0]), t
        else:
            undecided += 1
    w = r["w"].cpu().numpy().astype(np.float64)
    w_own = omoe.gate_weights(lg, idx)
    assert np.all(np.abs(w - w_own) <= 1e-5 * w_own + 1e-9)
    return idx, undecided


def run_factored(L, x_bits, rank):
    import ternary_quantized_moe_amd as tq
    c = L.cfg
    u, v = L.gen.delta_factor_bits(rank)
    d = L.tensors(x_bits, use_delta=False)
    du, dv = dev16(u), dev16(v)
    r = tq.route_factored(d["x"], d["router"], du, dv, c.n_experts, c.top_k)
    y = tq.forward_factored(d["x"], d["router"], du, dv, L.device(), d["a"], d["b"], c.top_k)
    torch.cuda.synchronize()
    idx, undecided = check_factored_routing(L, x_bits, u, v, r)
    say(f"  {len(x_bits)} tokens, {undecided} undecided (routing forced to the GPU's choice)")
    ref = forward_y(L, x_bits, L.router, None, L.corr_a, L.corr_b, c.top_k, idx, delta_factors=(u, v))
    return bits(y), ref


RANK = {"tiny": 64, "olmoe": 512, "a3b35": 512, "flashnext": 512}


@pytest.mark.parametrize("name,T", [("tiny", 16), ("olmoe", 1), ("olmoe", 64), ("flashnext", 37),
                                    ("flashnext", 64), ("a3b35", 300), ("flashnext", 4096)])
def test_factored_delta_against_the_oracle(name, T):
    L = Layer(name)
    say(f"factored delta {name} T={T} rank={RANK[name]}")
    y, ref = run_factored(L, L.gen.tokens(T, 7), RANK[name])
    m = row_metric(y, ref)
    say(f"  max row metric {m.max():.3e}")
    assert m.max() <= TOL


@pytest.mark.parametrize("name,T", [("olmoe", 8), ("flashnext", 64), ("a3b35", 300)])
def test_zero_factor_equals_no_delta(name, T):
    import ternary_quantized_moe_amd as tq
    L = Layer(name)
    c = L.cfg
    u, v = L.gen.delta_factor_bits(RANK[name])
    u = np.zeros_like(u)
    x_bits = L.gen.tokens(T, 8)
    say(f"zero U {name} T={T}")
    d = L.tensors(x_bits, use_delta=False)
    y_f = tq.forward_factored(d["x"], d["router"], dev16(u), dev16(v), L.device(), d["a"], d["b"], c.top_k)
    y_n = tq.forward(d["x"], d["router"], None, L.device(), d["a"], d["b"], c.top_k)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y_f), bits(y_n))


def test_factored_delta_batch_independence():
    import ternary_quantized_moe_amd as tq
    L = Layer("olmoe")
    c = L.cfg
    u, v = L.gen.delta_factor_bits(512)
    x_bits = L.gen.tokens(40, 9)
    du, dv = dev16(u), dev16(v)
    full = L.tensors(x_bits, use_delta=False)
    part = L.tensors(x_bits[7:15], use_delta=False)   # 8 tokens: the same kernels as 40
    y_full = tq.forward_factored(full["x"], full["router"], du, dv, L.device(), full["a"], full["b"], c.top_k)
    y_part = tq.forward_factored(part["x"], part["router"], du, dv, L.device(), part["a"], part["b"], c.top_k)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y_full)[7:15], bits(y_part))


# edge shapes: 13 experts (row groups of four with a ragged last one), the
# smallest and largest factor ranks, the 256 / 257 token boundary between the
# K-sliced and the tiled x-projection
ODD = LayerConfig("odd13", 21, 256, 13, 128, 3, 1, 16, "mixed")


@pytest.mark.parametrize("cfg,rank,T", [(ODD, 8, 5), (ODD, 1024, 16), (ODD, 1024, 300), (ODD, 24, 256),
                                        (ODD, 24, 257)])
def test_factored_delta_edge_shapes(cfg, rank, T):
    L = Layer(cfg)
    say(f"factored delta {cfg.name} E={cfg.n_experts} T={T} rank={rank}")
    y, ref = run_factored(L, L.gen.tokens(T, 11), rank)
    m = row_metric(y, ref)
    say(f"  max row metric {m.max():.3e}")
    assert m.max() <= TOL
