"""GPU tests of the forward pass with the router delta given as two low-rank
fp16 factors U, V (moe_ternary_forward_factored), through the C ABI.

The bars: with U = 0 the block equals bit for bit the block without a delta
(decode and large-batch paths); against the oracle's logits W_r x + U V x, the
block output is within the block tolerance on tokens whose fp64 k-th / k+1-th
logit gap is far above the fp32 error of both products (so the choice of experts
is decided); a token's output does not depend on its batch.
"""
import sys

import numpy as np
import pytest

from layer_fixtures import Layer, row_metric
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


def decided_tokens(L, u, v, n, set_index, pool=16):
    """n tokens whose fp64 top-k is decided: every chosen logit minus twice its
    bound lies above every other logit plus twice its bound, with the bound of
    the fp32 products gamma = 8 sqrt(K) 2^-24 sum |w x| applied to W_r x (K = d)
    and to U (V x) (K = d and rank, through |U| |V| |x|)."""
    c = L.cfg
    xs = L.gen.tokens(pool * n, set_index)
    x = omoe.bf16_to_f64(xs)
    wr, uf, vf = omoe.f16_to_f64(L.router), omoe.f16_to_f64(u), omoe.f16_to_f64(v)
    logits = x @ (wr + uf @ vf).T
    d, rd = wr.shape[1], uf.shape[1]
    eps = 8 * 2.0 ** -24
    gamma = eps * np.sqrt(d) * (np.abs(x) @ np.abs(wr).T) + \
        eps * (np.sqrt(d) + np.sqrt(rd)) * ((np.abs(x) @ np.abs(vf).T) @ np.abs(uf).T)
    keep = []
    for t in range(len(x)):
        sel = np.zeros(c.n_experts, bool)
        sel[omoe.select_topk(logits[t:t + 1], c.top_k)[0]] = True
        if sel.all() or (logits[t, sel] - 2 * gamma[t, sel]).min() > (logits[t, ~sel] + 2 * gamma[t, ~sel]).max():
            keep.append(t)
        if len(keep) == n:
            break
    assert len(keep) == n, f"only {len(keep)} decided tokens of {pool * n}"
    return xs[keep]


RANK = {"tiny": 64, "olmoe": 512, "a3b35": 512, "flashnext": 512}


@pytest.mark.parametrize("name,T", [("tiny", 16), ("olmoe", 1), ("olmoe", 64), ("flashnext", 37),
                                    ("a3b35", 300)])
def test_factored_delta_against_the_oracle(name, T):
    import ternary_quantized_moe_amd as tq
    L = Layer(name)
    c = L.cfg
    u, v = L.gen.delta_factor_bits(RANK[name])
    x_bits = decided_tokens(L, u, v, T, 7)
    say(f"factored delta {name} T={T} rank={RANK[name]}")
    d = L.tensors(x_bits, use_delta=False)
    y = tq.forward_factored(d["x"], d["router"], dev16(u), dev16(v), L.device(), d["a"], d["b"], c.top_k)
    torch.cuda.synchronize()
    ref = omoe.forward(x_bits, L.router, None, L.oracle_banks, L.corr_a, L.corr_b, c.top_k,
                       delta_factors=(u, v))
    m = row_metric(bits(y), ref.y)
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
    part = L.tensors(x_bits[7:9], use_delta=False)
    y_full = tq.forward_factored(full["x"], full["router"], du, dv, L.device(), full["a"], full["b"], c.top_k)
    y_part = tq.forward_factored(part["x"], part["router"], du, dv, L.device(), part["a"], part["b"], c.top_k)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y_full)[7:9], bits(y_part))


# edge shapes: 13 experts (row groups of four with a ragged last one), the
# smallest and largest factor ranks, the 256 / 257 token boundary between the
# K-sliced and the tiled x-projection
ODD = LayerConfig("odd13", 21, 256, 13, 128, 3, 1, 16, "mixed")


@pytest.mark.parametrize("cfg,rank,T", [(ODD, 8, 5), (ODD, 1024, 16), (ODD, 1024, 300), (ODD, 24, 256),
                                        (ODD, 24, 257)])
def test_factored_delta_edge_shapes(cfg, rank, T):
    import ternary_quantized_moe_amd as tq
    L = Layer(cfg)
    c = L.cfg
    u, v = L.gen.delta_factor_bits(rank)
    x_bits = decided_tokens(L, u, v, T, 11)
    say(f"factored delta {c.name} E={c.n_experts} T={T} rank={rank}")
    d = L.tensors(x_bits, use_delta=False)
    y = tq.forward_factored(d["x"], d["router"], dev16(u), dev16(v), L.device(), d["a"], d["b"], c.top_k)
    torch.cuda.synchronize()
    ref = omoe.forward(x_bits, L.router, None, L.oracle_banks, L.corr_a, L.corr_b, c.top_k,
                       delta_factors=(u, v))
    m = row_metric(bits(y), ref.y)
    say(f"  max row metric {m.max():.3e}")
    assert m.max() <= TOL
