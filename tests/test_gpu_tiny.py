"""GPU parity of the three-launch path of batches of at most four tokens.

Up to four tokens (E <= 512, T (k + S) <= 256) the block runs as the
x-projection, a gate/up kernel whose blocks each route the batch themselves,
and one kernel for the down projection and the combine.  The routing this path
makes is the one moe_route exports (the same top-k code on the same logit
partials), so the tests compare every token's output with the oracle forced
to moe_route's choice, after checking that choice (R1-R3).  Layers cover both
containers and their mix, a shared expert, d = 1152 (a group count with no
compiled-in shape), k = 1 and k = E, no correction, a ternary-coded correction,
and 4 against 5 tokens (the last batch of this path and the first of the next).
"""
import sys

import numpy as np
import pytest

from layer_fixtures import Layer, row_metric
from oracle_threads import forward_y
from synthetic import LayerConfig
from test_gpu_parity import RAGGED, SMALL_MIXED, check_routing

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


def run_and_check(L, T, set_index, k=None, use_corr=True):
    import ternary_quantized_moe_amd as tq
    c = L.cfg
    k = k or c.top_k
    x_bits = L.gen.tokens(T, set_index)
    d = L.tensors(x_bits, use_corr=use_corr)
    r = tq.route(d["x"], d["router"], d["delta"], c.n_experts, k)
    y = tq.forward(d["x"], d["router"], d["delta"], L.device(), d["a"], d["b"], k)
    torch.cuda.synchronize()
    if k == c.top_k:
        idx, _ = check_routing(L, x_bits, r, np.arange(T))
    else:
        idx = r["idx"].cpu().numpy().astype(np.int64)
        lg = r["logits"].cpu().numpy().astype(np.float64)
        assert np.array_equal(idx, np.argsort(-lg, axis=1, kind="stable")[:, :k])
    ref = forward_y(L, x_bits, L.router, L.delta, L.corr_a if use_corr else None,
                    L.corr_b if use_corr else None, k, idx)
    m = row_metric(y.cpu().numpy().view(np.uint16), ref)
    say(f"  {c.name} T={T} k={k} corr={use_corr}: max row metric {m.max():.3e}")
    assert m.max() <= TOL
    return y


@pytest.mark.parametrize("name,T", [("olmoe", 2), ("olmoe", 3), ("olmoe", 4), ("a3b35", 2), ("a3b35", 4),
                                    ("flashnext", 2), ("flashnext", 3), ("flashnext", 4), ("skewed", 1),
                                    ("skewed", 4), ("tiny", 1), ("tiny", 4)])
def test_tiny_batches(name, T):
    run_and_check(Layer(name), T, 11)


@pytest.mark.parametrize("T", [1, 2, 4, 5])
def test_tiny_ragged_and_mixed(T):
    run_and_check(Layer(RAGGED), T, 12)
    run_and_check(Layer(SMALL_MIXED), T, 12)


@pytest.mark.parametrize("k", [1, 8])
def test_tiny_top1_and_all_experts(k):
    run_and_check(Layer("tiny"), 3, 13, k=k)


def test_tiny_without_correction():
    run_and_check(Layer("flashnext"), 2, 14, use_corr=False)
    run_and_check(Layer("olmoe"), 1, 14, use_corr=False)


MANY = LayerConfig("many", 22, 256, 1000, 128, 9, 0, 16, "pq2_0")


def test_tiny_falls_back_beyond_512_experts():
    run_and_check(Layer(MANY), 3, 15)


def test_tiny_deterministic():
    import ternary_quantized_moe_amd as tq
    L = Layer("flashnext")
    c = L.cfg
    d = L.tensors(L.gen.tokens(3, 16))
    ys = [tq.forward(d["x"], d["router"], d["delta"], L.device(), d["a"], d["b"], c.top_k).cpu().numpy()
          for _ in range(3)]
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])
