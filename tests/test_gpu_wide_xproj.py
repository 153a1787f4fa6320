"""GPU tests of wide x-projections (33-256 tokens, 2048 or more rows), through
the C ABI.  The stand-alone branch with a wide A takes the LDS-staged kernel;
a block whose rank-2048 correction makes its projection wide (router rows with
the summed delta, then A's rows, a row tile straddling the two) keeps the
K-split kernel, so its logits stay the same with and without the correction
rows (checked bit for bit).  The bar otherwise is the oracle within the block
tolerance; block outputs are compared on tokens whose expert choice is decided
(fp64 top-k margin above four times the fp32 logit bound)."""
import sys

import numpy as np
import pytest

from layer_fixtures import Layer, row_metric
from oracle import moe as omoe
from synthetic import LayerConfig, bf16_bits, f16_bits

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3
# 20 experts (rows 16-31 hold four router rows and twelve of A's), rank 2048
WIDE = LayerConfig("widecorr", 41, 256, 20, 128, 2, 0, 2048, "pq2_0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_quantized_moe_amd as tq
    tq.lib()
    return tq


def decided(L, n, set_index, pool=8):
    c = L.cfg
    xs = L.gen.tokens(pool * n, set_index)
    x = omoe.bf16_to_f64(xs)
    w = omoe.f16_to_f64(L.router) + omoe.f16_to_f64(L.delta)
    l64 = x @ w.T
    gam = 8 * np.sqrt(c.d_model) * 2.0 ** -24 * (np.abs(x) @ np.abs(w).T)
    srt = -np.sort(-l64, axis=1)
    gap = srt[:, c.top_k - 1] - srt[:, c.top_k]
    keep = np.nonzero(gap > 4 * gam.max(axis=1))[0][:n]
    assert len(keep) == n
    return xs[keep]


@pytest.mark.parametrize("T", [40, 64, 200])
def test_wide_projection_block(T):
    import ternary_quantized_moe_amd as tq
    L = Layer(WIDE)
    c = L.cfg
    x_bits = decided(L, T, 3)
    say(f"wide x-projection block T={T} rows={c.n_experts + c.rank}")
    d = L.tensors(x_bits)
    y = tq.forward(d["x"], d["router"], d["delta"], L.device(), d["a"], d["b"], c.top_k)
    torch.cuda.synchronize()
    ref = omoe.forward(x_bits, L.router, L.delta, L.oracle_banks, L.corr_a, L.corr_b, c.top_k)
    m = row_metric(y.cpu().numpy().view(np.uint16), ref.y)
    say(f"  max row metric {m.max():.3e}")
    assert m.max() <= TOL


def test_wide_block_zero_correction_is_bit_exact():
    """Zero A and B of rank 2048 leave the block bit for bit as without them:
    the 2068-row projection sums each logit as the 20-row one does."""
    import ternary_quantized_moe_amd as tq
    L = Layer(WIDE)
    c = L.cfg
    x_bits = L.gen.tokens(64, 4)
    d = L.tensors(x_bits)
    za, zb = torch.zeros_like(d["a"]), torch.zeros_like(d["b"])
    y_z = tq.forward(d["x"], d["router"], d["delta"], L.device(), za, zb, c.top_k)
    y_n = tq.forward(d["x"], d["router"], d["delta"], L.device(), None, None, c.top_k)
    torch.cuda.synchronize()
    assert torch.equal(y_z, y_n)


# (4096, 4096, 160): 64 x 8 x 3 blocks, the four-wave form of the LDS-staged kernel
@pytest.mark.parametrize("d,r,T", [(256, 2048, 64), (512, 4096, 33), (384, 2056, 100), (4096, 4096, 160)])
def test_wide_projection_branch(d, r, T):
    import ternary_quantized_moe_amd as tq
    rng = np.random.default_rng(d + r + T)
    x = bf16_bits(rng.normal(size=(T, d)))
    yin = bf16_bits(rng.normal(size=(T, d)))
    a = f16_bits(rng.normal(scale=1 / np.sqrt(d), size=(r, d)))
    b = f16_bits(rng.normal(scale=1 / np.sqrt(r), size=(d, r)))
    say(f"wide branch d={d} r={r} T={T}")
    dev = lambda v: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).cuda()
    y = tq.lowrank_apply(dev(x), dev(yin), dev(a), dev(b), r)
    torch.cuda.synchronize()
    m = row_metric(y.cpu().numpy().view(np.uint16), omoe.lowrank_apply(x, yin, a, b))
    say(f"  max row metric {m.max():.3e}")
    assert m.max() <= TOL
