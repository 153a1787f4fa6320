"""GPU tests of the stand-alone rank-r branch (moe_lowrank_apply), y = y_in +
B (A x), through the C ABI: the correction the releases also place on the
attention output (Scion-35B-A3B card, "Weight Representation").

The bar: within the block tolerance of the oracle's fp64 y + B (A x), on the
decode path (up to 256 tokens, K-split products) and the tiled path beyond;
with ternary A, B bit for bit equal to the same call on their fp16 expansions;
the in-place form (y is y_in) equal bit for bit to the out-of-place one.
"""
import sys

import numpy as np
import pytest

from layer_fixtures import row_metric
from oracle import codec, moe as omoe
from synthetic import CONFIGS, LayerGen, bf16_bits, f16_bits

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


def f16_expansion(trits, scale_bits):
    rows, cols = trits.shape
    s = np.repeat(scale_bits.astype(np.uint32), 128, axis=1).reshape(rows, cols)
    b = np.where(trits < 0, s ^ 0x8000, s)
    return np.where(trits == 0, 0, b).astype(np.uint16)


def inputs(name, T):
    g = LayerGen(CONFIGS[name])
    return g, g.tokens(T, 5), g.tokens(T, 6), g.corr_a_bits(), g.corr_b_bits()


@pytest.mark.parametrize("name,T,with_y", [("tiny", 1, True), ("olmoe", 1, True), ("olmoe", 16, False),
                                           ("a3b35", 64, True), ("flashnext", 37, True), ("olmoe", 256, True),
                                           ("olmoe", 257, True), ("flashnext", 300, False)])
def test_lowrank_against_the_oracle(name, T, with_y):
    import ternary_quantized_moe_amd as tq
    c = CONFIGS[name]
    say(f"lowrank {name} T={T} y_in={with_y}")
    _, x, yin, a, b = inputs(name, T)
    y = tq.lowrank_apply(dev16(x), dev16(yin) if with_y else None, dev16(a), dev16(b), c.rank)
    torch.cuda.synchronize()
    ref = omoe.lowrank_apply(x, yin if with_y else None, a, b)
    m = row_metric(bits(y), ref)
    say(f"  max row metric {m.max():.3e}")
    assert m.max() <= TOL


@pytest.mark.parametrize("name,T", [("olmoe", 1), ("a3b35", 33), ("flashnext", 300)])
def test_lowrank_ternary_equals_its_fp16_expansion(name, T):
    import ternary_quantized_moe_amd as tq
    c = CONFIGS[name]
    say(f"lowrank ternary {name} T={T}")
    g, x, yin, _, _ = inputs(name, T)
    (ta, sa), (tb, sb) = g.corr_a_q_parts(), g.corr_b_q_parts()
    qa = torch.from_numpy(tq.pack(142, ta.reshape(-1), sa.reshape(-1))).cuda()
    qb = torch.from_numpy(tq.pack(142, tb.reshape(-1), sb.reshape(-1))).cuda()
    ea, eb = f16_expansion(ta, sa), f16_expansion(tb, sb)
    xd, yd = dev16(x), dev16(yin)
    y_q = tq.lowrank_apply(xd, yd, None, None, c.rank, a_q=qa, b_q=qb)
    y_d = tq.lowrank_apply(xd, yd, dev16(ea), dev16(eb), c.rank)
    y_m = tq.lowrank_apply(xd, yd, dev16(ea), None, c.rank, b_q=qb)     # one of each form
    torch.cuda.synchronize()
    assert np.array_equal(bits(y_q), bits(y_d))
    assert np.array_equal(bits(y_m), bits(y_d))
    # the oracle decodes the containers with its own codec
    ta2, sa2 = codec.unpack(142, qa.cpu().numpy(), ta.size)
    tb2, sb2 = codec.unpack(142, qb.cpu().numpy(), tb.size)
    da = f16_expansion(ta2.reshape(ta.shape), sa2.reshape(sa.shape))
    db = f16_expansion(tb2.reshape(tb.shape), sb2.reshape(sb.shape))
    m = row_metric(bits(y_q), omoe.lowrank_apply(x, yin, da, db))
    say(f"  max row metric {m.max():.3e}")
    assert m.max() <= TOL


@pytest.mark.parametrize("T", [5, 64, 300])
def test_lowrank_in_place(T):
    import ternary_quantized_moe_amd as tq
    c = CONFIGS["olmoe"]
    say(f"lowrank in place T={T}")
    _, x, yin, a, b = inputs("olmoe", T)
    xd, ad, bd = dev16(x), dev16(a), dev16(b)
    y_out = tq.lowrank_apply(xd, dev16(yin), ad, bd, c.rank)
    y_io = dev16(yin)
    r = tq.lowrank_apply(xd, y_io, ad, bd, c.rank, y=y_io)
    torch.cuda.synchronize()
    assert r.data_ptr() == y_io.data_ptr()
    assert np.array_equal(bits(y_io), bits(y_out))


def test_lowrank_batch_independence():
    """A token's output does not depend on the other tokens of its batch (up to
    256 tokens the K slicing depends on d alone)."""
    import ternary_quantized_moe_amd as tq
    c = CONFIGS["a3b35"]
    _, x, yin, a, b = inputs("a3b35", 40)
    ad, bd = dev16(a), dev16(b)
    full = bits(tq.lowrank_apply(dev16(x), dev16(yin), ad, bd, c.rank))
    part = bits(tq.lowrank_apply(dev16(x[7:9]), dev16(yin[7:9]), ad, bd, c.rank))
    torch.cuda.synchronize()
    assert np.array_equal(full[7:9], part)


def test_lowrank_errors_on_device():
    import ternary_quantized_moe_amd as tq
    c = CONFIGS["olmoe"]
    _, x, yin, a, b = inputs("olmoe", 4)
    xd = dev16(x)
    with pytest.raises(tq.MoeError):
        tq.lowrank_apply(xd, None, dev16(a), dev16(b), c.rank, y=xd)        # y aliases x
    with pytest.raises(tq.MoeError):
        tq.lowrank_apply(xd, None, dev16(a), dev16(b), c.rank, workspace=torch.empty(64, dtype=torch.uint8,
                                                                                      device="cuda"))


@pytest.mark.parametrize("d,r,T", [(128, 8, 3), (128, 8, 300), (256, 4096, 2), (256, 4096, 260), (384, 136, 64)])
def test_lowrank_edge_shapes(d, r, T):
    """The smallest width and rank, the largest rank, a rank that is not a
    multiple of 16, on both sides of the 256-token boundary."""
    import ternary_quantized_moe_amd as tq
    rng = np.random.default_rng(d * 7 + r + T)
    x = bf16_bits(rng.normal(size=(T, d)))
    yin = bf16_bits(rng.normal(size=(T, d)))
    a = f16_bits(rng.normal(scale=1 / np.sqrt(d), size=(r, d)))
    b = f16_bits(rng.normal(scale=1 / np.sqrt(r), size=(d, r)))
    say(f"lowrank edge d={d} r={r} T={T}")
    y = tq.lowrank_apply(dev16(x), dev16(yin), dev16(a), dev16(b), r)
    torch.cuda.synchronize()
    m = row_metric(bits(y), omoe.lowrank_apply(x, yin, a, b))
    say(f"  max row metric {m.max():.3e}")
    assert m.max() <= TOL
