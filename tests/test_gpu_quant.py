"""GPU parity of the ternary quantizer (moe_quantize_device) against the oracle
quantizer, through the C ABI.  The bar is bit-exact containers: the codes are
integers and the scale a binary16 pattern, decided on both sides in fp32 with
the same summation tree.
"""
import sys

import numpy as np
import pytest

from oracle import codec, quant
from synthetic import PQ2_0, PTQ1_0, bf16_bits
from synthetic.weights import weights_bf16, weights_bf16_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FMTS = [PQ2_0, PTQ1_0]
METHODS = [quant.ABSMEAN, quant.LLOYD]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_quantized_moe_amd as tq
    tq.lib()
    return tq


def gpu_quantize(fmt, method, w_bits):
    """(container bytes, Lloyd rounds per group) from the device quantizer."""
    import ternary_quantized_moe_amd as tq
    d_w = torch.from_numpy(np.ascontiguousarray(w_bits).view(np.int16)).cuda()
    rounds = torch.full((w_bits.size // 128,), 0xFF, dtype=torch.uint8, device="cuda")
    out = tq.quantize_device(fmt, method, d_w, rounds=rounds)
    torch.cuda.synchronize()
    return out.cpu().numpy(), rounds.cpu().numpy()


def assert_same_blocks(fmt, got, want):
    bb = codec.block_bytes(fmt)
    g, w = got.reshape(-1, bb), want.reshape(-1, bb)
    bad = np.nonzero(np.any(g != w, axis=1))[0]
    assert bad.size == 0, f"{bad.size} groups differ, first {bad[0]}: got {g[bad[0]]}, want {w[bad[0]]}"


def chain_group(n, seed):
    """A group on which Lloyd drops a few weights per round for a long time:
    magnitudes v_1 = 1, v_m = 0.97 (v_1 + ... + v_{m-1}) / (2m - 1), random
    signs and places, zeros elsewhere."""
    v, total = [1.0], 1.0
    for m in range(2, n + 1):
        x = 0.97 * total / (2 * m - 1)
        v.append(x)
        total += x
    g = np.zeros(128)
    g[:n] = v
    rng = np.random.default_rng(seed)
    rng.shuffle(g)
    return g * np.where(rng.random(128) < 0.5, -1.0, 1.0)


def special_groups():
    rng = np.random.default_rng(11)
    groups = [
        np.zeros(128),                                            # all zero
        np.concatenate([np.full(64, 1.0), np.full(64, -3.0)]),    # exact ties 2|w| = s
        np.eye(1, 128, 5)[0] * -0.75,                             # one nonzero
        np.full(128, 3.0e5),                                      # scale beyond binary16
        rng.standard_normal(128) * 1e-6,                          # binary16-subnormal scale
        rng.standard_normal(128) * 1e-39,                         # bfloat16-subnormal weights
        np.full(128, -0.0),                                       # negative zeros
        np.full(128, 3.0e38) * np.where(np.arange(128) % 2, 1, -1),  # the group sum overflows
        np.full(128, 0.5),                                        # one value, both signs below
        -np.full(128, 0.5),
        chain_group(40, 1), chain_group(100, 2), chain_group(128, 3),  # long Lloyd runs (32 rounds)
    ]
    return bf16_bits(np.concatenate(groups))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("groups", [1, 3, 4, 17, 1037])
def test_quantize_bit_exact(fmt, method, groups):
    w = weights_bf16(groups, 128, seed=groups).reshape(-1)
    say(f"quantize fmt={fmt} method={method} groups={groups}")
    got, rounds = gpu_quantize(fmt, method, w)
    assert_same_blocks(fmt, got, quant.quantize(fmt, w, method))
    assert np.array_equal(rounds, quant.quantize_groups(w, method)[3])


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("method", METHODS)
def test_quantize_special_groups(fmt, method):
    w = special_groups()
    say(f"quantize special groups fmt={fmt} method={method}")
    got, got_rounds = gpu_quantize(fmt, method, w)
    with np.errstate(over="ignore"):
        want = quant.quantize(fmt, w, method)
        _, _, _, rounds = quant.quantize_groups(w, method)
    if method == quant.LLOYD:
        assert rounds.max() == quant.MAX_ROUNDS  # the capped path is covered
    assert_same_blocks(fmt, got, want)
    assert np.array_equal(got_rounds, rounds)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("method", METHODS)
def test_quantize_full_matrix_sampled(fmt, method):
    """Every routed expert of the 35B-A3B-class layer (128 experts, gate, up
    and down of 768 x 2048 each) as one [128 * 3 * 768 x 2048] tensor, the size
    the quantizer is timed at: 9216 groups checked at random."""
    import ternary_quantized_moe_amd as tq
    rows, cols = 128 * 3 * 768, 2048
    d_w = weights_bf16_device(rows, cols, seed=fmt + 2 * method)
    say(f"quantize full matrix fmt={fmt} method={method} rows={rows} cols={cols}")
    n_groups = rows * cols // 128
    rounds = torch.empty(n_groups, dtype=torch.uint8, device="cuda")
    out = tq.quantize_device(fmt, method, d_w, rounds=rounds)
    torch.cuda.synchronize()
    bb = codec.block_bytes(fmt)
    pick = np.sort(np.random.default_rng(5).choice(n_groups, 9216, replace=False))
    w_groups = d_w.view(-1, 128).cpu().numpy().view(np.uint16)[pick]
    got = out.view(-1, bb).cpu().numpy()[pick]
    want = quant.quantize(fmt, w_groups.reshape(-1), method)
    assert_same_blocks(fmt, got.reshape(-1), want)
    assert np.array_equal(rounds.cpu().numpy()[pick], quant.quantize_groups(w_groups.reshape(-1), method)[3])


def test_quantize_two_calls_and_offsets():
    """A second call on a sub-range of the same tensor (23 groups from group 8
    on, written at block 8 of the first call's output) writes only its own
    blocks; the bytes past the container stay untouched."""
    import ternary_quantized_moe_amd as tq
    w = weights_bf16(64, 128, seed=99).reshape(-1)
    d_w = torch.from_numpy(w.view(np.int16)).cuda()
    for fmt in FMTS:
        bb = codec.block_bytes(fmt)
        out = torch.full((64 * bb + 8,), 0xA5, dtype=torch.uint8, device="cuda")
        tq.quantize_device(fmt, quant.LLOYD, d_w, out=out)
        sub = tq.quantize_device(fmt, quant.ABSMEAN, d_w[8 * 128:(8 + 23) * 128], out=out[8 * bb:])
        torch.cuda.synchronize()
        assert sub.numel() == 23 * bb
        o = out.cpu().numpy()
        want = quant.quantize(fmt, w, quant.LLOYD).copy()
        want[8 * bb:31 * bb] = quant.quantize(fmt, w[8 * 128:31 * 128], quant.ABSMEAN)
        assert_same_blocks(fmt, o[:64 * bb], want)
        assert np.all(o[64 * bb:] == 0xA5)

