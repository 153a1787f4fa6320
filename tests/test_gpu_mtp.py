"""GPU parity of the k=1 draft head (moe_draft_head) against the float64 oracle,
through the C ABI.  Bar: max_j |dy_j| / ||y||_2 <= 2e-3 per token row (the
block's tolerance; gelu(W1 x + b1) and y are rounded to bf16 on the GPU)."""
import sys

import numpy as np
import pytest

from oracle import moe as omoe, mtp
from synthetic.mtp import head_inputs, head_weights

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
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def run(h, m, T, bias=True, seed=0):
    import ternary_quantized_moe_amd as tq
    w1, b1, w2, b2 = head_weights(h, m, seed)
    if not bias:
        b1 = b2 = None
    hid, emb = head_inputs(T, h, seed)
    y = tq.draft_head(dev16(hid), dev16(emb), dev16(w1), dev16(b1), dev16(w2), dev16(b2))
    torch.cuda.synchronize()
    ref = mtp.head(hid, emb, w1, b1, w2, b2)
    got = omoe.bf16_to_f64(y.cpu().numpy().view(np.uint16))
    err = (np.abs(got - ref).max(axis=1) / np.linalg.norm(ref, axis=1)).max()
    say(f"  draft head h={h} m={m} T={T} bias={bias}: max row metric {err:.3e}")
    return err


@pytest.mark.parametrize("T", [1, 7, 64, 256, 257, 300])
def test_draft_head_small(T):
    # 256 is the last batch of the split-K path, 257 the first of the tiled one
    assert run(256, 512, T) <= TOL


@pytest.mark.parametrize("T", [1, 33, 64, 200, 300])
def test_draft_head_card_size(T):
    # from 33 tokens on, the 2048- and 4096-row products take the LDS-staged
    # kernel: eight waves per block while the grid has fewer than 1024 blocks,
    # four waves beyond (fc1 at 200 tokens: 64 x 8 x 4 blocks)
    # h = 2048, m = 4096: 25.2 M fp16 weights, the card's 50 MB
    assert run(2048, 4096, T) <= TOL


def test_draft_head_wide_inner_three_token_tiles():
    # m = 8192 rows at 40 tokens: three token tiles and 128 x 8 blocks, the
    # four-wave LDS-staged kernel with three token tiles
    assert run(2048, 8192, 40) <= TOL


def test_draft_head_without_biases():
    assert run(256, 384, 5, bias=False) <= TOL


def test_draft_head_deterministic():
    import ternary_quantized_moe_amd as tq
    w1, b1, w2, b2 = head_weights(256, 512, 1)
    hid, emb = head_inputs(40, 256, 1)
    outs = [tq.draft_head(dev16(hid), dev16(emb), dev16(w1), dev16(b1), dev16(w2), dev16(b2)).cpu().numpy()
            for _ in range(2)]
    # a token's output does not depend on the other tokens of the batch
    one = tq.draft_head(dev16(hid[7:8]), dev16(emb[7:8]), dev16(w1), dev16(b1), dev16(w2), dev16(b2)).cpu().numpy()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0][7:8], one)
