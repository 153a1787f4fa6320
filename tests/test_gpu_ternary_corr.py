"""GPU tests of the forward pass with a ternary-coded router delta and
correction (moe_ternary_forward_q), through the C ABI.

A code t times its fp16 group scale s is an fp16 value, so a ternary-coded
matrix has an exact fp16 expansion s * t.  The bar: the block output with the
containers equals bit for bit the output of moe_ternary_forward given those fp16
expansions (decode and large-batch paths), and the oracle, fed the expansions it
decodes itself from the same container bytes, agrees within the block tolerance.
"""
import sys

import numpy as np
import pytest

from layer_fixtures import Layer, row_metric
from oracle_threads import forward_y
from oracle import codec, moe as omoe
from synthetic import CONFIGS, LayerGen

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


def f16_expansion(trits, scale_bits):
    """fp16 bits of s * t: s with the sign flipped for t = -1, +0 for t = 0."""
    rows, cols = trits.shape
    s = np.repeat(scale_bits.astype(np.uint32), 128, axis=1).reshape(rows, cols)
    bits = np.where(trits < 0, s ^ 0x8000, s)
    return np.where(trits == 0, 0, bits).astype(np.uint16)


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def ternary_parts(L, use_corr):
    g = L.gen
    parts = {"delta": g.delta_q_parts()}
    if use_corr:
        parts["a"], parts["b"] = g.corr_a_q_parts(), g.corr_b_q_parts()
    return parts


def run_both(L, T, use_corr=True):
    import ternary_quantized_moe_amd as tq
    c = L.cfg
    x_bits = L.gen.tokens(T, 3)
    banks = L.device()
    parts = ternary_parts(L, use_corr)
    q = {k: torch.from_numpy(tq.pack(142, t.reshape(-1), s.reshape(-1))).cuda() for k, (t, s) in parts.items()}
    dense = {k: f16_expansion(t, s) for k, (t, s) in parts.items()}
    x, router = dev16(x_bits), dev16(L.router)
    y_q = tq.forward_q(x, router, q["delta"], banks, q.get("a"), q.get("b"), c.rank if use_corr else 0, c.top_k)
    y_d = tq.forward(x, router, dev16(dense["delta"]), banks, dev16(dense["a"]) if use_corr else None,
                     dev16(dense["b"]) if use_corr else None, c.top_k)
    torch.cuda.synchronize()
    return x_bits, q, dense, y_q.cpu().numpy().view(np.uint16), y_d.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name,T", [("olmoe", 1), ("olmoe", 8), ("olmoe", 64), ("flashnext", 37),
                                    ("a3b35", 300)])
def test_ternary_corrections_equal_their_fp16_expansion(name, T):
    L = Layer(name)
    say(f"ternary corrections {name} T={T}")
    _, _, _, y_q, y_d = run_both(L, T)
    assert np.array_equal(y_q, y_d)


def test_ternary_delta_without_correction():
    L = Layer("tiny")
    say("ternary delta, tiny, no correction")
    _, _, _, y_q, y_d = run_both(L, 16, use_corr=False)
    assert np.array_equal(y_q, y_d)


@pytest.mark.parametrize("name,T", [("olmoe", 16), ("olmoe", 64), ("a3b35", 300)])
def test_ternary_corrections_against_the_oracle(name, T):
    """Every token of the batch (300 tokens take the large-batch kernels)."""
    import ternary_quantized_moe_amd as tq
    L = Layer(name)
    c = L.cfg
    say(f"ternary corrections against the oracle {name} T={T}")
    x_bits, q, dense, y_q, _ = run_both(L, T)
    # the oracle decodes the containers the library packed with its own codec
    dec = {}
    for k, data in q.items():
        rows, cols = {"delta": (c.n_experts, c.d_model), "a": (c.rank, c.d_model), "b": (c.d_model, c.rank)}[k]
        t, s = codec.unpack(142, data.cpu().numpy(), rows * cols)
        dec[k] = f16_expansion(t.reshape(rows, cols), s.reshape(rows, cols // 128))
        assert np.array_equal(dec[k], dense[k])
    r = tq.route(dev16(x_bits), dev16(L.router), dev16(dec["delta"]), c.n_experts, c.top_k)
    idx = r["idx"].cpu().numpy()
    ref = forward_y(L, x_bits, L.router, dec["delta"], dec["a"], dec["b"], c.top_k, idx)
    m = row_metric(y_q, ref)
    say(f"  max row metric {m.max():.3e}")
    assert m.max() <= TOL


def test_ternary_forward_errors():
    import ternary_quantized_moe_amd as tq
    L = Layer("tiny")          # rank 16: a ternary B needs a rank that is a multiple of 128
    c = L.cfg
    banks = L.device()
    x = dev16(L.gen.tokens(4, 0))
    y = torch.empty_like(x)
    ws = tq.alloc_workspace(tq.workspace_bytes(banks, 4, c.top_k, c.rank), x.device)
    dummy = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    lib = tq.lib()
    rc = lib.moe_ternary_forward_q(x.data_ptr(), 4, dev16(L.router).data_ptr(), None, banks.c, dummy.data_ptr(),
                                   dummy.data_ptr(), c.rank, c.top_k, y.data_ptr(), ws.data_ptr(), ws.numel(), None)
    assert rc == -3 and "multiple of 128" in lib.moe_last_error().decode()
    rc = lib.moe_ternary_forward_q(x.data_ptr(), 4, dev16(L.router).data_ptr(), None, banks.c, dummy.data_ptr(),
                                   None, 128, c.top_k, y.data_ptr(), ws.data_ptr(), ws.numel(), None)
    assert rc == -1
