"""The forward pass writes only inside the buffers the C ABI gives it.

The workspace is exactly moe_workspace_bytes long, with 4 KB of a known
pattern on either side; y has guard rows of the same pattern before and after
it.  After the call (and a synchronisation) every guard byte still holds the
pattern, every row of y was written, and x and the expert banks are unchanged.
Batches cover the decode kernels (1 and 64 tokens), the large-batch kernels at
300 and 4096 tokens, and the Flash-Next shape with its shared expert.
"""
import sys

import numpy as np
import pytest

from layer_fixtures import Layer

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes of pattern on each side
PATTERN = 0xA5


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_quantized_moe_amd as tq
    tq.lib()
    return tq


def guarded(nbytes, align=256):
    """(whole buffer, view of nbytes starting align-aligned, GUARD or more bytes in)."""
    buf = torch.full((nbytes + 2 * GUARD + align,), PATTERN, dtype=torch.uint8, device="cuda")
    off = GUARD + (-(buf.data_ptr() + GUARD)) % align
    return buf, off, buf[off:off + nbytes]


@pytest.mark.parametrize("name,T", [("olmoe", 1), ("olmoe", 64), ("a3b35", 300), ("a3b35", 4096),
                                    ("flashnext", 64)])
def test_forward_writes_nothing_outside_its_buffers(name, T):
    import ternary_quantized_moe_amd as tq
    L = Layer(name)
    c = L.cfg
    banks = L.device()
    d = L.tensors(L.gen.tokens(T, 2))
    need = tq.workspace_bytes(banks, T, c.top_k, c.rank)
    ws_buf, ws_off, ws = guarded(need)
    y_buf, y_off, y_bytes = guarded(T * c.d_model * 2, align=16)
    y = y_bytes.view(torch.int16).view(T, c.d_model)
    x_before = d["x"].clone()
    banks_before = banks.data.clone()
    say(f"guards {name} T={T}: workspace {need} bytes")
    tq.forward(d["x"], d["router"], d["delta"], banks, d["a"], d["b"], c.top_k, y=y, workspace=ws)
    torch.cuda.synchronize()
    for buf, off, n in ((ws_buf, ws_off, need), (y_buf, y_off, T * c.d_model * 2)):
        head, tail = buf[:off].cpu().numpy(), buf[off + n:].cpu().numpy()
        assert len(head) >= GUARD and len(tail) >= GUARD
        assert np.all(head == PATTERN), "write before the buffer"
        assert np.all(tail == PATTERN), "write past the buffer"
    # every y row was written: a row of the fill pattern would be 0xA5A5 bits throughout
    rows = y.cpu().numpy().view(np.uint16)
    assert not np.any(np.all(rows == 0xA5A5, axis=1))
    assert torch.equal(d["x"], x_before)
    assert torch.equal(banks.data, banks_before)
