"""The forward pass without allocation (moe_ternary_forward_noalloc) against
moe_ternary_forward, through the C ABI.

The no-allocation entry point runs the same kernels with its workspace in the
library's own device array, so its output must equal moe_ternary_forward's bit
for bit.  Each case makes two calls in a row, the second with a smaller batch,
so the second reads an array the first has filled.  A batch whose workspace
exceeds the array is refused before any launch, leaving y as it was.
"""
import sys

import numpy as np
import pytest

from layer_fixtures import Layer

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MOE_E_SPACE = -6


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_quantized_moe_amd as tq
    tq.lib()
    return tq


def forward_both(L, T, set_index):
    import ternary_quantized_moe_amd as tq
    c = L.cfg
    d = L.tensors(L.gen.tokens(T, set_index))
    banks = L.device()
    y_ref = tq.forward(d["x"], d["router"], d["delta"], banks, d["a"], d["b"], c.top_k)
    y_na = torch.full_like(d["x"], 0x7FC0)           # bf16 NaN bits: every element must be written
    tq.forward_noalloc(d["x"], d["router"], d["delta"], banks, d["a"], d["b"], c.top_k, y=y_na)
    torch.cuda.synchronize()
    return y_ref.cpu().numpy(), y_na.cpu().numpy()


# (layer, first batch, second batch): decode kernels (16-token items), the
# large-batch kernels (300 tokens), and the Flash-Next shape with its shared
# expert from 256 tokens down to one
@pytest.mark.parametrize("name,T1,T2", [("olmoe", 64, 8), ("a3b35", 300, 16), ("flashnext", 256, 1)])
def test_noalloc_equals_forward_on_two_calls(name, T1, T2):
    L = Layer(name)
    for T, s in ((T1, 1), (T2, 2)):
        say(f"no-allocation forward {name} T={T}")
        y_ref, y_na = forward_both(L, T, s)
        assert np.array_equal(y_na.view(np.uint16), y_ref.view(np.uint16)), (name, T)


def test_noalloc_refuses_a_batch_beyond_its_scratch():
    import ternary_quantized_moe_amd as tq
    L = Layer("a3b35")
    c = L.cfg
    T = 4096
    need = tq.workspace_bytes(L.device(), T, c.top_k, c.rank)
    assert need > tq.binding.NOALLOC_SCRATCH_BYTES
    d = L.tensors(L.gen.tokens(T, 1))
    y = torch.full_like(d["x"], 0x1234)
    with pytest.raises(tq.MoeError) as ei:
        tq.forward_noalloc(d["x"], d["router"], d["delta"], L.device(), d["a"], d["b"], c.top_k, y=y)
    assert ei.value.code == MOE_E_SPACE and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((y == 0x1234).all())
