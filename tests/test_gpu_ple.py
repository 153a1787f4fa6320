"""GPU parity of the Q4_0 row gather (moe_ple_gather_q4_0) against the oracle
decode, through the C ABI.  The bar is exact: every decoded value d (q - 8) is
an fp32 value, so the device's fp32 rows must equal the oracle's float64 rows
(NaN rows where the index is out of range)."""
import sys

import numpy as np
import pytest

from oracle import ple
from synthetic.ple import q4_table, q4_table_device, row_list, row_list_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_quantized_moe_amd as tq
    tq.lib()
    return tq


def gpu_gather(table, n_rows, row_len, idx):
    import ternary_quantized_moe_amd as tq
    d_t = torch.from_numpy(np.ascontiguousarray(table)).cuda()
    d_i = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int64)).cuda()
    out = tq.ple_gather(d_t, n_rows, row_len, d_i)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def assert_rows_equal(got, want):
    assert got.shape == want.shape
    same = (got.astype(np.float64) == want) | (np.isnan(got) & np.isnan(want))
    bad = np.argwhere(~same)
    assert bad.size == 0, f"{len(bad)} values differ, first at {tuple(bad[0])}: {got[tuple(bad[0])]} vs {want[tuple(bad[0])]}"


@pytest.mark.parametrize("row_len", [32, 64, 160, 4096])
@pytest.mark.parametrize("n_idx", [1, 7, 1000])
def test_gather_exact(row_len, n_idx):
    n_rows = 997
    table = q4_table(n_rows, row_len, seed=row_len)
    idx = row_list(n_idx, n_rows, seed=n_idx)
    say(f"ple gather row_len={row_len} n_idx={n_idx}")
    assert_rows_equal(gpu_gather(table, n_rows, row_len, idx), ple.gather(table, n_rows, row_len, idx))


def test_gather_special_scales_and_indices():
    n_rows, row_len = 8, 160
    table = q4_table(n_rows, row_len, seed=5)
    t = table.reshape(n_rows, 5, 18)
    specials = np.array([0.0, -0.0, 6e-8, -65504.0, np.inf], dtype=np.float16).view(np.uint8).reshape(5, 2)
    t[0, :, 0:2] = specials                   # zero, negative zero, subnormal, largest, infinite scale
    t[1, :, 2:] = 0x88                        # code 8 everywhere: zeros
    t[2, :, 2:] = 0x0F                        # codes 15 and 0: +7 d and -8 d
    idx = np.array([0, 1, 2, 7, 2, -1, n_rows, 1 << 40, -(1 << 40), 3], dtype=np.int64)
    say("ple gather special scales and indices")
    got = gpu_gather(table, n_rows, row_len, idx)
    with np.errstate(invalid="ignore"):                      # inf * 0 in the infinite-scale block
        want = ple.gather(table, n_rows, row_len, idx)
    assert np.all(np.isnan(got[5:9]))
    assert_rows_equal(got, want)


def test_gather_empty_and_into_offset_output():
    import ternary_quantized_moe_amd as tq
    table = q4_table(16, 64, seed=9)
    d_t = torch.from_numpy(table).cuda()
    out = torch.full((10, 64), 7.0, device="cuda")
    tq.ple_gather(d_t, 16, 64, torch.zeros(0, dtype=torch.int64, device="cuda"), out=out)
    idx = row_list(3, 16, seed=3)
    tq.ple_gather(d_t, 16, 64, torch.from_numpy(idx).cuda(), out=out[4:])
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[:4] == 7.0) and np.all(o[7:] == 7.0)
    assert_rows_equal(o[4:7], ple.gather(table, 16, 64, idx))


def test_gather_full_table_sampled():
    """The card's table size (320,001,536 rows of 160 values, 28.8 GB) and the
    prefill row list the gather is timed on (4096 tokens x 48 rows): 2048 rows of
    the output checked against the oracle."""
    import ternary_quantized_moe_amd as tq
    n_rows, row_len, n_idx = 320_001_536, 160, 4096 * 48
    say(f"ple gather full table {n_rows} rows, {n_idx} indices")
    d_t = q4_table_device(n_rows, row_len, seed=0)
    d_i = row_list_device(n_idx, n_rows, seed=0)
    out = tq.ple_gather(d_t, n_rows, row_len, d_i)
    torch.cuda.synchronize()
    pick = np.sort(np.random.default_rng(1).choice(n_idx, 2048, replace=False))
    rows = d_i.cpu().numpy()[pick]
    sub = d_t[torch.from_numpy(rows).cuda()].cpu().numpy()      # the sampled rows' bytes
    want = ple.gather(sub, len(rows), row_len, np.arange(len(rows)))
    assert_rows_equal(out.cpu().numpy()[pick], want)
    del d_t
    torch.cuda.empty_cache()
