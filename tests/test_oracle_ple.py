"""Pins of the oracle Q4_0 row decode (oracle/ple.py) against what the pages and
the arithmetic fix."""
import os

import numpy as np

from golden_io import GOLDEN
from oracle import ple


def read_q4_fixture():
    vals = {}
    for line in open(os.path.join(GOLDEN, "q4_0_block.txt")):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.split()
    return (np.array([int(x, 16) for x in vals["bytes"]], dtype=np.uint8),
            np.array([float(x) for x in vals["values"]]))


def pack_rows(d_bits, nibbles):
    """Test-side packer: binary16 scales [rows, blocks], nibbles [rows, blocks, 32]."""
    rows, nb = d_bits.shape
    out = np.zeros((rows, nb, 18), dtype=np.uint8)
    out[:, :, 0] = d_bits & 0xFF
    out[:, :, 1] = d_bits >> 8
    out[:, :, 2:] = nibbles[:, :, :16] | (nibbles[:, :, 16:] << 4)
    return out.reshape(rows, -1)


def test_golden_block():
    data, want = read_q4_fixture()
    assert np.array_equal(ple.decode_block(data), want)


def test_table_size_matches_the_card():
    # 320,001,536 rows x 160 values in 18-byte blocks of 32: the card's 28.8 GB
    assert ple.row_bytes(160) == 90
    assert round(320_001_536 * ple.row_bytes(160) / 1e9, 1) == 28.8


def test_round_trip_of_chosen_codes():
    rng = np.random.default_rng(0)
    rows, nb = 7, 5
    d = rng.standard_normal((rows, nb)).astype(np.float16)
    d[0, 0], d[1, 1], d[2, 2] = 0.0, -0.0, np.float16(6e-8)      # zero, negative zero, subnormal
    nib = rng.integers(0, 16, size=(rows, nb, 32)).astype(np.uint8)
    table = pack_rows(d.view(np.uint16), nib)
    for r in range(rows):
        want = (d[r].astype(np.float64)[:, None] * (nib[r].astype(np.float64) - 8)).reshape(-1)
        assert np.array_equal(ple.decode_row(table, r, 32 * nb), want)


def test_invariants():
    rng = np.random.default_rng(1)
    d = rng.standard_normal((3, 5)).astype(np.float16)
    nib = rng.integers(0, 16, size=(3, 5, 32)).astype(np.uint8)
    base = ple.gather(pack_rows(d.view(np.uint16), nib), 3, 160, [0, 1, 2])
    # the code 8 is zero at any scale
    assert np.all(ple.gather(pack_rows(d.view(np.uint16), np.full_like(nib, 8)), 3, 160, [0, 1, 2]) == 0)
    # the value is linear in the scale: -d negates, 2d doubles
    assert np.array_equal(ple.gather(pack_rows((-d).view(np.uint16), nib), 3, 160, [0, 1, 2]), -base)
    d2 = (d.astype(np.float32) * 2).astype(np.float16)
    assert np.array_equal(ple.gather(pack_rows(d2.view(np.uint16), nib), 3, 160, [0, 1, 2]), 2 * base)
    # every value is d times an integer in [-8, 7]
    k = base.reshape(3, 5, 32) / d.astype(np.float64)[:, :, None]
    assert np.all(k == np.round(k)) and k.min() >= -8 and k.max() <= 7


def test_gather_order_duplicates_and_bad_indices():
    rng = np.random.default_rng(2)
    d = rng.standard_normal((4, 1)).astype(np.float16)
    nib = rng.integers(0, 16, size=(4, 1, 32)).astype(np.uint8)
    table = pack_rows(d.view(np.uint16), nib)
    out = ple.gather(table, 4, 32, [3, 0, 3, -1, 4])
    assert np.array_equal(out[0], ple.decode_row(table, 3, 32))
    assert np.array_equal(out[1], ple.decode_row(table, 0, 32))
    assert np.array_equal(out[2], out[0])
    assert np.all(np.isnan(out[3])) and np.all(np.isnan(out[4]))
