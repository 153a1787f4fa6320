"""Pins for the oracle's container codec (CPU only).

Each pin fixes the codec by something other than the codec itself: the byte
arithmetic the cards print, hand-derived fixture blocks, exhaustive round trips
over every byte value, and decoders written with different library routines.
"""
import math

import numpy as np
import pytest

from golden_io import read_block_fixture
from oracle import codec

PQ2_0, PTQ1_0 = codec.PQ2_0, codec.PTQ1_0


# ---- byte arithmetic printed on the cards ------------------------------------
def test_block_sizes_and_bits_per_weight():
    # 35B-A3B card, "Weight Representation": 2.125 bits per weight for PQ2_0
    assert codec.block_bytes(PQ2_0) == 34
    assert codec.block_bytes(PQ2_0) * 8 / 128 == 2.125
    # FlashNext card, "Weight Representation": 24 + 2 + 2 = 28 bytes = 1.75 bpw
    assert codec.block_bytes(PTQ1_0) == 24 + 2 + 2 == 28
    assert codec.block_bytes(PTQ1_0) * 8 / 128 == 1.75
    # FlashNext card, "Highlights": entropy of {-1,0,+1} is 1.585 bpw, overhead about 10%
    assert abs(math.log2(3) - 1.585) < 5e-4
    assert 1.09 < 1.75 / math.log2(3) < 1.11
    # 24 bytes of 5 trits plus 8 remaining trits cover the group
    assert 24 * 5 + 2 * 4 == 128 and 3 ** 5 <= 256 and 3 ** 4 <= 256
    assert codec.packed_bytes(PQ2_0, 3072 * 512) == 3072 * 512 // 128 * 34
    assert codec.packed_bytes(PTQ1_0, 128) == 28


def test_unknown_format_and_ragged_sizes_rejected():
    with pytest.raises(codec.ContainerError, match="unknown container id 42"):
        codec.block_bytes(42)
    with pytest.raises(codec.ContainerError):
        codec.packed_bytes(PQ2_0, 100)


# ---- hand-derived fixtures -----------------------------------------------------
@pytest.mark.parametrize("fmt,name", [(PQ2_0, "pq2_0_block.txt"), (PTQ1_0, "ptq1_0_block.txt")])
def test_golden_block(fmt, name):
    trits, scale, data = read_block_fixture(name)
    packed = codec.pack(fmt, trits, np.array([scale], dtype=np.uint16))
    assert packed.tobytes() == data.tobytes()
    t2, s2 = codec.unpack(fmt, data, 128)
    assert np.array_equal(t2, trits) and int(s2[0]) == scale
    w = codec.decode(fmt, data, 128)
    sval = float(np.array([scale], dtype=np.uint16).view(np.float16)[0])
    assert np.array_equal(w, sval * trits.astype(np.float64))


# ---- exhaustive round trips over byte values -----------------------------------
def _valid_pq2_bytes():
    vals = []
    for v in range(256):
        if all(((v >> (2 * i)) & 3) != 2 for i in range(4)):
            vals.append(v)
    return vals


def test_pq2_exhaustive_byte_values():
    valid = _valid_pq2_bytes()
    assert len(valid) == 81  # 3 valid codes per 2-bit field
    for pos in range(32):
        for chunk in range(0, 81, 27):
            nb = 27
            blocks = np.zeros((nb, 34), dtype=np.uint8)
            blocks[:, pos] = valid[chunk:chunk + nb]
            blocks[:, 32], blocks[:, 33] = 0x00, 0x3C
            raw = blocks.reshape(-1)
            t, s = codec.unpack(PQ2_0, raw, nb * 128)
            assert np.array_equal(codec.pack(PQ2_0, t, s), raw)


def test_pq2_invalid_code_located():
    for pos in (0, 7, 31):
        for field in range(4):
            blocks = np.zeros((3, 34), dtype=np.uint8)
            blocks[2, pos] = 2 << (2 * field)
            with pytest.raises(codec.ContainerError) as ei:
                codec.unpack(PQ2_0, blocks.reshape(-1), 3 * 128)
            assert ei.value.block == 2 and ei.value.byte == pos


def test_ptq1_exhaustive_byte_values():
    for pos in range(24):
        blocks = np.zeros((243, 28), dtype=np.uint8)
        blocks[:, pos] = np.arange(243)
        blocks[:, 27] = 0x3C
        raw = blocks.reshape(-1)
        t, s = codec.unpack(PTQ1_0, raw, 243 * 128)
        assert np.array_equal(codec.pack(PTQ1_0, t, s), raw)
    for pos in (24, 25):
        blocks = np.zeros((81, 28), dtype=np.uint8)
        blocks[:, pos] = np.arange(81)
        raw = blocks.reshape(-1)
        t, s = codec.unpack(PTQ1_0, raw, 81 * 128)
        assert np.array_equal(codec.pack(PTQ1_0, t, s), raw)


def test_ptq1_invalid_bytes_located():
    for pos, lo in [(0, 243), (23, 243), (24, 81), (25, 81)]:
        for v in range(lo, 256):
            blocks = np.zeros((2, 28), dtype=np.uint8)
            blocks[1, pos] = v
            with pytest.raises(codec.ContainerError) as ei:
                codec.unpack(PTQ1_0, blocks.reshape(-1), 256)
            assert ei.value.block == 1 and ei.value.byte == pos


def test_nonfinite_scales_rejected():
    t = np.zeros(256, dtype=np.int8)
    for bad in (0x7C00, 0xFC00, 0x7E00):
        with pytest.raises(codec.ContainerError):
            codec.pack(PQ2_0, t, np.array([0x3C00, bad], dtype=np.uint16))
    blocks = np.zeros((1, 28), dtype=np.uint8)
    blocks[0, 26], blocks[0, 27] = 0x00, 0x7C
    with pytest.raises(codec.ContainerError):
        codec.unpack(PTQ1_0, blocks.reshape(-1), 128)


def test_pack_rejects_out_of_range_trits():
    t = np.zeros(128, dtype=np.int8)
    t[5] = 2
    with pytest.raises(codec.ContainerError):
        codec.pack(PQ2_0, t, np.array([0x3C00], dtype=np.uint16))


# ---- decoders written with other library routines --------------------------------
def test_pq2_decode_matches_unpackbits_reader():
    rng = np.random.default_rng(1)
    t = rng.integers(-1, 2, size=128 * 9).astype(np.int8)
    s = np.abs(rng.normal(0, 1, 9)).astype(np.float16).view(np.uint16)
    raw = codec.pack(PQ2_0, t, s).reshape(9, 34)
    bits = np.unpackbits(raw[:, :32], axis=1, bitorder="little").reshape(9, 128, 2)
    lo, hi = bits[:, :, 0].astype(int), bits[:, :, 1].astype(int)
    # two's complement of the 2-bit field: value = lo - 2*hi
    vals = (lo - 2 * hi).reshape(-1)
    assert np.array_equal(vals, t)
    scales = raw[:, 32:34].copy().view("<f2").astype(np.float64).reshape(-1)
    assert np.array_equal(codec.decode(PQ2_0, raw.reshape(-1), 9 * 128),
                          np.repeat(scales, 128) * t)


def test_ptq1_decode_matches_base_repr_reader():
    rng = np.random.default_rng(2)
    t = rng.integers(-1, 2, size=128 * 5).astype(np.int8)
    s = np.abs(rng.normal(0, 1, 5)).astype(np.float16).view(np.uint16)
    raw = codec.pack(PTQ1_0, t, s).reshape(5, 28)
    got = []
    for blk in raw:
        for b in range(26):
            ndig = 5 if b < 24 else 4
            digits = np.base_repr(int(blk[b]), base=3).rjust(ndig, "0")[::-1]  # least significant first
            got += [{"0": 0, "1": 1, "2": -1}[c] for c in digits[:ndig]]
    assert np.array_equal(np.array(got), t)
