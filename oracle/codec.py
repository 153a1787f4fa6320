"""Oracle container codec (test infrastructure only; see the package docstring).

PQ2_0, 34 bytes per group of 128 weights (Scion-35B-A3B card, "Weight
Representation": ternary values, 2-bit slots, one shared FP16 scale per group of
128, 2.125 bits per weight):
    bytes 0..31   2-bit codes; weight j of the group sits in byte j // 4,
                  bits 2*(j % 4) .. 2*(j % 4) + 1 (least significant first)
                  code 00 -> 0, 01 -> +1, 11 -> -1; 10 is not a valid code
    bytes 32..33  the group scale, IEEE binary16, little-endian

PTQ1_0, 28 bytes per group of 128 weights (Scion-FlashNext-176B-A6B card,
"Weight Representation": 24 bytes of 5-trit data, 2 bytes holding the remaining
trits, the 2-byte group scale, 1.75 bits per weight):
    bytes 0..23   byte b holds weights 5b .. 5b+4 as sum_i d_i * 3**i (<= 242)
    bytes 24..25  byte 24+m holds weights 120+4m .. 123+4m as sum_i d_i * 3**i (<= 80)
    bytes 26..27  the group scale, IEEE binary16, little-endian
    base-3 digit d of a weight t: d = t mod 3 (0 -> 0, 1 -> +1, 2 -> -1)

The value of a weight is scale * t, with no offset.  Groups run along the input
(K) dimension of each matrix row.
"""
from __future__ import annotations

import numpy as np

PQ2_0 = 142
PTQ1_0 = 143
GROUP = 128
BLOCK_BYTES = {PQ2_0: 34, PTQ1_0: 28}


class ContainerError(ValueError):
    """Invalid container content or argument.  `block` and `byte` locate a bad byte."""

    def __init__(self, msg, block=None, byte=None):
        super().__init__(msg)
        self.block = block
        self.byte = byte


def block_bytes(fmt: int) -> int:
    if fmt not in BLOCK_BYTES:
        raise ContainerError(f"unknown container id {fmt}; valid ids are 142 (PQ2_0) and 143 (PTQ1_0)")
    return BLOCK_BYTES[fmt]


def packed_bytes(fmt: int, n_weights: int) -> int:
    if n_weights % GROUP:
        raise ContainerError(f"weight count {n_weights} is not a multiple of {GROUP}")
    return n_weights // GROUP * block_bytes(fmt)


def _check_scales(scale_bits: np.ndarray):
    bad = np.nonzero((scale_bits & 0x7C00) == 0x7C00)[0]
    if bad.size:
        raise ContainerError(f"non-finite fp16 scale in group {int(bad[0])}", block=int(bad[0]))


# --------------------------------------------------------------------------- PQ2_0
def _pq2_pack(trits: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    nb = trits.size // GROUP
    t = trits.reshape(nb, 32, 4).astype(np.int64)
    # two's-complement 2-bit code: 0 -> 00, +1 -> 01, -1 -> 11
    codes = np.where(t < 0, 3, t)
    byte = codes[:, :, 0] | (codes[:, :, 1] << 2) | (codes[:, :, 2] << 4) | (codes[:, :, 3] << 6)
    out = np.empty((nb, 34), dtype=np.uint8)
    out[:, :32] = byte.astype(np.uint8)
    out[:, 32] = (scale_bits & 0xFF).astype(np.uint8)
    out[:, 33] = (scale_bits >> 8).astype(np.uint8)
    return out.reshape(-1)


def _pq2_unpack(data: np.ndarray, nb: int):
    blk = data.reshape(nb, 34).astype(np.int64)
    codes = np.stack([(blk[:, :32] >> (2 * i)) & 3 for i in range(4)], axis=2)  # [nb, 32, 4]
    bad = np.argwhere(codes == 2)
    if bad.size:
        b, byte, _ = (int(v) for v in bad[0])
        raise ContainerError(f"invalid 2-bit code 10 in group {b}, byte {byte}", block=b, byte=byte)
    trits = np.where(codes == 3, -1, codes).astype(np.int8).reshape(-1)
    scale_bits = (blk[:, 32] | (blk[:, 33] << 8)).astype(np.uint16)
    return trits, scale_bits


# --------------------------------------------------------------------------- PTQ1_0
_POW3 = np.array([1, 3, 9, 27, 81], dtype=np.int64)


def _ptq1_pack(trits: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    nb = trits.size // GROUP
    d = np.mod(trits.reshape(nb, GROUP).astype(np.int64), 3)  # -1 -> 2
    out = np.empty((nb, 28), dtype=np.uint8)
    out[:, :24] = (d[:, :120].reshape(nb, 24, 5) * _POW3).sum(axis=2).astype(np.uint8)
    out[:, 24:26] = (d[:, 120:].reshape(nb, 2, 4) * _POW3[:4]).sum(axis=2).astype(np.uint8)
    out[:, 26] = (scale_bits & 0xFF).astype(np.uint8)
    out[:, 27] = (scale_bits >> 8).astype(np.uint8)
    return out.reshape(-1)


def _ptq1_unpack(data: np.ndarray, nb: int):
    blk = data.reshape(nb, 28).astype(np.int64)
    bad = np.argwhere(blk[:, :24] >= 243)
    if bad.size:
        b, byte = (int(v) for v in bad[0])
        raise ContainerError(f"base-3 data byte {int(blk[b, byte])} > 242 in group {b}, byte {byte}",
                             block=b, byte=byte)
    bad = np.argwhere(blk[:, 24:26] >= 81)
    if bad.size:
        b, m = (int(v) for v in bad[0])
        raise ContainerError(f"base-3 tail byte {int(blk[b, 24 + m])} > 80 in group {b}, byte {24 + m}",
                             block=b, byte=24 + m)
    data_digits = (blk[:, :24, None] // _POW3) % 3            # [nb, 24, 5]
    tail_digits = (blk[:, 24:26, None] // _POW3[:4]) % 3      # [nb, 2, 4]
    digits = np.concatenate([data_digits.reshape(nb, 120), tail_digits.reshape(nb, 8)], axis=1)
    trits = np.where(digits == 2, -1, digits).astype(np.int8).reshape(-1)
    scale_bits = (blk[:, 26] | (blk[:, 27] << 8)).astype(np.uint16)
    return trits, scale_bits


# --------------------------------------------------------------------------- public
def pack(fmt: int, trits: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """trits int8 in {-1,0,+1} (n, n % 128 == 0), scale_bits uint16 (n/128) -> uint8 container."""
    trits = np.ascontiguousarray(trits, dtype=np.int8).reshape(-1)
    scale_bits = np.ascontiguousarray(scale_bits, dtype=np.uint16).reshape(-1)
    block_bytes(fmt)
    if trits.size % GROUP:
        raise ContainerError(f"weight count {trits.size} is not a multiple of {GROUP}")
    if scale_bits.size != trits.size // GROUP:
        raise ContainerError("need one scale per group of 128 weights")
    bad = np.nonzero((trits < -1) | (trits > 1))[0]
    if bad.size:
        raise ContainerError(f"weight {int(bad[0])} is not in {{-1, 0, +1}}", block=int(bad[0]) // GROUP)
    _check_scales(scale_bits)
    return _pq2_pack(trits, scale_bits) if fmt == PQ2_0 else _ptq1_pack(trits, scale_bits)


def unpack(fmt: int, data: np.ndarray, n_weights: int):
    """uint8 container of n_weights -> (trits int8[n], scale_bits uint16[n/128]); validates codes."""
    nbytes = packed_bytes(fmt, n_weights)
    data = np.ascontiguousarray(data, dtype=np.uint8).reshape(-1)
    if data.size < nbytes:
        raise ContainerError(f"container holds {data.size} bytes, {nbytes} needed")
    data = data[:nbytes]
    nb = n_weights // GROUP
    trits, scales = _pq2_unpack(data, nb) if fmt == PQ2_0 else _ptq1_unpack(data, nb)
    _check_scales(scales)
    return trits, scales


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def decode(fmt: int, data: np.ndarray, n_weights: int) -> np.ndarray:
    """Weight values scale * t (float64, length n_weights) of a container."""
    trits, scales = unpack(fmt, data, n_weights)
    return trits.astype(np.float64) * np.repeat(f16_to_f64(scales), GROUP)
