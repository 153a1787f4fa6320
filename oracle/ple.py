"""Oracle gather-and-decode of a Q4_0 per-row table (test infrastructure only;
see the package docstring).

The FlashNext release keeps an n-gram table of 320,001,536 rows of 160 values as
one Q4_0 tensor with groups of 32 along each row, decoded one row at a time
(Scion-FlashNext-176B-A6B card, "Model Overview" and "Weight Representation:
ternary PTQ1_0 + trained corrections + Q4_0 PLE").  The pages name the format
without spelling out its bytes; this oracle reads the name as ggml's Q4_0 block:

    bytes 0..1    the block scale d, IEEE binary16, little-endian
    bytes 2..17   16 code bytes; value j (0..15) is the low nibble of byte j,
                  value 16 + j the high nibble of byte j
    value = d * (nibble - 8)

A row of n values (n a multiple of 32) is n / 32 blocks back to back; rows
follow each other without padding.  Gathering row list idx gives out[i] = the
decoded row idx[i]; an index outside [0, rows) gives a row of NaN and reads
nothing.  Values are float64 (every d * (nibble - 8) is exact in float32 too).
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
BLOCK_BYTES = 18


def row_bytes(row_len: int) -> int:
    if row_len <= 0 or row_len % BLOCK:
        raise ValueError(f"row length {row_len} is not a positive multiple of {BLOCK}")
    return row_len // BLOCK * BLOCK_BYTES


def decode_block(block: np.ndarray) -> np.ndarray:
    """18 bytes -> the 32 values of one block (float64)."""
    b = np.asarray(block, dtype=np.uint8)
    d = float(b[:2].copy().view(np.float16)[0])
    q = b[2:18].astype(np.int64)
    nibbles = np.concatenate([q & 0x0F, q >> 4])
    return d * (nibbles - 8).astype(np.float64)


def decode_row(table: np.ndarray, r: int, row_len: int) -> np.ndarray:
    rb = row_bytes(row_len)
    row = np.asarray(table, dtype=np.uint8).reshape(-1)[r * rb:(r + 1) * rb]
    return np.concatenate([decode_block(row[k * BLOCK_BYTES:(k + 1) * BLOCK_BYTES])
                           for k in range(row_len // BLOCK)])


def gather(table: np.ndarray, n_rows: int, row_len: int, idx: np.ndarray) -> np.ndarray:
    """Decoded rows idx of a table of n_rows rows -> float64 [len(idx), row_len]."""
    idx = np.asarray(idx, dtype=np.int64).reshape(-1)
    out = np.full((idx.size, row_len), np.nan)
    for i, r in enumerate(idx):
        if 0 <= r < n_rows:
            out[i] = decode_row(table, int(r), row_len)
    return out
