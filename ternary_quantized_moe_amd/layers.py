"""Host-side assembly of a layer's expert containers with the library's packer."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .binding import pack, packed_bytes, tile_container

BANK_SLACK = 16  # readable bytes the library needs after the last bank (MOE_BANK_SLACK)


def pack_expert(fmt: int, trits, scales) -> np.ndarray:
    """[gate, up, down] trits ([rows, cols] int8) and fp16-bit scales -> one
    bank's bytes: each matrix packed row-major, then put in the tile-major block
    order the expert kernels read."""
    out = []
    for t, s in zip(trits, scales):
        rows, cols = np.shape(t)
        out.append(tile_container(fmt, pack(fmt, t, s), rows, cols))
    return np.concatenate(out)


def build_banks(source, n_banks: int, formats: np.ndarray, d_model: int, d_ff: int, threads: int = 0):
    """Pack every bank back to back.  source(e) -> ([gate, up, down] trits,
    [gate, up, down] fp16 scale bits).  Returns (data uint8, offsets int64); data
    ends with BANK_SLACK zero bytes."""
    sizes = [3 * packed_bytes(int(formats[e]), d_model * d_ff) for e in range(n_banks)]
    offsets = np.zeros(n_banks, dtype=np.int64)
    offsets[1:] = np.cumsum(sizes)[:-1]
    data = np.zeros(int(sum(sizes)) + BANK_SLACK, dtype=np.uint8)

    def one(e):
        trits, scales = source(e)
        data[offsets[e]:offsets[e] + sizes[e]] = pack_expert(int(formats[e]), trits, scales)

    threads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(n_banks)))
    return data, offsets
