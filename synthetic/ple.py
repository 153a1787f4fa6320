"""Seeded Q4_0 n-gram tables and row lists, the input of the row gather.

The FlashNext release's table has 320,001,536 rows of 160 values in Q4_0
(Scion-FlashNext-176B-A6B card, "Model Overview"); the pages publish neither
its contents nor how rows are chosen per token.  These tables hold uniform
random code bytes and binary16 scales 0.01 * N(0, 1) (both signs, as a block
scale can have); row lists are uniform over the table, the way hashed n-gram
rows would fall.  Only numbers are drawn here, nothing of the decode.
"""
from __future__ import annotations

import numpy as np

_SEED = 0x5C1B
BLOCK, BLOCK_BYTES = 32, 18
SCALE_SIGMA = 0.01


def q4_table(n_rows: int, row_len: int, seed: int = 0) -> np.ndarray:
    """uint8 [n_rows, row_len / 32 * 18], host memory."""
    nb = row_len // BLOCK
    rng = np.random.default_rng(np.random.SeedSequence(_SEED, spawn_key=(seed, n_rows, row_len)))
    t = rng.integers(0, 256, size=(n_rows, nb, BLOCK_BYTES), dtype=np.uint8)
    d = (rng.standard_normal((n_rows, nb)) * SCALE_SIGMA).astype(np.float16)
    t[:, :, 0:2] = d.view(np.uint8).reshape(n_rows, nb, 2)
    return t.reshape(n_rows, nb * BLOCK_BYTES)


def q4_table_device(n_rows: int, row_len: int, seed: int = 0, device="cuda"):
    """The same distribution drawn on the device with torch's generator (the
    full 28.8 GB table would take the host minutes): uint8 [n_rows, row bytes]."""
    import torch
    nb = row_len // BLOCK
    g = torch.Generator(device=device)
    g.manual_seed(_SEED * 1_000_003 + seed)
    t = torch.empty((n_rows, nb, BLOCK_BYTES), dtype=torch.uint8, device=device)
    step = 1 << 24
    for r0 in range(0, n_rows, step):
        r1 = min(n_rows, r0 + step)
        t[r0:r1].random_(0, 256, generator=g)
        d = (torch.randn((r1 - r0, nb), generator=g, device=device) * SCALE_SIGMA).to(torch.float16)
        t[r0:r1, :, 0:2] = d.view(torch.uint8).view(r1 - r0, nb, 2)
    return t.view(n_rows, nb * BLOCK_BYTES)


def row_list(n: int, n_rows: int, seed: int = 0) -> np.ndarray:
    """n row numbers uniform over [0, n_rows), int64, host memory."""
    rng = np.random.default_rng(np.random.SeedSequence(_SEED, spawn_key=(seed, n, n_rows, 1)))
    return rng.integers(0, n_rows, size=n, dtype=np.int64)


def row_list_device(n: int, n_rows: int, seed: int = 0, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_SEED * 1_000_033 + seed)
    return torch.randint(0, n_rows, (n,), generator=g, device=device, dtype=torch.int64)
