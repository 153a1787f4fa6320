"""Reader for the hand-derived text fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_block_fixture(name):
    """-> (trits int8[128], scale_bits int, bytes uint8[n]) of a container fixture."""
    scale, data = None, None
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line.startswith("scale_f16"):
            scale = int(line.split("=")[1], 16)
        elif line.startswith("bytes"):
            data = np.array([int(v, 16) for v in line.split("=")[1].split()], dtype=np.uint8)
    j = np.arange(128)
    trits = np.where(j % 3 == 0, 1, np.where(j % 3 == 1, -1, 0)).astype(np.int8)
    return trits, scale, data
