"""Reader for the hand-derived fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, vals = line.split(":", 1)
            out[key.strip()] = [int(v, 16) for v in vals.split()]
    return out


def bf16_row(vals):
    return np.array(vals, dtype=np.uint16).reshape(1, -1)


def u8(vals):
    return np.array(vals, dtype=np.uint8)
