"""Reader for the hand-derived text fixtures in tests/golden/ (key: value lines)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            out[key.strip()] = val.strip()
    return out


def hex_bytes(s: str) -> np.ndarray:
    return np.array([int(t, 16) for t in s.split()], dtype=np.uint8)


def ints(s: str) -> np.ndarray:
    return np.array([int(t) for t in s.split()], dtype=np.int64)


def floats(s: str) -> np.ndarray:
    return np.array([float(t) for t in s.split()], dtype=np.float64)


def sparse_block(s: str, length: int) -> np.ndarray:
    """'i=v i=v ...' -> dense fp32 vector of the given length."""
    w = np.zeros(length, dtype=np.float32)
    for tok in s.split():
        i, _, v = tok.partition("=")
        w[int(i)] = np.float32(float(v))
    return w
