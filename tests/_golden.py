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


def stored_code_rows(plane, N: int, K: int, fmt: int):
    """Row-major code bytes [N][32 * blocks] as stored in a packed buffer: the
    code plane holds tiles of 16 rows x 32 bytes (one block), row r of a tile
    at byte 32 r, tiles ordered by 16-row block and then by block along K."""
    nb = K // (128 if fmt == 1 else 32)
    nt = (N + 15) // 16
    tiles = np.asarray(plane)[:nt * nb * 512].reshape(nt, nb, 16, 32)
    return tiles.transpose(0, 2, 1, 3).reshape(nt * 16, nb * 32)[:N]


def pq2_word_view(stored):
    """Stored PQ2_0 code bytes -> the block's own qs bytes (GGUF word view,
    code j of a little-endian word at bits 2j, 2j + 1).  A stored word keeps
    the even bits (the codes' low bits) in place and holds the odd bits (the
    high bits) rotated up by two, so they rotate back down by two."""
    s = np.ascontiguousarray(stored, dtype=np.uint8)
    w = s.view("<u4").astype(np.uint64)
    hi = w & 0xAAAAAAAA
    back = (w & 0x55555555) | (hi >> 2) | ((hi << 30) & 0xFFFFFFFF)
    return back.astype("<u4").view(np.uint8).reshape(s.shape)


def code_rows(plane, N: int, K: int, fmt: int):
    """Row-major code bytes [N][32 * blocks] of a packed buffer in the
    blocks' own byte order (PQ2_0 words back in the GGUF word view)."""
    rows = stored_code_rows(plane, N, K, fmt)
    return pq2_word_view(rows) if fmt == 1 else rows


def d_offset(N: int, K: int, fmt: int) -> int:
    """Byte offset of the fp16 scale plane: after whole 16-row code tiles,
    rounded up to 256."""
    nb = K // (128 if fmt == 1 else 32)
    qs = (N + 15) // 16 * 16 * nb * 32
    return (qs + 255) // 256 * 256


def scale_bytes(plane, N: int, K: int, fmt: int):
    """Scale bytes [N][blocks][2] (little-endian fp16) from a packed buffer:
    the scale plane holds chunks of 16 rows x 8 blocks (256 bytes, row r at
    byte 16 r, block b % 8 at byte 2 (b % 8)), ordered by 16-row block and
    then by 8-block run along K.  Also returns the padding slots (rows past N,
    blocks past the row's last) as a flat array, which must be zero."""
    import numpy as np
    nb = K // (128 if fmt == 1 else 32)
    nt, nc = (N + 15) // 16, (nb + 7) // 8
    off = d_offset(N, K, fmt)
    chunks = np.asarray(plane)[off:off + nt * nc * 256].reshape(nt, nc, 16, 8, 2)
    full = chunks.transpose(0, 2, 1, 3, 4).reshape(nt * 16, nc * 8, 2)
    pad = np.concatenate([full[N:].reshape(-1), full[:N, nb:].reshape(-1)])
    return full[:N, :nb], pad
