"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method (no quantizer, no rotation, no
product): it only draws seeded random tensors with the shapes and value
distributions of the pages' workloads (the Bonsai 27B decoder's linear layers,
K x N ne-order: 5120 x 10240 fused QKV, 5120 x 248320 output head, 5120 x 17408
FFN) so that the GPU path and the CPU oracle see identical bytes.

Generator: NumPy ``Generator(PCG64(seed))``, ``standard_normal(dtype=float32)``.
"""
from __future__ import annotations

import numpy as np

W_SEED_BASE = 1000
X_SEED_BASE = 2000


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def gaussian(seed: int, shape, offset: float = 0.0) -> np.ndarray:
    """fp32 N(0,1) (+ a constant DC offset) of the given shape."""
    a = rng(seed).standard_normal(size=shape, dtype=np.float32)
    if offset:
        a += np.float32(offset)
    return a


def weights(seed: int, N: int, K: int) -> np.ndarray:
    """Dense fp32 weights W [N][K] (K contiguous), N(0,1)."""
    return gaussian(seed, (N, K))


def activations(seed: int, M: int, K: int, offset: float = 0.0) -> np.ndarray:
    """fp32 activations x [M][K], N(0,1) plus an optional DC offset."""
    return gaussian(seed, (M, K), offset)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (torch CPU, nearest-even) and return the
    raw 16-bit patterns; used to make bf16 activation inputs."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 patterns to fp32 (exact: a 16-bit left shift)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def ternary_exact_weights(seed: int, N: int, K: int, exp2: int = 3,
                          group: int = 128) -> np.ndarray:
    """Weights t * 2^-exp2 with t in {-1, 0, +1} and one |t| = 1 forced into
    the first slot of every group, so the group's max|w| is exactly 2^-exp2.
    Used for integer-exact (tolerance 0) product tests."""
    r = rng(seed)
    t = r.integers(-1, 2, size=(N, K), dtype=np.int8)
    t = t.reshape(N, K // group, group)
    t[:, :, 0] = np.where(r.integers(0, 2, size=(N, K // group)) == 0, -1, 1)
    return (t.reshape(N, K).astype(np.float32) * np.float32(2.0 ** -exp2))


def int8_exact_weights(seed: int, N: int, K: int, exp2: int = 7) -> np.ndarray:
    """Weights q * 2^-exp2 with q in [-127, 127] and |q| = 127 forced into the
    first slot of every 32-group, so max|w| / 127 is exactly 2^-exp2."""
    r = rng(seed)
    q = r.integers(-127, 128, size=(N, K // 32, 32), dtype=np.int32)
    q[:, :, 0] = np.where(r.integers(0, 2, size=(N, K // 32)) == 0, -127, 127)
    return (q.reshape(N, K).astype(np.float32) * np.float32(2.0 ** -exp2))


def integer_activations(seed: int, M: int, K: int, lim: int = 64) -> np.ndarray:
    """Small integers in [-lim, lim] stored as fp32 (exact in fp32 and bf16
    for lim <= 256)."""
    return rng(seed).integers(-lim, lim + 1, size=(M, K)).astype(np.float32)


def signs(seed: int, K: int) -> np.ndarray:
    """A +-1 int8 sign vector of length K (about half negative, as on the
    Bonsai page's sign vectors)."""
    return np.where(rng(seed).integers(0, 2, size=K) == 0, -1, 1).astype(np.int8)


def random_bytes(seed: int, n: int) -> np.ndarray:
    """Uniform random bytes (foreign packed blobs, including code 3)."""
    return rng(seed).integers(0, 256, size=n, dtype=np.uint8)
