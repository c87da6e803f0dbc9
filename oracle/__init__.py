"""CPU oracle for the quantized GEMV / GEMM path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library
(``gemm_kq_gemv_amd``) never imports it, and this package never imports the
product library: the two share no code.

The arithmetic lives in ``kq_oracle.c`` (plain C, binary64 products); this
module only marshals NumPy arrays into it with ctypes.  Each function names the
page passage it follows; see the header ``kq_oracle.h``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkq_oracle.so")
_SRC = os.path.join(_HERE, "kq_oracle.c")

FMT_PQ2_0 = 1
FMT_Q8_0 = 2
GROUP = {FMT_PQ2_0: 128, FMT_Q8_0: 32}


def build(verbose: bool = False) -> str:
    """Compile kq_oracle.c into libkq_oracle.so with gcc (no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", _LIB_PATH, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        L = C.CDLL(_LIB_PATH)
        p = C.c_void_p
        i64 = C.c_int64
        L.kqo_f16_from_f32.restype = C.c_uint16
        L.kqo_f16_from_f32.argtypes = [C.c_float]
        L.kqo_f32_from_f16.restype = C.c_float
        L.kqo_f32_from_f16.argtypes = [C.c_uint16]
        L.kqo_bf16_from_f32.restype = C.c_uint16
        L.kqo_bf16_from_f32.argtypes = [C.c_float]
        L.kqo_f32_from_bf16.restype = C.c_float
        L.kqo_f32_from_bf16.argtypes = [C.c_uint16]
        for name in ("kqo_f16_from_f32_n", "kqo_f32_from_f16_n",
                     "kqo_bf16_from_f32_n", "kqo_f32_from_bf16_n"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [p, p, i64]
        for name in ("kqo_pack_pq2_aos", "kqo_pack_q8_aos", "kqo_unpack_pq2_aos",
                     "kqo_unpack_pq2_aos_words", "kqo_unpack_q8_aos"):
            getattr(L, name).restype = C.c_int
            getattr(L, name).argtypes = [p, i64, i64, p]
        for name in ("kqo_pq2_to_ptq1_aos", "kqo_ptq1_to_pq2_aos", "kqo_unpack_ptq1_aos"):
            getattr(L, name).restype = C.c_int
            getattr(L, name).argtypes = [p, i64, i64, p]
        L.kqo_planar_bytes.restype = i64
        L.kqo_planar_bytes.argtypes = [C.c_int, i64, i64]
        L.kqo_aos_to_planar.restype = C.c_int
        L.kqo_aos_to_planar.argtypes = [C.c_int, p, i64, i64, p]
        L.kqo_hadamard_matrix.restype = C.c_int
        L.kqo_hadamard_matrix.argtypes = [C.c_int32, p]
        L.kqo_rotate.restype = C.c_int
        L.kqo_rotate.argtypes = [p, i64, i64, C.c_int32, p, p]
        L.kqo_matmul.restype = None
        L.kqo_matmul.argtypes = [p, p, i64, i64, i64, p, p]
        L.kqo_gemv_aos.restype = C.c_int
        L.kqo_gemv_aos.argtypes = [C.c_int, p, i64, i64, p, i64, C.c_int32,
                                   p, p, p]
        L.kqo_num_threads.restype = C.c_int
        L.kqo_num_threads.argtypes = []
        L.kqo_set_num_threads.restype = None
        L.kqo_set_num_threads.argtypes = [C.c_int]
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments")


# ---- codecs -------------------------------------------------------------

def f16_from_f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().kqo_f16_from_f32_n(_ptr(a), _ptr(out), a.size)
    return out


def f32_from_f16(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().kqo_f32_from_f16_n(_ptr(h), _ptr(out), h.size)
    return out


def bf16_from_f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().kqo_bf16_from_f32_n(_ptr(a), _ptr(out), a.size)
    return out


def f32_from_bf16(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    lib().kqo_f32_from_bf16_n(_ptr(b), _ptr(out), b.size)
    return out


# ---- formats ------------------------------------------------------------

def pack_pq2_aos(W) -> np.ndarray:
    """PQ2_0 AoS bytes [N * K/128 * 34] (Bonsai page sec. 3.1)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    out = np.empty(N * (K // 128) * 34, dtype=np.uint8)
    _check(lib().kqo_pack_pq2_aos(_ptr(W), N, K, _ptr(out)), "pack_pq2")
    return out


def pack_q8_aos(W) -> np.ndarray:
    """Q8_0 AoS bytes [N * K/32 * 34] (Kipp architecture, Weight quantization)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    out = np.empty(N * (K // 32) * 34, dtype=np.uint8)
    _check(lib().kqo_pack_q8_aos(_ptr(W), N, K, _ptr(out)), "pack_q8")
    return out


def pq2_to_ptq1_aos(pq2, N: int, K: int) -> np.ndarray:
    """PTQ1_0 blocks [N * K/128 * 28] holding the trits of PQ2_0 blocks
    (Bonsai page sec. 3.2)."""
    pq2 = np.ascontiguousarray(pq2, dtype=np.uint8)
    out = np.empty(N * (K // 128) * 28, dtype=np.uint8)
    _check(lib().kqo_pq2_to_ptq1_aos(_ptr(pq2), N, K, _ptr(out)), "pq2_to_ptq1")
    return out


def ptq1_to_pq2_aos(ptq1, N: int, K: int) -> np.ndarray:
    """The lossless PTQ1_0 -> PQ2_0 transcode (Bonsai page sec. 3.2)."""
    ptq1 = np.ascontiguousarray(ptq1, dtype=np.uint8)
    out = np.empty(N * (K // 128) * 34, dtype=np.uint8)
    _check(lib().kqo_ptq1_to_pq2_aos(_ptr(ptq1), N, K, _ptr(out)), "ptq1_to_pq2")
    return out


def unpack_ptq1_aos(ptq1, N: int, K: int) -> np.ndarray:
    ptq1 = np.ascontiguousarray(ptq1, dtype=np.uint8)
    out = np.empty((N, K), dtype=np.float64)
    _check(lib().kqo_unpack_ptq1_aos(_ptr(ptq1), N, K, _ptr(out)), "unpack_ptq1")
    return out


def planar_bytes(fmt: int, N: int, K: int) -> int:
    return int(lib().kqo_planar_bytes(fmt, N, K))


def aos_to_planar(fmt: int, aos, N: int, K: int) -> np.ndarray:
    aos = np.ascontiguousarray(aos, dtype=np.uint8)
    out = np.empty(planar_bytes(fmt, N, K), dtype=np.uint8)
    _check(lib().kqo_aos_to_planar(fmt, _ptr(aos), N, K, _ptr(out)), "aos_to_planar")
    return out


def unpack_pq2_aos(aos, N: int, K: int, word_view: bool = False) -> np.ndarray:
    aos = np.ascontiguousarray(aos, dtype=np.uint8)
    out = np.empty((N, K), dtype=np.float64)
    fn = lib().kqo_unpack_pq2_aos_words if word_view else lib().kqo_unpack_pq2_aos
    _check(fn(_ptr(aos), N, K, _ptr(out)), "unpack_pq2")
    return out


def unpack_q8_aos(aos, N: int, K: int) -> np.ndarray:
    aos = np.ascontiguousarray(aos, dtype=np.uint8)
    out = np.empty((N, K), dtype=np.float64)
    _check(lib().kqo_unpack_q8_aos(_ptr(aos), N, K, _ptr(out)), "unpack_q8")
    return out


def unpack_aos(fmt: int, aos, N: int, K: int) -> np.ndarray:
    return unpack_pq2_aos(aos, N, K) if fmt == FMT_PQ2_0 else unpack_q8_aos(aos, N, K)


# ---- rotation -----------------------------------------------------------

def hadamard_matrix(n: int) -> np.ndarray:
    out = np.empty((n, n), dtype=np.int8)
    _check(lib().kqo_hadamard_matrix(n, _ptr(out)), "hadamard_matrix")
    return out


def rotate(x, block_len: int, signs=None) -> np.ndarray:
    """x' = (1/sqrt(n)) H_n (s (.) x) per n-block of each row (Bonsai sec. 4.1-4.2)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    squeeze = x.ndim == 1
    x2 = x.reshape(1, -1) if squeeze else x
    M, K = x2.shape
    s = None if signs is None else np.ascontiguousarray(signs, dtype=np.int8)
    out = np.empty((M, K), dtype=np.float64)
    _check(lib().kqo_rotate(_ptr(x2), M, K, block_len, _ptr(s), _ptr(out)), "rotate")
    return out.reshape(-1) if squeeze else out


# ---- product ------------------------------------------------------------

def matmul(Wd, xr):
    """y[m][n] = sum_k Wd[n][k] xr[m][k] and the bound sum_k |Wd[n][k] xr[m][k]|."""
    Wd = np.ascontiguousarray(Wd, dtype=np.float64)
    xr = np.ascontiguousarray(xr, dtype=np.float64)
    N, K = Wd.shape
    M = xr.shape[0]
    y = np.empty((M, N), dtype=np.float64)
    b = np.empty((M, N), dtype=np.float64)
    lib().kqo_matmul(_ptr(Wd), _ptr(xr), M, N, K, _ptr(y), _ptr(b))
    return y, b


def gemv_aos(fmt: int, aos, N: int, K: int, x, block_len: int, signs=None):
    """Whole path on the CPU: unpack, rotate, binary64 product.  x fp32 [M][K]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    M = x.shape[0]
    aos = np.ascontiguousarray(aos, dtype=np.uint8)
    s = None if signs is None else np.ascontiguousarray(signs, dtype=np.int8)
    y = np.empty((M, N), dtype=np.float64)
    b = np.empty((M, N), dtype=np.float64)
    _check(lib().kqo_gemv_aos(fmt, _ptr(aos), N, K, _ptr(x), M, block_len, _ptr(s),
                              _ptr(y), _ptr(b)), "gemv")
    return y, b


def num_threads() -> int:
    return int(lib().kqo_num_threads())


def set_num_threads(n: int) -> None:
    lib().kqo_set_num_threads(int(n))
