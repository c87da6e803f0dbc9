"""ctypes binding for libkq.so -- argument marshalling only.

Every function here has the name of the C entry point it calls (see
include/kq.h) and does nothing but turn tensors into device pointers, pick
the current HIP stream and turn a non-zero kq_status into a KQError.  All
arithmetic happens in the HIP kernels behind the C ABI; there is no fallback:
if libkq.so is missing, importing this module raises.

Pointer arguments accept a torch tensor (its data_ptr), None (NULL) or a raw
integer address.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -m gemm_kq_gemv_amd.build or __graft_entry__.build())")

_lib = C.CDLL(LIB_PATH)

KQ_FMT_PQ2_0 = 1
KQ_FMT_Q8_0 = 2
KQ_F32 = 0
KQ_BF16 = 1
KQ_OK = 0
STATUS_NAMES = {0: "KQ_OK", 1: "KQ_EINVAL", 2: "KQ_ESHAPE", 3: "KQ_EALIGN",
                4: "KQ_EWORKSPACE", 5: "KQ_EUNSUPPORTED", 6: "KQ_EDEVICE"}

# exported symbols, in include/kq.h order, then the measurement instruments of
# include/kq_probe.h
EXPORTS = ("kq_status_string", "kq_packed_bytes", "kq_pack_pq2", "kq_pack_q8",
           "kq_transcode_ptq1", "kq_unpack", "kq_hadamard_blocks", "kq_workspace_bytes", "kq_gemv",
           "kq_gemv_noalloc", "kq_gemv_multi", "kq_gemm")
PROBE_EXPORTS = ("kq_probe_read", "kq_probe_mfma", "kq_probe_gemv_loads")
MAX_SETS = 4

_p = C.c_void_p
_i64 = C.c_int64
_i32 = C.c_int32
_lib.kq_status_string.restype = C.c_char_p
_lib.kq_status_string.argtypes = [C.c_int]
_lib.kq_packed_bytes.restype = C.c_size_t
_lib.kq_packed_bytes.argtypes = [C.c_int, _i64, _i64]
for _n in ("kq_pack_pq2", "kq_pack_q8"):
    getattr(_lib, _n).restype = C.c_int
    getattr(_lib, _n).argtypes = [_p, _i64, _i64, _p, _p]
_lib.kq_transcode_ptq1.restype = C.c_int
_lib.kq_transcode_ptq1.argtypes = [_p, _i64, _i64, _p, _p]
_lib.kq_unpack.restype = C.c_int
_lib.kq_unpack.argtypes = [C.c_int, _p, _i64, _i64, _p, _p]
_lib.kq_hadamard_blocks.restype = C.c_int
_lib.kq_hadamard_blocks.argtypes = [_p, C.c_int, _p, C.c_int, _i64, _i64, _i32, _p, _p]
_lib.kq_workspace_bytes.restype = C.c_size_t
_lib.kq_workspace_bytes.argtypes = [_i32, C.c_int, _i64, _i64, _i64, _i32, _i32]
_lib.kq_gemv.restype = C.c_int
_lib.kq_gemv.argtypes = [C.c_int, _p, _i64, _i64, _p, _i64, _i32, _p, _i32, _p, _p,
                         C.c_size_t, _p]
_lib.kq_gemv_noalloc.restype = C.c_int
_lib.kq_gemv_noalloc.argtypes = [C.c_int, _p, _i64, _i64, _p, _i64, _i32, _p, _i32, _p, _p]
_lib.kq_gemv_multi.restype = C.c_int
_lib.kq_gemv_multi.argtypes = [C.c_int, _i32, C.POINTER(_p), C.POINTER(_i64), _i64, _p, _i64,
                               _i32, _p, C.POINTER(_p), _p]
_lib.kq_gemm.restype = C.c_int
_lib.kq_gemm.argtypes = [C.c_int, _p, _i64, _i64, _p, C.c_int, _i64, _i32, _p, _p, _p,
                         C.c_size_t, _p]
_lib.kq_probe_read.restype = C.c_int
_lib.kq_probe_read.argtypes = [_p, C.c_size_t, _i32, _i32, _i32, _p, _p]
_lib.kq_probe_mfma.restype = C.c_int
_lib.kq_probe_mfma.argtypes = [_i32, _i32, _i32, _p, _p]
_lib.kq_probe_gemv_loads.restype = C.c_int
_lib.kq_probe_gemv_loads.argtypes = [C.c_int, _p, _i64, _i64, _p, _i64, _i32, _i32, _p, _p]


class KQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{where}: {kq_status_string(status)}")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        if not torch.cuda.is_available():
            return None
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str):
    if rc != KQ_OK:
        raise KQError(rc, where)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return KQ_F32
    if t.dtype == torch.bfloat16:
        return KQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def kq_status_string(status: int) -> str:
    return _lib.kq_status_string(status).decode()


def kq_packed_bytes(fmt: int, N: int, K: int) -> int:
    return int(_lib.kq_packed_bytes(fmt, N, K))


def kq_pack_pq2(W, N: int, K: int, packed, stream=None):
    _check(_lib.kq_pack_pq2(_ptr(W), N, K, _ptr(packed), _stream(stream)), "kq_pack_pq2")


def kq_pack_q8(W, N: int, K: int, packed, stream=None):
    _check(_lib.kq_pack_q8(_ptr(W), N, K, _ptr(packed), _stream(stream)), "kq_pack_q8")


def kq_transcode_ptq1(ptq1, N: int, K: int, packed, stream=None):
    _check(_lib.kq_transcode_ptq1(_ptr(ptq1), N, K, _ptr(packed), _stream(stream)),
           "kq_transcode_ptq1")


def kq_unpack(fmt: int, packed, N: int, K: int, W_out, stream=None):
    _check(_lib.kq_unpack(fmt, _ptr(packed), N, K, _ptr(W_out), _stream(stream)), "kq_unpack")


def kq_hadamard_blocks(x, x_dt: int, xr, xr_dt: int, M: int, K: int, block_len: int,
                       signs=None, stream=None):
    _check(_lib.kq_hadamard_blocks(_ptr(x), x_dt, _ptr(xr), xr_dt, M, K, block_len,
                                   _ptr(signs), _stream(stream)), "kq_hadamard_blocks")


def kq_workspace_bytes(op: int, fmt: int, M: int, N: int, K: int, block_len: int,
                       split_k: int = 0) -> int:
    return int(_lib.kq_workspace_bytes(op, fmt, M, N, K, block_len, split_k))


def kq_gemv(fmt: int, packed, N: int, K: int, x, M: int, block_len: int, signs,
            split_k: int, y, workspace, ws_bytes: int, stream=None):
    _check(_lib.kq_gemv(fmt, _ptr(packed), N, K, _ptr(x), M, block_len, _ptr(signs),
                        split_k, _ptr(y), _ptr(workspace), ws_bytes, _stream(stream)),
           "kq_gemv")


def kq_gemv_noalloc(fmt: int, packed, N: int, K: int, x, M: int, block_len: int, signs,
                    split_k: int, y, stream=None):
    _check(_lib.kq_gemv_noalloc(fmt, _ptr(packed), N, K, _ptr(x), M, block_len, _ptr(signs),
                                split_k, _ptr(y), _stream(stream)), "kq_gemv_noalloc")


def kq_gemv_multi(fmt: int, nsets: int, packed, N, K: int, x, M: int, block_len: int, signs,
                  y, stream=None):
    """packed, N, y: sequences of nsets entries (host arrays of the C call)."""
    P = (_p * max(nsets, 1))(*[_ptr(t) for t in packed[:nsets]])
    Ns = (_i64 * max(nsets, 1))(*[int(n) for n in N[:nsets]])
    Y = (_p * max(nsets, 1))(*[_ptr(t) for t in y[:nsets]])
    _check(_lib.kq_gemv_multi(fmt, nsets, P, Ns, K, _ptr(x), M, block_len, _ptr(signs), Y,
                              _stream(stream)), "kq_gemv_multi")


def kq_gemm(fmt: int, packed, N: int, K: int, x, x_dt: int, M: int, block_len: int,
            signs, y, workspace, ws_bytes: int, stream=None):
    _check(_lib.kq_gemm(fmt, _ptr(packed), N, K, _ptr(x), x_dt, M, block_len, _ptr(signs),
                        _ptr(y), _ptr(workspace), ws_bytes, _stream(stream)), "kq_gemm")


def kq_probe_read(buf, nbytes: int, layout: int, grid: int, block: int, sink, stream=None):
    _check(_lib.kq_probe_read(_ptr(buf), nbytes, layout, grid, block, _ptr(sink),
                              _stream(stream)), "kq_probe_read")


def kq_probe_mfma(iters: int, grid: int, block: int, sink, stream=None):
    _check(_lib.kq_probe_mfma(iters, grid, block, _ptr(sink), _stream(stream)), "kq_probe_mfma")


def kq_probe_gemv_loads(fmt: int, packed, N: int, K: int, x, M: int, block_len: int,
                        split_k: int, sink, stream=None):
    _check(_lib.kq_probe_gemv_loads(fmt, _ptr(packed), N, K, _ptr(x), M, block_len, split_k,
                                    _ptr(sink), _stream(stream)), "kq_probe_gemv_loads")


# ---- allocation conveniences (torch.empty + one call above) -----------------

def pack(fmt: int, W, stream=None):
    """Pack fp32 device weights W [N][K]; returns the planar uint8 buffer."""
    import torch
    N, K = W.shape
    out = torch.empty(kq_packed_bytes(fmt, N, K), dtype=torch.uint8, device=W.device)
    (kq_pack_pq2 if fmt == KQ_FMT_PQ2_0 else kq_pack_q8)(W, N, K, out, stream)
    return out


def transcode_ptq1(ptq1, N: int, K: int, stream=None):
    """PTQ1_0 blocks (uint8 device tensor) -> the planar PQ2_0 buffer."""
    import torch
    out = torch.empty(kq_packed_bytes(KQ_FMT_PQ2_0, N, K), dtype=torch.uint8, device=ptq1.device)
    kq_transcode_ptq1(ptq1, N, K, out, stream)
    return out


def unpack(fmt: int, packed, N: int, K: int, stream=None):
    import torch
    out = torch.empty((N, K), dtype=torch.float32, device=packed.device)
    kq_unpack(fmt, packed, N, K, out, stream)
    return out


def hadamard(x, block_len: int, signs=None, out_dtype=None, stream=None):
    import torch
    M, K = x.shape
    out = torch.empty((M, K), dtype=out_dtype or x.dtype, device=x.device)
    kq_hadamard_blocks(x, _dtype_code(x), out, _dtype_code(out), M, K, block_len, signs, stream)
    return out


def workspace(op: int, fmt: int, M: int, N: int, K: int, block_len: int, split_k: int = 0,
              device="cuda"):
    import torch
    n = kq_workspace_bytes(op, fmt, M, N, K, block_len, split_k)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device), n


def gemv(fmt: int, packed, N: int, K: int, x, block_len: int, signs=None, split_k: int = 0,
         ws=None, y=None, stream=None):
    import torch
    M = x.shape[0]
    if ws is None:
        ws, _ = workspace(0, fmt, M, N, K, block_len, split_k, device=x.device)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    kq_gemv(fmt, packed, N, K, x, M, block_len, signs, split_k, y, ws, ws.numel(), stream)
    return y


def gemv_multi(fmt: int, packed, N, K: int, x, block_len: int, signs=None, y=None,
               stream=None):
    """One launch over several weight sets sharing x; returns the list of y."""
    import torch
    M = x.shape[0]
    if y is None:
        y = [torch.empty((M, n), dtype=torch.float32, device=x.device) for n in N]
    kq_gemv_multi(fmt, len(N), packed, N, K, x, M, block_len, signs, y, stream)
    return y


def gemm(packed, N: int, K: int, x, block_len: int, signs=None, ws=None, y=None, stream=None,
         fmt: int = KQ_FMT_PQ2_0):
    import torch
    M = x.shape[0]
    if ws is None:
        ws, _ = workspace(1, fmt, M, N, K, block_len, 0, device=x.device)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    kq_gemm(fmt, packed, N, K, x, _dtype_code(x), M, block_len, signs, y, ws, ws.numel(), stream)
    return y
