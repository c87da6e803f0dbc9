"""gemm_kq_gemv_amd: quantized-weight GEMV / GEMM for AMD MI355X (gfx950).

PQ2_0 ternary (128 weights: fp16 scale + 2-bit codes) and Q8_0 (32 int8 +
fp16 scale) weights, an activation rotated by a blockwise orthonormal
Walsh-Hadamard transform, hand-written HIP kernels behind the C ABI of
include/kq.h.  The ctypes binding (same function names as the C entry points)
is loaded on first use, so ``gemm_kq_gemv_amd.inputs`` imports without the
built library.
"""

_BINDING_NAMES = (
    "kq_status_string", "kq_packed_bytes", "kq_pack_pq2", "kq_pack_q8", "kq_transcode_ptq1",
    "transcode_ptq1", "kq_unpack",
    "kq_hadamard_blocks", "kq_workspace_bytes", "kq_gemv", "kq_gemv_noalloc", "kq_gemv_multi", "kq_gemm", "KQError",
    "KQ_FMT_PQ2_0", "KQ_FMT_Q8_0", "KQ_F32", "KQ_BF16", "pack", "unpack", "hadamard",
    "workspace", "gemv", "gemv_multi", "gemm", "LIB_PATH", "EXPORTS", "MAX_SETS",
    "PROBE_EXPORTS", "kq_probe_read", "kq_probe_mfma", "kq_probe_gemv_loads",
)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
