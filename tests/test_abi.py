"""Host-side checks of the C ABI: the library loads, exports every symbol that
include/kq.h declares, sizes its buffers as documented, and rejects every
out-of-contract call before any launch (no GPU needed: validation runs before
the HIP runtime is touched).  The rejected calls use fake addresses, so these
tests skip where a GPU is visible -- a validation bug must never turn into a
launch on a bogus pointer."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kq.h")


def _lib():
    import gemm_kq_gemv_amd as kq
    return kq


def _declared(header):
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|size_t|kq_status)\s*(kq_\w+)\s*\(",
                                 text, re.M)))


def test_exports_match_header():
    kq = _lib()
    declared = _declared(HEADER)
    assert declared == sorted(kq.EXPORTS)
    probes = _declared(os.path.join(ROOT, "include", "kq_probe.h"))
    assert probes == sorted(kq.PROBE_EXPORTS)
    cdll = C.CDLL(kq.LIB_PATH)
    for name in declared + probes:
        assert hasattr(cdll, name), name
    # every header under include/ is covered
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["kq.h", "kq_probe.h"]


def test_status_strings():
    kq = _lib()
    for s in range(7):
        assert kq.kq_status_string(s).startswith("KQ_")
    assert kq.kq_status_string(99) == "unknown kq_status"


def test_packed_bytes_layout(oracle_lib):
    kq = _lib()
    import oracle
    for fmt, g in ((1, 128), (2, 32)):
        for N, K in ((1, g), (3, 4 * g), (10240, 5120), (248320, 5120), (17408, 5120)):
            assert kq.kq_packed_bytes(fmt, N, K) == oracle.planar_bytes(fmt, N, K)
    assert kq.kq_packed_bytes(1, 10240, 5120) == 13926400   # 1280 B codes + 80 B scales per row
    assert kq.kq_packed_bytes(1, 10, 100) == 0
    assert kq.kq_packed_bytes(2, 0, 64) == 0
    assert kq.kq_packed_bytes(3, 10, 128) == 0


def test_workspace_sizes():
    kq = _lib()
    # the rotation runs in the GEMV prologue: no workspace without split-K
    assert kq.kq_workspace_bytes(0, 1, 1, 10240, 5120, 128, 1) == 0
    assert kq.kq_workspace_bytes(0, 1, 1, 10240, 5120, 128, 0) == 0
    # split-K: S*M*N fp32 partials
    assert kq.kq_workspace_bytes(0, 1, 1, 248320, 5120, 128, 2) == 2 * 248320 * 4
    # K-slices hold whole rotation blocks (n = 1024: 5 blocks over 3 slices):
    # still only the partials
    assert kq.kq_workspace_bytes(0, 1, 1, 10240, 5120, 1024, 3) == 3 * 10240 * 4
    # more slices than rotation blocks: no plan
    assert kq.kq_workspace_bytes(0, 1, 1, 10240, 5120, 1024, 6) == 0
    assert kq.kq_workspace_bytes(1, 1, 2048, 10240, 5120, 128, 0) == 2048 * 5120 * 2
    # a 16-token chunk splits K in 6 slices of 14 K-tiles: x' then the partials
    assert kq.kq_workspace_bytes(1, 1, 16, 10240, 5120, 128, 0) == 16 * 5120 * 2 + 6 * 16 * 10240 * 4
    assert kq.kq_workspace_bytes(0, 1, 9, 64, 128, 0, 0) == 0   # M > 8
    assert kq.kq_workspace_bytes(0, 1, 1, 64, 100, 0, 0) == 0   # bad K


FAKE = 1 << 30          # 16-byte aligned fake device address (never dereferenced)
MISALIGNED = FAKE + 4


@pytest.fixture
def nogpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only validation test (fake addresses); runs where no GPU is visible")


def _status(fn, *args):
    kq = _lib()
    try:
        fn(*args)
    except kq.KQError as e:
        return e.name
    return "KQ_OK"


@pytest.mark.usefixtures("nogpu")
def test_pack_rejections():
    kq = _lib()
    assert _status(kq.kq_pack_pq2, None, 4, 128, FAKE, 0) == "KQ_EINVAL"
    assert _status(kq.kq_pack_pq2, FAKE, 4, 128, None, 0) == "KQ_EINVAL"
    assert _status(kq.kq_pack_pq2, FAKE, -1, 128, FAKE, 0) == "KQ_EINVAL"
    assert _status(kq.kq_pack_pq2, FAKE, 0, 128, FAKE, 0) == "KQ_ESHAPE"
    assert _status(kq.kq_pack_pq2, FAKE, 4, 96, FAKE, 0) == "KQ_ESHAPE"
    assert _status(kq.kq_pack_pq2, FAKE, 4, 64, FAKE, 0) == "KQ_ESHAPE"
    assert _status(kq.kq_pack_pq2, MISALIGNED, 4, 128, FAKE, 0) == "KQ_EALIGN"
    assert _status(kq.kq_pack_q8, FAKE, 4, 48, FAKE, 0) == "KQ_ESHAPE"
    assert _status(kq.kq_pack_q8, FAKE, 4, 32, MISALIGNED, 0) == "KQ_EALIGN"
    assert _status(kq.kq_transcode_ptq1, None, 4, 128, FAKE, 0) == "KQ_EINVAL"
    assert _status(kq.kq_transcode_ptq1, FAKE, 4, 96, FAKE, 0) == "KQ_ESHAPE"
    assert _status(kq.kq_transcode_ptq1, FAKE, 0, 128, FAKE, 0) == "KQ_ESHAPE"
    assert _status(kq.kq_transcode_ptq1, FAKE, 4, 128, MISALIGNED, 0) == "KQ_EALIGN"
    assert _status(kq.kq_unpack, 7, FAKE, 4, 128, FAKE, 0) == "KQ_EINVAL"
    assert _status(kq.kq_unpack, 1, FAKE, 4, 160, FAKE, 0) == "KQ_ESHAPE"


@pytest.mark.usefixtures("nogpu")
def test_hadamard_rejections():
    kq = _lib()
    h = kq.kq_hadamard_blocks
    assert _status(h, None, 0, FAKE, 0, 1, 128, 128, None, 0) == "KQ_EINVAL"
    assert _status(h, FAKE, 2, FAKE, 0, 1, 128, 128, None, 0) == "KQ_EINVAL"
    assert _status(h, FAKE, 0, FAKE, 0, 1, 128, 96, None, 0) == "KQ_ESHAPE"      # not 2^i
    assert _status(h, FAKE, 0, FAKE, 0, 1, 128, 2048, None, 0) == "KQ_ESHAPE"    # > 1024
    assert _status(h, FAKE, 0, FAKE, 0, 1, 128, 0, None, 0) == "KQ_ESHAPE"
    assert _status(h, FAKE, 0, FAKE, 0, 1, 136, 8, None, 0) == "KQ_ESHAPE"       # K % 16
    assert _status(h, FAKE, 0, FAKE, 0, 1, 96, 64, None, 0) == "KQ_ESHAPE"       # n !| K
    assert _status(h, FAKE, 0, FAKE, 0, 0, 128, 128, None, 0) == "KQ_ESHAPE"
    assert _status(h, FAKE, 0, FAKE, 0, 1, 128, 128, MISALIGNED, 0) == "KQ_EALIGN"


@pytest.mark.usefixtures("nogpu")
def test_gemv_rejections():
    kq = _lib()
    g = kq.kq_gemv
    ws = 1 << 20
    assert _status(g, 3, FAKE, 64, 128, FAKE, 1, 128, None, 0, FAKE, FAKE, ws, 0) == "KQ_EINVAL"
    assert _status(g, 1, None, 64, 128, FAKE, 1, 128, None, 0, FAKE, FAKE, ws, 0) == "KQ_EINVAL"
    assert _status(g, 1, FAKE, 64, 128, FAKE, 9, 128, None, 0, FAKE, FAKE, ws, 0) == "KQ_ESHAPE"
    assert _status(g, 1, FAKE, 64, 128, FAKE, 0, 128, None, 0, FAKE, FAKE, ws, 0) == "KQ_ESHAPE"
    assert _status(g, 1, FAKE, 64, 192, FAKE, 1, 128, None, 0, FAKE, FAKE, ws, 0) == "KQ_ESHAPE"
    assert _status(g, 1, FAKE, 64, 384, FAKE, 1, 256, None, 0, FAKE, FAKE, ws, 0) == "KQ_ESHAPE"
    assert _status(g, 1, FAKE, 64, 256, FAKE, 1, 128, None, 3, FAKE, FAKE, ws, 0) == "KQ_ESHAPE"
    assert _status(g, 1, FAKE, 64, 256, FAKE, 1, 128, None, -1, FAKE, FAKE, ws, 0) == "KQ_ESHAPE"
    assert _status(g, 1, FAKE, 64, 256, FAKE, 1, 128, None, 0, MISALIGNED, FAKE, ws, 0) == "KQ_EALIGN"
    # split-K needs its partial buffer
    need = kq.kq_workspace_bytes(0, 1, 1, 64, 256, 0, 2)
    assert need == 2 * 64 * 4                  # S*M*N*4 partials
    assert _status(g, 1, FAKE, 64, 256, FAKE, 1, 0, None, 2, FAKE, None, 0, 0) == "KQ_EWORKSPACE"
    assert _status(g, 1, FAKE, 64, 256, FAKE, 1, 0, None, 2, FAKE, FAKE, need - 4, 0) == "KQ_EWORKSPACE"
    # slices hold whole rotation blocks: 1024-blocks over 3 slices need only
    # the partials; more slices than blocks is a valid request with no plan
    need = kq.kq_workspace_bytes(0, 1, 1, 64, 5120, 1024, 3)
    assert need == 3 * 64 * 4
    assert _status(g, 1, FAKE, 64, 5120, FAKE, 1, 1024, None, 3, FAKE, FAKE, need - 4, 0) == "KQ_EWORKSPACE"
    assert _status(g, 1, FAKE, 64, 5120, FAKE, 1, 1024, None, 6, FAKE, FAKE, ws, 0) == "KQ_EUNSUPPORTED"


@pytest.mark.usefixtures("nogpu")
def test_gemv_noalloc_rejections():
    kq = _lib()
    g = kq.kq_gemv_noalloc
    assert _status(g, 3, FAKE, 64, 128, FAKE, 1, 128, None, 0, FAKE, 0) == "KQ_EINVAL"
    assert _status(g, 1, FAKE, 64, 128, FAKE, 9, 128, None, 0, FAKE, 0) == "KQ_ESHAPE"
    assert _status(g, 1, FAKE, 64, 256, FAKE, 1, 128, None, 3, FAKE, 0) == "KQ_ESHAPE"
    assert _status(g, 1, FAKE, 64, 256, FAKE, 1, 128, None, 0, MISALIGNED, 0) == "KQ_EALIGN"
    assert _status(g, 1, FAKE, 64, 5120, FAKE, 1, 1024, None, 6, FAKE, 0) == "KQ_EUNSUPPORTED"
    # partials beyond the 8 MiB scratch array: 2 x 8 x 140000 x 4 bytes
    assert _status(g, 1, FAKE, 140000, 256, FAKE, 8, 0, None, 2, FAKE, 0) == "KQ_EWORKSPACE"


@pytest.mark.usefixtures("nogpu")
def test_gemm_rejections():
    kq = _lib()
    g = kq.kq_gemm
    ws = 1 << 20
    assert _status(g, 3, FAKE, 64, 128, FAKE, 1, 4, 128, None, FAKE, FAKE, ws, 0) == "KQ_EINVAL"
    assert _status(g, 2, FAKE, 64, 48, FAKE, 1, 4, 0, None, FAKE, FAKE, ws, 0) == "KQ_ESHAPE"
    assert _status(g, 1, FAKE, 64, 128, FAKE, 5, 4, 128, None, FAKE, FAKE, ws, 0) == "KQ_EINVAL"
    assert _status(g, 1, FAKE, 64, 96, FAKE, 1, 4, 0, None, FAKE, FAKE, ws, 0) == "KQ_ESHAPE"
    assert _status(g, 1, FAKE, 64, 128, FAKE, 1, 0, 128, None, FAKE, FAKE, ws, 0) == "KQ_ESHAPE"
    assert _status(g, 1, FAKE, 64, 128, FAKE, 1, 4, 128, None, FAKE, None, 0, 0) == "KQ_EWORKSPACE"
    assert _status(g, 1, FAKE, 64, 128, FAKE, 0, 4, 0, None, FAKE, FAKE, 16, 0) == "KQ_EWORKSPACE"
    assert _status(g, 1, FAKE, 64, 128, FAKE, 1, 4, 128, None, MISALIGNED, FAKE, ws, 0) == "KQ_EALIGN"
    # 32-bit buffer ranges: K above 2^21, or more output tiles than an int holds
    assert _status(g, 1, FAKE, 64, (1 << 21) + 128, FAKE, 1, 4, 0, None, FAKE, FAKE, ws, 0) == "KQ_EUNSUPPORTED"
    assert _status(g, 1, FAKE, 1 << 32, 128, FAKE, 1, 1 << 32, 0, None, FAKE, FAKE, ws, 0) == "KQ_EUNSUPPORTED"


@pytest.mark.usefixtures("nogpu")
def test_probe_rejections():
    kq = _lib()
    r = kq.kq_probe_read
    assert _status(r, None, 1024, 0, 256, 256, FAKE, 0) == "KQ_EINVAL"
    assert _status(r, FAKE, 1024, 2, 256, 256, FAKE, 0) == "KQ_EINVAL"
    assert _status(r, FAKE, 1024, 0, 0, 256, FAKE, 0) == "KQ_ESHAPE"
    assert _status(r, FAKE, 1024, 0, 256, 96, FAKE, 0) == "KQ_ESHAPE"
    assert _status(r, FAKE, 1000, 0, 256, 256, FAKE, 0) == "KQ_ESHAPE"
    assert _status(r, MISALIGNED, 1024, 0, 256, 256, FAKE, 0) == "KQ_EALIGN"
    m = kq.kq_probe_mfma
    assert _status(m, 16, 256, 256, None, 0) == "KQ_EINVAL"
    assert _status(m, 0, 256, 256, FAKE, 0) == "KQ_ESHAPE"
    assert _status(m, (1 << 20) + 1, 256, 256, FAKE, 0) == "KQ_ESHAPE"
    assert _status(m, 16, 0, 256, FAKE, 0) == "KQ_ESHAPE"
    assert _status(m, 16, 256, 1088, FAKE, 0) == "KQ_ESHAPE"
    assert _status(m, 16, 256, 256, MISALIGNED, 0) == "KQ_EALIGN"
    t = kq.kq_probe_gemv_loads
    assert _status(t, 3, FAKE, 64, 128, FAKE, 1, 128, 0, FAKE, 0) == "KQ_EINVAL"
    assert _status(t, 1, FAKE, 64, 192, FAKE, 1, 128, 0, FAKE, 0) == "KQ_ESHAPE"
    assert _status(t, 1, FAKE, 64, 128, FAKE, 9, 128, 0, FAKE, 0) == "KQ_ESHAPE"
    assert _status(t, 1, FAKE, 64, 128, FAKE, 1, 128, 0, MISALIGNED, 0) == "KQ_EALIGN"
    assert _status(t, 1, FAKE, 64, 5120, FAKE, 1, 1024, 6, FAKE, 0) == "KQ_EUNSUPPORTED"


@pytest.mark.usefixtures("nogpu")
def test_gemv_multi_rejections():
    kq = _lib()
    g = kq.kq_gemv_multi
    two = [FAKE, FAKE]
    assert _status(g, 3, 2, two, [64, 64], 128, FAKE, 1, 128, None, two, 0) == "KQ_EINVAL"
    assert _status(g, 1, 2, [FAKE, None], [64, 64], 128, FAKE, 1, 128, None, two, 0) == "KQ_EINVAL"
    assert _status(g, 1, 2, two, [64, 64], 128, None, 1, 128, None, two, 0) == "KQ_EINVAL"
    assert _status(g, 1, 2, two, [64, 64], 128, FAKE, 1, 128, None, [FAKE, None], 0) == "KQ_EINVAL"
    assert _status(g, 1, 2, two, [64, -1], 128, FAKE, 1, 128, None, two, 0) == "KQ_EINVAL"
    assert _status(g, 1, 0, two, [64, 64], 128, FAKE, 1, 128, None, two, 0) == "KQ_ESHAPE"
    assert _status(g, 1, 5, [FAKE] * 5, [64] * 5, 128, FAKE, 1, 128, None, [FAKE] * 5, 0) == "KQ_ESHAPE"
    assert _status(g, 1, 2, two, [64, 0], 128, FAKE, 1, 128, None, two, 0) == "KQ_ESHAPE"
    assert _status(g, 1, 2, two, [64, 64], 192, FAKE, 1, 128, None, two, 0) == "KQ_ESHAPE"
    assert _status(g, 1, 2, two, [64, 64], 128, FAKE, 9, 128, None, two, 0) == "KQ_ESHAPE"
    assert _status(g, 1, 2, two, [64, 64], 384, FAKE, 1, 256, None, two, 0) == "KQ_ESHAPE"
    assert _status(g, 1, 2, [FAKE, MISALIGNED], [64, 64], 128, FAKE, 1, 128, None, two, 0) == "KQ_EALIGN"
    assert _status(g, 1, 2, two, [64, 64], 128, FAKE, 1, 128, None, [MISALIGNED, FAKE], 0) == "KQ_EALIGN"
    # one K slice must fit a workgroup: K = 2^20 PQ2_0 codes do not
    assert _status(g, 1, 2, two, [64, 64], 1 << 20, FAKE, 1, 128, None, two, 0) == "KQ_EUNSUPPORTED"
