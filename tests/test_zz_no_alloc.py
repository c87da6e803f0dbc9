"""kq_gemv_noalloc: kq_gemv without a workspace argument, its split-K partials
in the library's static per-GPU scratch array.  Through the C ABI on the GPU:
two calls in a row (the second with a smaller input) must give bitwise the
outputs of kq_gemv with a caller workspace, and a plan larger than the array
must be rejected before any launch."""
import numpy as np
import pytest
import torch

from gemm_kq_gemv_amd import inputs
from tests._gpu import check_guard, dev, gpu, guarded_empty, host, need_gpu

pytestmark = gpu


@pytest.fixture(autouse=True)
def _need():
    need_gpu()


def _kq():
    import gemm_kq_gemv_amd as kq
    return kq


def _both(kq, fmt, packed, N, K, x, M, bl, S):
    ws, nws = kq.workspace(0, fmt, M, N, K, bl, S)
    y_ws = torch.empty((M, N), device="cuda")
    kq.kq_gemv(fmt, packed, N, K, x, M, bl, None, S, y_ws, ws, nws)
    y_na, buf = guarded_empty((M, N))
    kq.kq_gemv_noalloc(fmt, packed, N, K, x, M, bl, None, S, y_na)
    a, b = host(y_ws), host(y_na)
    check_guard(buf, M * N)
    return a, b


def test_noalloc_two_calls_match_workspace_calls():
    kq = _kq()
    # first call: the 248320-row head split in four (3.97 MB of partials)
    N, K = 248320, 5120
    packed = kq.pack(1, dev(inputs.weights(1003, N, K)))
    x = dev(inputs.activations(2003, 1, K))
    a, b = _both(kq, 1, packed, N, K, x, 1, 128, 4)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    del packed
    torch.cuda.empty_cache()
    # second call, smaller: Q8_0, three rows, five slices
    N2, K2 = 1000, 5120
    p2 = kq.pack(2, dev(inputs.weights(3001, N2, K2)))
    x2 = dev(inputs.activations(3002, 3, K2))
    a, b = _both(kq, 2, p2, N2, K2, x2, 3, 0, 5)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # one pass over K: no scratch at all
    a, b = _both(kq, 2, p2, N2, K2, x2, 3, 0, 1)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_noalloc_rejects_plans_larger_than_scratch():
    kq = _kq()
    N, K, M = 140000, 256, 8          # partials 2 x 8 x 140000 x 4 B > 8 MiB at S = 2
    packed = kq.pack(1, dev(inputs.weights(3003, N, K)))
    x = dev(inputs.activations(3004, M, K))
    y, buf = guarded_empty((M, N))
    y.fill_(-1.0)
    with pytest.raises(kq.KQError) as e:
        kq.kq_gemv_noalloc(1, packed, N, K, x, M, 0, None, 2, y)
    assert e.value.name == "KQ_EWORKSPACE"
    assert np.all(host(y) == -1.0)
    check_guard(buf, M * N)
