"""The measurement instruments of include/kq_probe.h run through the C ABI on
the GPU: the streaming read and the GEMV's loads-only twin complete, write
nothing but the sink (which they leave alone unless their XOR hits its
sentinel), and the twin accepts exactly the plans kq_gemv accepts."""
import numpy as np
import pytest
import torch

from gemm_kq_gemv_amd import inputs
from tests._gpu import dev, gpu, host, need_gpu

pytestmark = gpu


@pytest.fixture(autouse=True)
def _need():
    need_gpu()


def _kq():
    import gemm_kq_gemv_amd as kq
    return kq


@pytest.mark.parametrize("layout,grid,block", [(0, 256, 256), (1, 37, 640), (0, 1, 64)])
def test_probe_read(layout, grid, block):
    kq = _kq()
    buf = torch.arange(1 << 18, dtype=torch.int32, device="cuda")
    sink = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    kq.kq_probe_read(buf, buf.numel() * 4 - 16 * 3, layout, grid, block, sink)
    assert np.all(host(sink) == -7)


@pytest.mark.parametrize("fmt,M,bl,S", [(1, 1, 128, 1), (1, 3, 1024, 0), (1, 1, 128, 4),
                                        (2, 1, 0, 1), (2, 4, 0, 1), (2, 8, 32, 0)])
def test_gemv_loads_twin(fmt, M, bl, S):
    kq = _kq()
    N, K = 1000, 5120
    packed = kq.pack(fmt, dev(inputs.weights(60, N, K)))
    x = dev(inputs.activations(61, M, K))
    sink = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    guard = packed.clone()
    kq.kq_probe_gemv_loads(fmt, packed, N, K, x, M, bl, S, sink)
    assert np.all(host(sink) == -7)
    assert torch.equal(packed, guard)
    with pytest.raises(kq.KQError) as e:
        kq.kq_probe_gemv_loads(fmt, packed, N, K, x, M, bl, K // (128 if fmt == 1 else 32) + 1, sink)
    assert e.value.name == "KQ_ESHAPE"


@pytest.mark.parametrize("iters,grid,block", [(1, 1, 64), (64, 256, 256), (8, 37, 1024)])
def test_probe_mfma(iters, grid, block):
    kq = _kq()
    sink = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    kq.kq_probe_mfma(iters, grid, block, sink)
    assert np.all(host(sink) == -7)
    with pytest.raises(kq.KQError) as e:
        kq.kq_probe_mfma(iters, grid, 96, sink)
    assert e.value.name == "KQ_ESHAPE"
