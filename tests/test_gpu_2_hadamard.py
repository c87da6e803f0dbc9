"""GPU parity of kq_hadamard_blocks against the oracle's explicit-matrix
rotation (Bonsai ternary g128 page sec. 4.1-4.2: sign flip, then
(1/sqrt(n)) H_n per n-block, Sylvester natural order).

Tolerance: the GPU adds fp32 values in log2(n) butterfly levels and scales
once, so each output is within (log2 n + 2) * 2^-24 * (sum_block |x|)/sqrt(n)
of the exact value; bf16 output adds half a bf16 ulp (2^-9 relative)."""
import math

import numpy as np
import pytest
import torch

import oracle
from gemm_kq_gemv_amd import inputs
from tests._gpu import dev, gpu, host, need_gpu

pytestmark = gpu


@pytest.fixture(autouse=True)
def _need():
    need_gpu()


def _kq():
    import gemm_kq_gemv_amd as kq
    return kq


def _bound(x, n):
    M, K = x.shape
    if n == 1:
        return np.zeros_like(x)     # sign flip only: exact
    blk = np.abs(x).reshape(M, K // n, n).sum(axis=2) / math.sqrt(n)
    return np.repeat(blk, n, axis=1) * (math.log2(n) + 2) * 2.0 ** -24


@pytest.mark.parametrize("n", [1, 2, 16, 32, 128, 1024])
@pytest.mark.parametrize("M,K", [(1, 1024), (3, 5120), (2, 17408)])
@pytest.mark.parametrize("with_signs", [False, True])
def test_hadamard_f32(n, M, K, with_signs):
    kq = _kq()
    x = inputs.activations(300 + n, M, K, offset=0.3)
    s = inputs.signs(301, K) if with_signs else None
    ref = oracle.rotate(x.astype(np.float64), n, s)
    got = host(kq.hadamard(dev(x), n, None if s is None else dev(s)))
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(err <= _bound(x.astype(np.float64), n) + 1e-30)


@pytest.mark.parametrize("n", [16, 128])
def test_hadamard_bf16_in_out(n):
    kq = _kq()
    M, K = 64, 5120
    xb = inputs.to_bf16_bits(inputs.activations(310, M, K))
    xf = inputs.bf16_bits_to_f32(xb)
    s = inputs.signs(311, K)
    ref = oracle.rotate(xf.astype(np.float64), n, s)
    xt = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    got = kq.hadamard(xt, n, dev(s), out_dtype=torch.bfloat16)
    gotf = host(got.float())
    err = np.abs(gotf.astype(np.float64) - ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(ref) + _bound(xf.astype(np.float64), n) + 1e-30)
    # f32 output from bf16 input
    got32 = host(kq.hadamard(xt, n, dev(s), out_dtype=torch.float32))
    assert np.all(np.abs(got32 - ref) <= _bound(xf.astype(np.float64), n) + 1e-30)


def test_hadamard_is_an_involution_without_signs():
    kq = _kq()
    x = inputs.activations(320, 4, 2048)
    t = dev(x)
    back = host(kq.hadamard(kq.hadamard(t, 256), 256))
    assert np.allclose(back, x, rtol=0, atol=1e-5)
