"""GPU parity of kq_gemm (PQ2_0 prefill GEMM on bf16 MFMA) against the CPU
oracle.  The oracle rotates the bf16 input values exactly (binary64) and does
not round x' or W to bf16; the GPU's two bf16 roundings (x' after the
rotation, (q-1)*d of the weights) are what the tolerance absorbs:
|y_gpu - y_ref| <= 1e-2 * sum_k |deq(W)[n][k] x'[m][k]|.
The integer-exact case (block_len 0, d = 2^-3, small integers) must match
with tolerance 0."""
import numpy as np
import pytest
import torch

import oracle
from gemm_kq_gemv_amd import inputs
from tests._gpu import assert_within_bound, check_guard, dev, gpu, guarded_empty, host, need_gpu

pytestmark = gpu
TOL = 1e-2


@pytest.fixture(autouse=True)
def _need():
    need_gpu()


def _kq():
    import gemm_kq_gemv_amd as kq
    return kq


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _oracle_sub(W_rows, x_rows_f32, block_len, signs=None):
    N, K = W_rows.shape
    Wd = oracle.unpack_pq2_aos(oracle.pack_pq2_aos(W_rows), N, K)
    xr = oracle.rotate(x_rows_f32.astype(np.float64), block_len, signs)
    return oracle.matmul(Wd, xr)


def _gemm(W, xbits, block_len, signs=None, packed=None, x_tensor=None):
    kq = _kq()
    N, K = W.shape
    M = xbits.shape[0] if x_tensor is None else x_tensor.shape[0]
    if packed is None:
        packed = kq.pack(1, dev(W))
    y, buf = guarded_empty((M, N))
    xt = _bf16_dev(xbits) if x_tensor is None else x_tensor
    kq.gemm(packed, N, K, xt, block_len, None if signs is None else dev(signs), y=y)
    out = host(y)
    check_guard(buf, M * N)
    return out


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (5, 7, 256), (130, 200, 384), (256, 256, 1024),
                                   (300, 520, 5120)])
def test_gemm_small_full(M, N, K):
    W = inputs.weights(1500 + M, N, K)
    xb = inputs.to_bf16_bits(inputs.activations(1501 + M, M, K, offset=0.2))
    s = inputs.signs(1502, K)
    y = _gemm(W, xb, 128, s)
    y_ref, b = _oracle_sub(W, inputs.bf16_bits_to_f32(xb), 128, s)
    assert_within_bound(y, y_ref, b, TOL, f"gemm {M}x{N}x{K}")


def test_gemm_c5_full_size_sampled():
    """M=2048, K=5120, N=10240 on the GPU; 48 token rows x 384 weight rows
    compared with the oracle (plus the four corners)."""
    kq = _kq()
    M, N, K = 2048, 10240, 5120
    W = inputs.weights(1005, N, K)
    xb = inputs.to_bf16_bits(inputs.activations(2005, M, K))
    y = _gemm(W, xb, 128)
    r = inputs.rng(9)
    ms = np.unique(np.concatenate([r.integers(0, M, 48), [0, M - 1]]))
    ns = np.unique(np.concatenate([r.integers(0, N, 384), [0, N - 1]]))
    y_ref, b = _oracle_sub(W[ns], inputs.bf16_bits_to_f32(xb[ms]), 128)
    assert_within_bound(y[np.ix_(ms, ns)], y_ref, b, TOL, "C5 sampled")
    assert np.all(np.isfinite(y))


def test_gemm_f32_input():
    M, N, K = 64, 128, 1024
    W = inputs.weights(1600, N, K)
    x = inputs.activations(1601, M, K)
    y = _gemm(W, None, 128, x_tensor=dev(x))
    y_ref, b = _oracle_sub(W, x, 128)
    assert_within_bound(y, y_ref, b, TOL, "gemm f32 x")


@pytest.mark.parametrize("M,N,K", [(1, 3, 128), (129, 131, 640), (256, 512, 5120)])
def test_gemm_integer_exact(M, N, K):
    W = inputs.ternary_exact_weights(1700 + M, N, K, exp2=3)
    x = inputs.integer_activations(1701 + M, M, K, lim=64)
    xb = inputs.to_bf16_bits(x)
    assert np.array_equal(inputs.bf16_bits_to_f32(xb), x)
    y = _gemm(W, xb, 0)
    y_ref, _ = _oracle_sub(W, x, 0)
    assert np.array_equal(y.astype(np.float64), y_ref)


def test_gemm_deterministic():
    kq = _kq()
    M, N, K = 512, 1024, 5120
    W = inputs.weights(1800, N, K)
    xt = _bf16_dev(inputs.to_bf16_bits(inputs.activations(1801, M, K)))
    packed = kq.pack(1, dev(W))
    a = host(kq.gemm(packed, N, K, xt, 128))
    b = host(kq.gemm(packed, N, K, xt, 128))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
