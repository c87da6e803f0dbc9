"""GPU parity of kq_gemm (prefill GEMM on bf16 MFMA, PQ2_0 and Q8_0 weights,
token tiles of 256, 64 and 16) against the CPU oracle.  The oracle rotates the
bf16 input values exactly (binary64) and does not round x' or W to bf16; the
GPU's two bf16 roundings (x' after the rotation, the dequantized weights) are
what the tolerance absorbs:
|y_gpu - y_ref| <= 1e-2 * sum_k |deq(W)[n][k] x'[m][k]|.
Integer-exact cases (block_len 0, power-of-two scales, small integers, every
weight exact in bf16) must match with tolerance 0."""
import numpy as np
import pytest
import torch

import oracle
from gemm_kq_gemv_amd import inputs
from tests._gpu import assert_within_bound, check_guard, dev, gpu, guarded_empty, host, need_gpu

pytestmark = gpu
TOL = 1e-2
PQ2, Q8 = 1, 2


@pytest.fixture(autouse=True)
def _need():
    need_gpu()


def _kq():
    import gemm_kq_gemv_amd as kq
    return kq


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _oracle_sub(fmt, W_rows, x_rows_f32, block_len, signs=None):
    N, K = W_rows.shape
    if fmt == PQ2:
        Wd = oracle.unpack_pq2_aos(oracle.pack_pq2_aos(W_rows), N, K)
    else:
        Wd = oracle.unpack_q8_aos(oracle.pack_q8_aos(W_rows), N, K)
    xr = oracle.rotate(x_rows_f32.astype(np.float64), block_len, signs)
    return oracle.matmul(Wd, xr)


def _gemm(fmt, W, xbits, block_len, signs=None, packed=None, x_tensor=None):
    kq = _kq()
    N, K = W.shape
    M = xbits.shape[0] if x_tensor is None else x_tensor.shape[0]
    if packed is None:
        packed = kq.pack(fmt, dev(W))
    y, buf = guarded_empty((M, N))
    xt = _bf16_dev(xbits) if x_tensor is None else x_tensor
    kq.gemm(packed, N, K, xt, block_len, None if signs is None else dev(signs), y=y, fmt=fmt)
    out = host(y)
    check_guard(buf, M * N)
    return out


# token tiles: 16 (M <= 16), 64 (M <= 96), 256; ragged M, N and K tails
SHAPES = [(1, 1, 128), (5, 7, 256), (16, 64, 384), (17, 65, 512), (64, 200, 640),
          (96, 130, 1024), (97, 161, 384), (130, 200, 384), (256, 256, 1024), (300, 520, 5120)]


@pytest.mark.parametrize("fmt", [PQ2, Q8])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_small_full(fmt, M, N, K):
    W = inputs.weights(1500 + M, N, K)
    xb = inputs.to_bf16_bits(inputs.activations(1501 + M, M, K, offset=0.2))
    s = inputs.signs(1502, K)
    y = _gemm(fmt, W, xb, 128, s)
    y_ref, b = _oracle_sub(fmt, W, inputs.bf16_bits_to_f32(xb), 128, s)
    assert_within_bound(y, y_ref, b, TOL, f"gemm fmt {fmt} {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(3, 40, 96), (20, 33, 160), (70, 17, 32), (260, 48, 224)])
def test_gemm_q8_half_k_tiles(M, N, K):
    """Q8_0 K that ends in half a 64-wide K-tile (K % 64 == 32)."""
    W = inputs.weights(1520 + K, N, K)
    x = inputs.activations(1521 + K, M, K)
    y = _gemm(Q8, W, None, 32, x_tensor=dev(x))
    y_ref, b = _oracle_sub(Q8, W, x, 32)
    assert_within_bound(y, y_ref, b, TOL, f"q8 gemm {M}x{N}x{K}")


def test_gemm_c5_full_size_sampled():
    """M=2048, K=5120, N=10240 on the GPU; 48 token rows x 384 weight rows
    compared with the oracle (plus the four corners)."""
    M, N, K = 2048, 10240, 5120
    W = inputs.weights(1005, N, K)
    xb = inputs.to_bf16_bits(inputs.activations(2005, M, K))
    y = _gemm(PQ2, W, xb, 128)
    r = inputs.rng(9)
    ms = np.unique(np.concatenate([r.integers(0, M, 48), [0, M - 1]]))
    ns = np.unique(np.concatenate([r.integers(0, N, 384), [0, N - 1]]))
    y_ref, b = _oracle_sub(PQ2, W[ns], inputs.bf16_bits_to_f32(xb[ms]), 128)
    assert_within_bound(y[np.ix_(ms, ns)], y_ref, b, TOL, "C5 sampled")
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("M", [2048, 64, 16])
def test_gemm_q8_ffn_full_size_sampled(M):
    """Q8_0 prefill at the FFN shape K=5120, N=17408 (the Q8_0 GEMV's
    weights), for a prompt and for 64- and 16-token chunks; sampled rows."""
    N, K = 17408, 5120
    W = inputs.weights(1004, N, K)
    xb = inputs.to_bf16_bits(inputs.activations(2014 + M, M, K))
    y = _gemm(Q8, W, xb, 0)
    r = inputs.rng(19)
    ms = np.unique(np.concatenate([r.integers(0, M, min(M, 24)), [0, M - 1]]))
    ns = np.unique(np.concatenate([r.integers(0, N, 300), [0, N - 1]]))
    y_ref, b = _oracle_sub(Q8, W[ns], inputs.bf16_bits_to_f32(xb[ms]), 0)
    assert_within_bound(y[np.ix_(ms, ns)], y_ref, b, TOL, f"Q8 FFN M={M} sampled")


def test_gemm_f32_input():
    M, N, K = 64, 128, 1024
    W = inputs.weights(1600, N, K)
    x = inputs.activations(1601, M, K)
    for fmt in (PQ2, Q8):
        y = _gemm(fmt, W, None, 128, x_tensor=dev(x))
        y_ref, b = _oracle_sub(fmt, W, x, 128)
        assert_within_bound(y, y_ref, b, TOL, f"gemm f32 x fmt {fmt}")


@pytest.mark.parametrize("M,N,K", [(1, 3, 128), (16, 100, 384), (64, 131, 640), (129, 131, 640),
                                   (256, 512, 5120)])
def test_gemm_integer_exact_pq2(M, N, K):
    W = inputs.ternary_exact_weights(1700 + M, N, K, exp2=3)
    x = inputs.integer_activations(1701 + M, M, K, lim=64)
    xb = inputs.to_bf16_bits(x)
    assert np.array_equal(inputs.bf16_bits_to_f32(xb), x)
    y = _gemm(PQ2, W, xb, 0)
    y_ref, _ = _oracle_sub(PQ2, W, x, 0)
    assert np.array_equal(y.astype(np.float64), y_ref)


@pytest.mark.parametrize("M,N,K", [(1, 3, 32), (16, 100, 160), (64, 131, 640), (129, 45, 96),
                                   (256, 300, 5120)])
def test_gemm_integer_exact_q8(M, N, K):
    """Q8_0 weights q * 2^-7 (|q| <= 127: exact in bf16), integer activations
    |x| <= 8: every product and partial sum is exact in fp32."""
    W = inputs.int8_exact_weights(1710 + M, N, K, exp2=7)
    x = inputs.integer_activations(1711 + M, M, K, lim=8)
    xb = inputs.to_bf16_bits(x)
    y = _gemm(Q8, W, xb, 0)
    y_ref, _ = _oracle_sub(Q8, W, x, 0)
    assert np.array_equal(y.astype(np.float64), y_ref)


def test_gemm_deterministic():
    kq = _kq()
    M, N, K = 512, 1024, 5120
    W = inputs.weights(1800, N, K)
    xt = _bf16_dev(inputs.to_bf16_bits(inputs.activations(1801, M, K)))
    for fmt in (PQ2, Q8):
        packed = kq.pack(fmt, dev(W))
        a = host(kq.gemm(packed, N, K, xt, 128, fmt=fmt))
        b = host(kq.gemm(packed, N, K, xt, 128, fmt=fmt))
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
