"""GPU parity: kq_pack_pq2 / kq_pack_q8 / kq_unpack must reproduce the CPU
oracle's bytes and values bit for bit (Bonsai ternary g128 page sec. 3.1;
Kipp architecture page "Weight quantization")."""
import numpy as np
import pytest

import oracle
from gemm_kq_gemv_amd import inputs
from tests import _golden as G
from tests._gpu import check_guard, dev, gpu, host, need_gpu

pytestmark = gpu


@pytest.fixture(autouse=True)
def _need():
    need_gpu()


def _kq():
    import gemm_kq_gemv_amd as kq
    return kq


def special_weights(seed, N, K, group):
    """Gaussian rows with edge-case groups mixed in: all-zero groups, groups
    whose scale is an fp16 subnormal or rounds to zero, large groups, exact
    ties at half a step, a DC offset."""
    W = inputs.weights(seed, N, K)
    r = inputs.rng(seed + 1)
    ng = N * K // group
    Wg = W.reshape(ng, group)
    pick = r.permutation(ng)
    k = max(1, ng // 16)
    Wg[pick[0:k]] = 0.0
    Wg[pick[k:2 * k]] *= np.float32(3e-6)     # fp16 subnormal scale
    Wg[pick[2 * k:3 * k]] *= np.float32(2e-8)  # scale rounds to 0 in fp16
    Wg[pick[3 * k:4 * k]] *= np.float32(900.0)
    Wg[pick[4 * k:5 * k]] += np.float32(0.75)  # DC offset
    ties = pick[5 * k:6 * k]
    Wg[ties] = 0.0
    if group == 128:
        Wg[ties, 0] = 2.0                       # d = 2: r = +-0.5 ties at +-1
        Wg[ties, 1:9] = np.array([1, -1, 1, -1, 0.5, -0.5, 3 * 0.5, -1.5], np.float32)
    else:
        Wg[ties, 0] = 127.0                     # d = 1: ties at k + 0.5
        Wg[ties, 1:9] = np.array([2.5, -2.5, 0.5, -0.5, 126.5, -126.5, 3.5, -7.5], np.float32)
    return W


def oracle_planar(fmt, W):
    N, K = W.shape
    aos = oracle.pack_pq2_aos(W) if fmt == 1 else oracle.pack_q8_aos(W)
    return oracle.aos_to_planar(fmt, aos, N, K)


@pytest.mark.parametrize("fmt", [1, 2])
@pytest.mark.parametrize("N,K", [(1, 128), (7, 384), (37, 1152), (64, 5120), (3, 17408)])
def test_pack_bit_exact(fmt, N, K):
    import torch
    kq = _kq()
    W = special_weights(100 + N, N, K, 128 if fmt == 1 else 32)
    want = oracle_planar(fmt, W)
    nbytes = kq.kq_packed_bytes(fmt, N, K)
    assert nbytes == want.size
    buf = torch.full((nbytes + 512,), 0xA5, dtype=torch.uint8, device="cuda")
    (kq.kq_pack_pq2 if fmt == 1 else kq.kq_pack_q8)(dev(W), N, K, buf)
    got = host(buf)
    # whole 16-row code tiles (padding rows written as zeros); the bytes
    # between the code plane and the 256-aligned d plane are not written
    qs_bytes = (N + 15) // 16 * 16 * (K // 4 if fmt == 1 else K)
    d_off = G.d_offset(N, K, fmt)
    assert np.array_equal(got[:qs_bytes], want[:qs_bytes])
    assert np.array_equal(got[d_off:nbytes], want[d_off:])
    assert np.all(got[nbytes:] == 0xA5), "write past the packed buffer"


def test_pack_golden_fixtures():
    kq = _kq()
    g = G.load("pq2_quantize_blocks.txt")
    W = np.stack([G.sparse_block(g[f"block{c}_w"], 128) for c in "ABCD"])
    packed = kq.pack(1, dev(W))
    got = host(packed)
    rows = G.code_rows(got, 4, 128, 1)
    sc, pad = G.scale_bytes(got, 4, 128, 1)
    assert not pad.any()
    for i, c in enumerate("ABCD"):
        assert np.array_equal(rows[i], G.hex_bytes(g[f"block{c}_qs"])), c
        d = int(sc[i, 0, 0]) | (int(sc[i, 0, 1]) << 8)
        assert d == int(g[f"block{c}_d16"], 16), c
    g8 = G.load("q8_quantize_block.txt")
    W8 = np.stack([G.sparse_block(g8["w"], 32), G.sparse_block(g8["b2_w"], 32)])
    got8 = host(kq.pack(2, dev(W8)))
    rows8 = G.code_rows(got8, 2, 32, 2)
    sc8, pad8 = G.scale_bytes(got8, 2, 32, 2)
    assert not pad8.any()
    assert np.array_equal(rows8[0].view(np.int8).astype(np.int64), G.ints(g8["q"]))
    assert np.array_equal(rows8[1].view(np.int8).astype(np.int64), G.ints(g8["b2_q"]))
    assert int(sc8[0, 0, 0]) | (int(sc8[0, 0, 1]) << 8) == int(g8["d16"], 16)
    assert int(sc8[1, 0, 0]) | (int(sc8[1, 0, 1]) << 8) == int(g8["b2_d16"], 16)


@pytest.mark.parametrize("fmt", [1, 2])
@pytest.mark.parametrize("N,K", [(5, 256), (33, 1024)])
def test_unpack_random_blobs_bit_exact(fmt, N, K):
    import torch
    kq = _kq()
    g = 128 if fmt == 1 else 32
    aos = inputs.random_bytes(7 + N, N * (K // g) * 34)
    aos[1::34] &= 0x3F           # finite fp16 scales (sign kept)
    planar = oracle.aos_to_planar(fmt, aos, N, K)
    want = oracle.unpack_aos(fmt, aos, N, K).astype(np.float32)
    out = torch.full((N * K + 256,), 7.0, dtype=torch.float32, device="cuda")
    kq.kq_unpack(fmt, dev(planar), N, K, out)
    got = host(out)
    assert np.array_equal(got[:N * K].reshape(N, K).view(np.uint32), want.view(np.uint32))
    assert np.all(got[N * K:] == 7.0)


def test_pack_unpack_roundtrip_c2_shape():
    kq = _kq()
    N, K = 10240, 5120
    W = inputs.weights(1002, N, K)
    packed = kq.pack(1, dev(W))
    Wd = host(kq.unpack(1, packed, N, K))
    # quantizer invariant: nearest ternary level, |w - deq| <= d/2
    sc, pad = G.scale_bytes(host(packed), N, K, 1)
    assert not pad.any()
    dpl = np.ascontiguousarray(sc).view("<f2").astype(np.float32).reshape(N, K // 128)
    dF = np.repeat(dpl, 128, axis=1)
    assert np.all(np.abs(W - Wd) <= 0.5 * dF * (1 + 2 ** -20))
    # and repacking the dequantized weights reproduces the bytes
    again = kq.pack(1, dev(Wd))
    assert np.array_equal(host(again), host(packed))


# ---- PTQ1_0 -> PQ2_0 load-time transcode (Bonsai page, sec. 3.2) ----------

@pytest.mark.parametrize("N,K", [(1, 128), (17, 640), (37, 5120), (100, 17408)])
def test_transcode_ptq1_bit_exact(N, K):
    """PTQ1_0 blocks made by the oracle from quantized weights: the GPU's
    planar PQ2_0 bytes equal the oracle's transcode laid out planar, and equal
    what kq_pack_pq2 writes for the same weights."""
    import torch
    kq = _kq()
    W = special_weights(2100 + N, N, K, 128)
    aos = oracle.pack_pq2_aos(W)
    p1 = oracle.pq2_to_ptq1_aos(aos, N, K)
    want = oracle.aos_to_planar(1, oracle.ptq1_to_pq2_aos(p1, N, K), N, K)
    nb = kq.kq_packed_bytes(1, N, K)
    buf = torch.full((nb + 1024,), 0xA5, dtype=torch.uint8, device="cuda")
    kq.kq_transcode_ptq1(dev(p1), N, K, buf)
    got = host(buf)
    assert np.array_equal(got[:nb], want)
    assert np.all(got[nb:] == 0xA5), "write past the end of the packed buffer"
    assert np.array_equal(got[:nb], host(kq.pack(1, dev(W))))


@pytest.mark.parametrize("N,K", [(3, 256), (33, 1152)])
def test_transcode_ptq1_every_byte_value(N, K):
    """Arbitrary blobs (every byte value at every trit position) decode as the
    oracle decodes them."""
    kq = _kq()
    p1 = inputs.random_bytes(2200 + N, N * (K // 128) * 28)
    want = oracle.aos_to_planar(1, oracle.ptq1_to_pq2_aos(p1, N, K), N, K)
    got = host(kq.transcode_ptq1(dev(p1), N, K))
    assert np.array_equal(got, want)
    # the decoded values are the oracle's PTQ1_0 reading (random scale bytes
    # include NaN and infinite halves: NaN compares equal to NaN here)
    deq = host(kq.unpack(1, kq.transcode_ptq1(dev(p1), N, K), N, K))
    assert np.array_equal(deq.astype(np.float64), oracle.unpack_ptq1_aos(p1, N, K), equal_nan=True)


def test_transcode_ptq1_gemv_matches_pq2():
    """A GEMV over transcoded PTQ1_0 weights is bitwise the GEMV over the same
    weights packed as PQ2_0 (the buffers are identical)."""
    kq = _kq()
    N, K = 10240, 5120
    W = inputs.weights(1002, N, K)
    p1 = oracle.pq2_to_ptq1_aos(oracle.pack_pq2_aos(W), N, K)
    x = dev(inputs.activations(2002, 1, K))
    a = host(kq.gemv(1, kq.transcode_ptq1(dev(p1), N, K), N, K, x, 128))
    b = host(kq.gemv(1, kq.pack(1, dev(W)), N, K, x, 128))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
