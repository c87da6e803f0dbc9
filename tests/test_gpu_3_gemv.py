"""GPU parity of kq_gemv against the CPU oracle.

Acceptance (per output): |y_gpu - y_ref| <= 1e-3 * sum_k |deq(W)[n][k] x'[m][k]|
with y_ref and the bound from the oracle in binary64.  The oracle packs the
weights itself (from the same seeded fp32 W); the GPU path uses its own
packed bytes (bit-exactness of the two packers is tested separately).
Integer-exact cases (block_len 0, power-of-two scales, small integer
activations) must match with tolerance 0, including under split-K."""
import numpy as np
import pytest
import torch

import oracle
from gemm_kq_gemv_amd import inputs
from tests import _golden as G
from tests._gpu import assert_within_bound, check_guard, dev, gpu, guarded_empty, host, need_gpu

pytestmark = gpu
TOL = 1e-3


@pytest.fixture(autouse=True)
def _need():
    need_gpu()


def _kq():
    import gemm_kq_gemv_amd as kq
    return kq


def _oracle_ref(fmt, W, x, block_len, signs=None):
    N, K = W.shape
    aos = oracle.pack_pq2_aos(W) if fmt == 1 else oracle.pack_q8_aos(W)
    return oracle.gemv_aos(fmt, aos, N, K, x, block_len, signs)


def _run(fmt, W, x, block_len, signs=None, split_k=0, packed=None):
    kq = _kq()
    N, K = W.shape
    M = x.shape[0]
    if packed is None:
        packed = kq.pack(fmt, dev(W))
    y, buf = guarded_empty((M, N))
    kq.gemv(fmt, packed, N, K, dev(x), block_len, None if signs is None else dev(signs),
            split_k, y=y)
    out = host(y)
    check_guard(buf, M * N)
    return out


# ---- the configurations ------------------------------------------------------

def test_c1_pq2_k512_n1024():
    W = inputs.weights(1001, 1024, 512)
    x = inputs.activations(2001, 1, 512)
    y_ref, b = _oracle_ref(1, W, x, 128)
    assert_within_bound(_run(1, W, x, 128), y_ref, b, TOL, "C1")


def test_c2_pq2_k5120_n10240():
    W = inputs.weights(1002, 10240, 5120)
    x = inputs.activations(2002, 1, 5120)
    y_ref, b = _oracle_ref(1, W, x, 128)
    assert_within_bound(_run(1, W, x, 128), y_ref, b, TOL, "C2")


@pytest.fixture(scope="module")
def c3_inputs():
    kq = _kq()
    N, K = 248320, 5120
    W = inputs.weights(1003, N, K)
    Wd = dev(W)
    packed = kq.pack(1, Wd)
    del Wd
    torch.cuda.empty_cache()
    return W, packed


@pytest.mark.parametrize("split_k", [1, 2, 4, 0])
def test_c3_pq2_lm_head_full_size_sampled(split_k, c3_inputs):
    """N = 248320 on the GPU, checked on 1500 sampled rows (plus the ends)."""
    N, K = 248320, 5120
    W, packed = c3_inputs
    x = inputs.activations(2003, 1, K)
    y = _run(1, W, x, 128, split_k=split_k, packed=packed)
    rows = np.unique(np.concatenate([inputs.rng(5).integers(0, N, 1500), [0, 1, N - 2, N - 1]]))
    y_ref, b = _oracle_ref(1, W[rows], x, 128)
    assert_within_bound(y[:, rows], y_ref, b, TOL, f"C3 split {split_k}")
    # the GPU-packed bytes of the sampled rows are the oracle's
    want = oracle.aos_to_planar(1, oracle.pack_pq2_aos(W[rows]), len(rows), K)
    got = host(packed)
    assert np.array_equal(G.code_rows(got, N, K, 1)[rows], G.code_rows(want, len(rows), K, 1))
    assert np.array_equal(G.scale_bytes(got, N, K, 1)[0][rows], G.scale_bytes(want, len(rows), K, 1)[0])


@pytest.mark.parametrize("M", [1, 4, 8])
def test_c4_q8_k5120_n17408(M):
    W = inputs.weights(1004, 17408, 5120)
    x = inputs.activations(2004, M, 5120)
    y_ref, b = _oracle_ref(2, W, x, 0)
    assert_within_bound(_run(2, W, x, 0), y_ref, b, TOL, f"C4 M={M}")


# ---- coverage of shapes, M, split-K, signs -----------------------------------

@pytest.mark.parametrize("fmt", [1, 2])
@pytest.mark.parametrize("M", [1, 2, 3, 5, 6, 7, 8])
def test_all_m(fmt, M):
    N, K = 300, 2048
    W = inputs.weights(400 + M, N, K)
    x = inputs.activations(500 + M, M, K, offset=0.5)
    bl = 128 if fmt == 1 else 0
    y_ref, b = _oracle_ref(fmt, W, x, bl)
    assert_within_bound(_run(fmt, W, x, bl), y_ref, b, TOL, f"fmt {fmt} M {M}")


@pytest.mark.parametrize("fmt,N,K", [(1, 1, 128), (1, 5, 256), (1, 67, 384), (1, 129, 640),
                                     (1, 1000, 6144), (1, 33, 17408), (2, 1, 32), (2, 3, 96),
                                     (2, 71, 1056), (2, 257, 4096)])
def test_ragged_shapes(fmt, N, K):
    W = inputs.weights(600 + N, N, K)
    x = inputs.activations(601 + N, 2, K, offset=-0.25)
    bl = 128 if (fmt == 1 and K % 128 == 0) else 32
    s = inputs.signs(602, K)
    y_ref, b = _oracle_ref(fmt, W, x, bl, s)
    assert_within_bound(_run(fmt, W, x, bl, s), y_ref, b, TOL, f"{fmt} {N}x{K}")


@pytest.mark.parametrize("block_len", [0, 2, 8, 64, 128, 256, 512, 1024])
def test_block_lengths(block_len):
    N, K = 256, 5120
    W = inputs.weights(700, N, K)
    x = inputs.activations(701, 1, K)
    s = inputs.signs(702, K) if block_len in (0, 1024) else None
    y_ref, b = _oracle_ref(1, W, x, block_len, s)
    assert_within_bound(_run(1, W, x, block_len, s), y_ref, b, TOL, f"n={block_len}")


@pytest.mark.parametrize("N,K,split_k", [(1, 128, 1), (17, 640, 1), (17, 640, 2), (33, 2048, 1),
                                         (33, 2048, 2), (300, 5120, 1), (300, 5120, 2),
                                         (4097, 1152, 1), (4097, 1152, 2)])
def test_pq2_one_row_shapes(N, K, split_k):
    """PQ2_0, one activation row, at wave counts 1 to 10 and ragged row
    counts: the instance whose workgroups own at most three row blocks (its
    final sum reads zero-filled slots of absent waves) and the looping one."""
    W = inputs.weights(760 + N, N, K)
    x = inputs.activations(761 + N, 1, K, offset=0.2)
    y_ref, b = _oracle_ref(1, W, x, 128)
    assert_within_bound(_run(1, W, x, 128, split_k=split_k), y_ref, b, TOL,
                        f"N={N} K={K} S={split_k}")


@pytest.mark.parametrize("M", [2, 4, 5, 8])
@pytest.mark.parametrize("block_len", [512, 1024])
def test_block_lengths_many_rows(M, block_len):
    """PQ2_0 with several activation rows at the widest rotation blocks: the
    1024-block instances hold 16 elements per lane and load rows past the
    first inside the prologue; two operand tiles from five rows on."""
    N, K = 300, 5120
    W = inputs.weights(703 + M, N, K)
    x = inputs.activations(704 + M, M, K, offset=0.3)
    s = inputs.signs(705, K)
    y_ref, b = _oracle_ref(1, W, x, block_len, s)
    assert_within_bound(_run(1, W, x, block_len, s), y_ref, b, TOL, f"n={block_len} M={M}")
    assert_within_bound(_run(1, W, x, block_len, s, split_k=5), y_ref, b, TOL,
                        f"n={block_len} M={M} S=5")


# Activations shaped like an LLM's: a few outlier channels 10^3 - 10^4 times
# the typical magnitude, on top of a DC offset.  Inside the representation
# envelope kq.h states, so the 1e-3 bound must hold.
def _outlier_activations(seed, M, K):
    x = inputs.activations(seed, M, K, offset=0.75)
    r = inputs.rng(seed + 1)
    ch = r.choice(K, size=6, replace=False)
    mag = np.array([1e3, -2e3, 4e3, -1e4, 1e4, 3e3], np.float32)
    x[:, ch] = mag[None, :] * (1.0 + 0.1 * r.standard_normal((M, 6)).astype(np.float32))
    return x


@pytest.mark.parametrize("fmt,M,block_len", [(1, 1, 128), (1, 3, 128), (1, 8, 1024), (1, 1, 0),
                                             (2, 1, 0), (2, 4, 0), (2, 5, 0), (2, 8, 0),
                                             (2, 2, 128)])
def test_outlier_channels(fmt, M, block_len):
    N, K = 400, 5120
    W = inputs.weights(1900 + M, N, K)
    x = _outlier_activations(1910 + M, M, K)
    y_ref, b = _oracle_ref(fmt, W, x, block_len)
    assert_within_bound(_run(fmt, W, x, block_len), y_ref, b, TOL,
                        f"outliers fmt {fmt} M {M} n {block_len}")


@pytest.mark.parametrize("M", [1, 3])
@pytest.mark.parametrize("block_len", [128, 1024])
def test_q8_rotation_blocks(M, block_len):
    """Q8_0 with a rotation: one activation row (16-wave shape) and several
    (8-wave shape), blocks that stay inside a wave and blocks that span
    waves."""
    N, K = 200, 5120
    W = inputs.weights(710 + M, N, K)
    x = inputs.activations(711 + M, M, K)
    s = inputs.signs(712, K)
    y_ref, b = _oracle_ref(2, W, x, block_len, s)
    assert_within_bound(_run(2, W, x, block_len, s), y_ref, b, TOL, f"q8 n={block_len} M={M}")


@pytest.mark.parametrize("M,K,block_len", [(2, 5120, 2), (4, 5120, 16), (3, 1056, 16), (4, 1056, 0),
                                           (2, 96, 8)])
def test_q8_small_blocks_register_digits(M, K, block_len):
    """Q8_0, two to four rows, rotation blocks of at most 16 (stages in
    registers, digits made from registers, rows split over two thread
    groups), with signs; K = 1056 puts both groups' units in one wave."""
    N = 150
    W = inputs.weights(730 + M, N, K)
    x = inputs.activations(731 + M, M, K, offset=-0.4)
    s = inputs.signs(732, K)
    y_ref, b = _oracle_ref(2, W, x, block_len, s)
    assert_within_bound(_run(2, W, x, block_len, s), y_ref, b, TOL, f"q8 K={K} n={block_len} M={M}")
    assert_within_bound(_run(2, W, x, block_len, s, split_k=2), y_ref, b, TOL,
                        f"q8 K={K} n={block_len} M={M} S=2")


@pytest.mark.parametrize("M,block_len", [(1, 128), (3, 128), (1, 1024), (5, 1024)])
def test_code_3_is_a_zero_weight(M, block_len):
    """Code 3 is not a PQ2_0 value (the format maps codes 0, 1 and 2); the
    GEMV reads it as a zero weight.  A blob with random codes set to 3 gives
    the same bits as the same blob with code 1 there, and the oracle's
    product over the latter."""
    kq = _kq()
    N, K = 100, 2048
    W = inputs.weights(1900 + M, N, K)
    aos = oracle.pack_pq2_aos(W)
    blk = aos.reshape(-1, 34)
    assert not any(np.any(((blk[:, 2:] >> s_) & 3) == 3) for s_ in (0, 2, 4, 6))
    r = inputs.rng(1901 + M)
    nb = blk.shape[0]
    pick_b = r.integers(0, nb, 600)
    pick_byte = 2 + r.integers(0, 32, 600)
    pick_sh = 2 * r.integers(0, 4, 600)
    a3 = blk.copy()
    for b_, c_, s_ in zip(pick_b, pick_byte, pick_sh):
        a3[b_, c_] |= np.uint8(3 << s_)
    a1 = a3.copy()
    q = a1[:, 2:]
    for s_ in (0, 2, 4, 6):
        is3 = ((q >> s_) & 3) == 3
        q[is3] = (q[is3] & ~np.uint8(3 << s_)) | np.uint8(1 << s_)
    a3 = a3.reshape(-1)
    a1 = a1.reshape(-1)
    assert np.count_nonzero(a3 != a1) > 0
    x = inputs.activations(1902 + M, M, K)
    y3 = _run(1, W, x, block_len, packed=dev(oracle.aos_to_planar(1, a3, N, K)))
    y1 = _run(1, W, x, block_len, packed=dev(oracle.aos_to_planar(1, a1, N, K)))
    assert np.array_equal(y3.view(np.uint32), y1.view(np.uint32))
    y_ref, b = oracle.gemv_aos(1, a1, N, K, x, block_len, None)
    assert_within_bound(y3, y_ref, b, TOL, f"code 3, M={M}, block {block_len}")


@pytest.mark.parametrize("fmt", [1, 2])
@pytest.mark.parametrize("split_k", [1, 2, 3, 5, 40])
def test_split_k(fmt, split_k):
    N, K = 777, 5120
    W = inputs.weights(800, N, K)
    x = inputs.activations(801, 2, K)
    bl = 128 if fmt == 1 else 0
    y_ref, b = _oracle_ref(fmt, W, x, bl)
    assert_within_bound(_run(fmt, W, x, bl, split_k=split_k), y_ref, b, TOL, f"S={split_k}")


def test_deterministic_run_to_run():
    kq = _kq()
    N, K = 10240, 5120
    W = inputs.weights(900, N, K)
    x = dev(inputs.activations(901, 1, K))
    packed = kq.pack(1, dev(W))
    for split_k in (1, 4):
        a = host(kq.gemv(1, packed, N, K, x, 128, split_k=split_k))
        b = host(kq.gemv(1, packed, N, K, x, 128, split_k=split_k))
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ---- integer-exact, tolerance 0 ----------------------------------------------

@pytest.mark.parametrize("N,K,M,split_k", [(1, 128, 1, 1), (37, 384, 2, 1), (37, 384, 2, 3),
                                           (300, 5120, 1, 1), (300, 5120, 1, 3),
                                           (65, 17408, 3, 0), (65, 17408, 3, 7)])
def test_integer_exact_pq2(N, K, M, split_k):
    W = inputs.ternary_exact_weights(1100 + N, N, K, exp2=3)
    x = inputs.integer_activations(1101 + N, M, K, lim=64)
    y_ref, _ = _oracle_ref(1, W, x, 0)
    y = _run(1, W, x, 0, split_k=split_k)
    assert np.array_equal(y.astype(np.float64), y_ref)


@pytest.mark.parametrize("N,K,M,split_k", [(1, 32, 1, 1), (45, 160, 4, 1), (45, 160, 4, 2),
                                           (300, 5120, 8, 0), (300, 5120, 8, 8)])
def test_integer_exact_q8(N, K, M, split_k):
    W = inputs.int8_exact_weights(1200 + N, N, K, exp2=7)
    x = inputs.integer_activations(1201 + N, M, K, lim=8)
    y_ref, _ = _oracle_ref(2, W, x, 0)
    y = _run(2, W, x, 0, split_k=split_k)
    assert np.array_equal(y.astype(np.float64), y_ref)


def test_infeasible_split_is_rejected_without_writing():
    kq = _kq()
    N, K = 64, 5120
    W = inputs.weights(1250, N, K)
    packed = kq.pack(1, dev(W))
    x = dev(inputs.activations(1251, 8, K))
    ws, nws = kq.workspace(0, 1, 8, N, K, 0, 0)
    y, buf = guarded_empty((8, N))
    y.fill_(-1.0)
    for split_k, status in ((1, "KQ_EUNSUPPORTED"), (41, "KQ_ESHAPE")):
        with pytest.raises(kq.KQError) as e:
            kq.kq_gemv(1, packed, N, K, x, 8, 0, None, split_k, y, ws, nws)
        assert e.value.name == status
    assert np.all(host(y) == -1.0)
    check_guard(buf, 8 * N)


def test_all_plus_one_rows_closed_form():
    # every code 2 with d = 1 and no signs: y = sum_b sqrt(n) x[b n]
    N, K, n = 64, 1024, 128
    W = np.ones((N, K), np.float32)
    x = inputs.activations(1300, 1, K)
    y = _run(1, W, x, n)
    want = np.sqrt(n) * x[0, ::n].astype(np.float64).sum()
    bound = np.abs(oracle.rotate(x.astype(np.float64), n)).sum()   # sum_k |W x'| with W = 1
    assert np.all(np.abs(y[0] - want) <= TOL * bound)


# ---- several weight sets in one launch ----------------------------------------

def _multi(fmt, Ws, x, block_len, signs=None):
    """kq_gemv_multi over the sets of Ws (each packed on the GPU), outputs in
    guarded buffers; returns (outputs, packed buffers)."""
    kq = _kq()
    K = Ws[0].shape[1]
    M = x.shape[0]
    packed = [kq.pack(fmt, dev(W)) for W in Ws]
    outs = [guarded_empty((M, W.shape[0])) for W in Ws]
    kq.kq_gemv_multi(fmt, len(Ws), packed, [W.shape[0] for W in Ws], K, dev(x), M, block_len,
                     None if signs is None else dev(signs), [y for y, _ in outs])
    ys = [host(y) for y, _ in outs]
    for (y, buf), W in zip(outs, Ws):
        check_guard(buf, M * W.shape[0])
    return ys, packed


@pytest.mark.parametrize("fmt,M", [(1, 1), (1, 3), (1, 8), (2, 1), (2, 4), (2, 6)])
@pytest.mark.parametrize("Ns", [(300, 77), (1024, 16, 257), (640, 640, 48, 1)])
def test_multi_sets_match_single_calls(fmt, M, Ns):
    """Each set's output is the oracle's within the GEMV bound and bitwise the
    one-set call's (same plan, same fixed reduction order)."""
    kq = _kq()
    K = 2048
    Ws = [inputs.weights(1400 + 7 * i + len(Ns), n, K) for i, n in enumerate(Ns)]
    x = inputs.activations(1450 + M, M, K, offset=0.1)
    bl = 128 if fmt == 1 else 32
    s = inputs.signs(1460, K)
    ys, packed = _multi(fmt, Ws, x, bl, s)
    for i, (W, y, p) in enumerate(zip(Ws, ys, packed)):
        y_ref, b = _oracle_ref(fmt, W, x, bl, s)
        assert_within_bound(y, y_ref, b, TOL, f"set {i} of {Ns}")
        one = host(kq.gemv(fmt, p, W.shape[0], K, dev(x), bl, dev(s), split_k=1))
        assert np.array_equal(y.view(np.uint32), one.view(np.uint32)), f"set {i} differs from its own call"


@pytest.mark.parametrize("M", [1, 3, 8])
def test_multi_sets_block_1024(M):
    """Several PQ2_0 sets at the 1024-element rotation block (16 elements per
    lane in the prologue, the multi-set kernel instances)."""
    kq = _kq()
    # eight rows of 4 e5m2 terms at 5120 take more operand LDS than one
    # workgroup has (the call is rejected, see below); 3072 fits
    K = 5120 if M < 8 else 3072
    Ns = (300, 77, 520)
    Ws = [inputs.weights(1490 + 3 * i + M, n, K) for i, n in enumerate(Ns)]
    x = inputs.activations(1495 + M, M, K, offset=-0.2)
    s = inputs.signs(1496, K)
    ys, packed = _multi(1, Ws, x, 1024, s)
    for i, (W, y, p) in enumerate(zip(Ws, ys, packed)):
        y_ref, b = _oracle_ref(1, W, x, 1024, s)
        assert_within_bound(y, y_ref, b, TOL, f"n=1024 set {i} M {M}")
        one = host(kq.gemv(1, p, W.shape[0], K, dev(x), 1024, dev(s), split_k=1))
        assert np.array_equal(y.view(np.uint32), one.view(np.uint32)), f"set {i} differs from its own call"
    if M == 8:
        K2 = 5120
        p2 = [kq.pack(1, dev(inputs.weights(1499, 64, K2)))]
        y2, buf2 = guarded_empty((8, 64))
        y2.fill_(-1.0)
        with pytest.raises(kq.KQError) as e:
            kq.kq_gemv_multi(1, 1, p2, [64], K2, dev(inputs.activations(1498, 8, K2)), 8, 1024,
                             None, [y2])
        assert e.value.name == "KQ_EUNSUPPORTED"
        assert np.all(host(y2) == -1.0)
        check_guard(buf2, 8 * 64)


def test_multi_gate_up_full_size_sampled():
    """Two PQ2_0 sets of 17408 x 5120 (gate and up), one activation row:
    sampled rows against the oracle, every row bitwise against one-set calls."""
    kq = _kq()
    N, K = 17408, 5120
    Ws = [inputs.weights(1470 + i, N, K) for i in range(2)]
    x = inputs.activations(1480, 1, K)
    ys, packed = _multi(1, Ws, x, 128)
    rows = np.unique(np.concatenate([inputs.rng(11).integers(0, N, 400), [0, N - 1]]))
    for i, (W, y, p) in enumerate(zip(Ws, ys, packed)):
        y_ref, b = _oracle_ref(1, W[rows], x, 128)
        assert_within_bound(y[:, rows], y_ref, b, TOL, f"gate/up set {i}")
        one = host(kq.gemv(1, p, N, K, dev(x), 128, split_k=1))
        assert np.array_equal(y.view(np.uint32), one.view(np.uint32))
