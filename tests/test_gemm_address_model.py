"""Address model of the prefill GEMM's global loads (CPU only).

The kernel reads x' rows, weight codes and scales through raw buffer loads
whose hardware range check covers the per-lane (vector) offset only.  Rows past
M or N and K-tiles past the end must therefore be kept out of range by the
offset itself.  This test restates the offset arithmetic of every load the
kernel issues (x' chunks, PQ2_0 code words and scales, Q8_0 code pairs and
scales) for the three token tiles, and checks at tail shapes (M % TM, N % TN,
M = 1, a Q8_0 K ending in half a K-tile) that every load either reads exactly
the element it stands for, inside its resource, or sits at or past the end of
the resource (so the hardware returns zeros without touching memory).  The
16- and 64-token tiles split K into slices of whole K-tiles (pairs for
PQ2_0); each slice's loads are checked over its own K-tiles and prefetches."""
import pytest

OOR = 0x7FFFFFF0
TK = 64
CFGS = {256: (256, 160, 512), 64: (64, 64, 256), 16: (16, 64, 256)}  # TM: (TM, TN, threads)


def tile_m(M):
    return 16 if M <= 16 else (64 if M <= 96 else 256)


def k_slices(fmt, M, N, K):
    """(first, end) K-tiles of each slice: the small tiles are split into up
    to 1024 workgroups, in units of 2 K-tiles for PQ2_0."""
    TM, TN, _ = CFGS[tile_m(M)]
    KT = -(-K // TK)
    tiles = -(-M // TM) * -(-N // TN)
    if TM == 256 or tiles >= 1024:
        return [(0, KT)]
    unit = 2 if fmt == 1 else 1
    units = -(-KT // unit)
    S = max(1, min(1024 // tiles, units, 16))
    per = -(-units // S) * unit
    return [(k0, min(k0 + per, KT)) for k0 in range(0, KT, per)]


def check(fmt, M, N, K):
    TM, TN, NT = CFGS[tile_m(M)]
    RPP = NT // 8                      # rows staged per pass
    AROWS = max(TM, 32)
    ALOADS = AROWS // RPP
    UNITS = -(-(TN * TK // 8) // NT)   # the last pass covers the first UNIT_TAIL threads
    UNIT_TAIL = TN * TK // 8 - (UNITS - 1) * NT
    assert AROWS % RPP == 0 and UNIT_TAIL % 64 == 0
    group = 128 if fmt == 1 else 32
    G = K // group
    C = (G + 7) // 8
    d_tile = 256 * C
    KT = -(-K // TK)
    mt, nt = -(-M // TM), -(-N // TN)
    for m_tile in sorted({0, mt - 1}):
        for n_tile in sorted({0, nt - 1}):
            m0, n0 = m_tile * TM, n_tile * TN
            arows, brows = min(M - m0, TM), min(N - n0, TN)
            a_size = arows * K * 2
            q_size = -(-brows // 16) * G * 512
            d_size = -(-brows // 16) * d_tile
            assert max(a_size, q_size, d_size) < OOR
            for tid in range(NT):
                arow, ach = tid >> 3, tid & 7
                a_off = (arow * K + ach * (16 if fmt == 1 else 8)) * 2
                for kt0, kt1 in k_slices(fmt, M, N, K):
                  for kt in range(kt0, kt1 + 2):    # the kernel prefetches two tiles ahead
                    in_k = kt < kt1 if fmt == 1 else kt < kt1 and kt * TK + 8 * ach < K
                    for i in range(ALOADS):
                        row = RPP * i + arow
                        if fmt == 1:
                            k = (kt >> 1) * 128 + (kt & 1) * 8 + 16 * ach
                            ak = a_off + ((kt >> 1) * 128 + (kt & 1) * 8) * 2
                        else:
                            k = kt * TK + 8 * ach
                            ak = a_off + kt * TK * 2
                        off = ak + i * RPP * K * 2 if (in_k and row < TM) else OOR
                        valid = in_k and row < TM and row < arows and k < K
                        if valid:
                            assert off == (row * K + k) * 2 and off + 16 <= a_size
                        else:
                            assert off >= a_size, (fmt, M, N, K, tid, kt, i)
                    # weight units: row RPP i + t / 8, chunk t % 8
                    if fmt == 1:
                        if kt % 2:
                            continue                  # a block's words come with its even K-tile
                        kb = kt >> 1
                        q_off = (tid >> 7) * G * 512 + ((tid >> 3) & 15) * 32 + ach * 4
                        d_off = (tid >> 7) * d_tile + ((tid >> 3) & 15) * 16
                        for i in range(UNITS):
                            row = RPP * i + (tid >> 3)
                            ok = in_k and (i < UNITS - 1 or tid < UNIT_TAIL)
                            qo = q_off + kb * 512 + i * (RPP // 16) * G * 512 if ok else OOR
                            do = d_off + (kb >> 3) * 256 + (kb & 7) * 2 + i * (RPP // 16) * 256 * C if ok else OOR
                            if ok:
                                assert row < TN
                            if ok and row < -(-brows // 16) * 16:
                                assert qo == ((row // 16) * G + kb) * 512 + (row % 16) * 32 + ach * 4
                                assert qo + 4 <= q_size
                                assert do == ((row // 16) * C + kb // 8) * 256 + (row % 16) * 16 + 2 * (kb % 8)
                                assert do + 2 <= d_size
                            else:
                                assert qo >= q_size and do >= d_size
                    else:
                        b = 2 * kt + (ach >> 2)
                        q_off = ((tid >> 7) * G * 512 + ((tid >> 3) & 15) * 32 + (ach & 3) * 8
                                 + (ach >> 2) * 512)
                        d_off = (tid >> 7) * d_tile + ((tid >> 3) & 15) * 16
                        for i in range(UNITS):
                            row = RPP * i + (tid >> 3)
                            ok = in_k and (i < UNITS - 1 or tid < UNIT_TAIL)
                            qo = q_off + kt * 1024 + i * (RPP // 16) * G * 512 if ok else OOR
                            do = (d_off + (b >> 3) * 256 + (b & 7) * 2 + i * (RPP // 16) * 256 * C) if ok else OOR
                            if ok:
                                assert row < TN
                            if ok and row < -(-brows // 16) * 16:
                                assert b < G
                                assert qo == ((row // 16) * G + b) * 512 + (row % 16) * 32 + (ach & 3) * 8
                                assert qo + 8 <= q_size
                                assert do == ((row // 16) * C + b // 8) * 256 + (row % 16) * 16 + 2 * (b % 8)
                                assert do + 2 <= d_size
                            else:
                                assert qo >= q_size and do >= d_size


@pytest.mark.parametrize("fmt,M,N,K", [
    (1, 1, 1, 128), (1, 300, 170, 640), (1, 2048, 10240, 256), (1, 17, 65, 384), (1, 97, 161, 128),
    (1, 64, 64, 256), (2, 1, 1, 32), (2, 300, 170, 96), (2, 70, 17, 160), (2, 16, 100, 224),
    (2, 257, 161, 352), (1, 16, 640, 5120), (2, 64, 640, 1056), (1, 96, 130, 2048)])
def test_gemm_loads_stay_in_range(fmt, M, N, K):
    check(fmt, M, N, K)


def test_k_slices_cover_k_once():
    for fmt, M, N, K in ((1, 16, 10240, 5120), (1, 64, 10240, 5120), (2, 16, 17408, 5120),
                         (2, 5, 100, 96), (1, 96, 130, 2048), (1, 1, 1, 128)):
        sl = k_slices(fmt, M, N, K)
        KT = -(-K // TK)
        assert sl[0][0] == 0 and sl[-1][1] == KT
        assert all(a[1] == b[0] for a, b in zip(sl, sl[1:]))
        assert all(k1 > k0 for k0, k1 in sl)
        if fmt == 1:
            assert all(k0 % 2 == 0 for k0, _ in sl)
