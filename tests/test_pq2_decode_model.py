"""Model of the PQ2_0 GEMV's code decode on the stored word layout (CPU only).

A stored PQ2_0 code word holds 16 codes: code j's low bit b0 at bit 2j and
its high bit b1 at bit (2j + 3) mod 32.  The GEMV turns a word into two words
of eight signed E2M1 (fp4) nibbles with three vector instructions:
    ev = ~w & 0x99999999            (nibble i: code 2i)
    od = ~rotr(w, 2) & 0x99999999   (nibble i: code 2i + 1)
Nibble bit 3 is the sign and bit 0 the mantissa bit of a subnormal (0.5), so
a code c must give the nibble of (c - 1) / 2: 0 -> 1001 (-0.5), 1 -> 1000
(-0), 2 -> 0001 (+0.5), and code 3, which the format does not use, 0000 (+0).
This test restates the placement rule (bit by bit, not via the packer's word
rotation) and checks the decode against that table for every code value at
every position.  The kernel's products are checked against the oracle by the
GPU tests."""
import numpy as np

import oracle
from gemm_kq_gemv_amd import inputs
from tests import _golden as G

MASK = 0x99999999
FP4 = {0: -0.5, 1: -0.0, 2: 0.5, 3: 0.0}


def place(codes):
    w = 0
    for j, q in enumerate(codes):
        w |= (q & 1) << (2 * j)
        w |= (q >> 1) << ((2 * j + 3) % 32)
    return w


def fp4_value(nib):
    sign = -1.0 if nib & 8 else 1.0
    exp, man = (nib >> 1) & 3, nib & 1
    mag = man * 0.5 if exp == 0 else (1 + man * 0.5) * 2.0 ** (exp - 1)
    return sign * mag


def decode(w):
    rot = ((w >> 2) | (w << 30)) & 0xFFFFFFFF
    return (~w) & MASK, (~rot) & MASK


def test_every_code_at_every_position():
    for j in range(16):
        for q in range(4):
            for fill in (0, 1, 2, 3):
                codes = [fill] * 16
                codes[j] = q
                ev, od = decode(place(codes))
                nib = (ev if j % 2 == 0 else od) >> (4 * (j // 2)) & 15
                want = FP4[q]
                assert fp4_value(nib) == want and np.signbit(fp4_value(nib)) == np.signbit(want), (j, q, fill)
                # the other nibble bits are clear
                assert nib & 6 == 0


def test_random_words_all_nibbles():
    r = np.random.default_rng(11)
    for _ in range(500):
        codes = r.integers(0, 4, 16)
        ev, od = decode(place(codes))
        for i in range(8):
            assert fp4_value((ev >> (4 * i)) & 15) == FP4[codes[2 * i]]
            assert fp4_value((od >> (4 * i)) & 15) == FP4[codes[2 * i + 1]]


def test_oracle_layout_matches_the_rule():
    """The oracle's planar words are `place` of the block's codes, and the
    numpy word view of tests/_golden.py inverts them."""
    N, K = 5, 384
    aos = oracle.pack_pq2_aos(inputs.weights(21, N, K)).reshape(N, K // 128, 34)
    pl = oracle.aos_to_planar(oracle.FMT_PQ2_0, aos, N, K)
    stored = G.stored_code_rows(pl, N, K, 1).reshape(N, K // 128, 8, 4)
    for n in range(N):
        for b in range(K // 128):
            for i in range(8):
                qs = aos[n, b, 2 + 4 * i: 6 + 4 * i]
                codes = [(int(qs[j // 4]) >> (2 * (j % 4))) & 3 for j in range(16)]
                w = int(stored[n, b, i].copy().view("<u4")[0])
                assert w == place(codes), (n, b, i)
    assert np.array_equal(G.code_rows(pl, N, K, 1).reshape(N, K // 128, 32), aos[:, :, 2:])
