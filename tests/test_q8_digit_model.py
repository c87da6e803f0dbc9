"""Model of the Q8_0 GEMV's activation digits (CPU only).

For one to four activation rows the kernel feeds x' to the int8 matrix cores
as four signed base-256 digits of one integer per element.  This test
restates that arithmetic on the CPU, step by step as the kernel takes it, and
checks what the design relies on:

* the exponent s puts the row's largest |x'| in [2^29, 2^30) (or leaves s at
  its clamp), so I = rne(x' 2^s) fits 31 bits;
* J = I + 0x80808080 stays in [0, 2^32), and the byte transpose by
  v_perm_b32 selectors followed by flipping each byte's top bit gives digit
  planes d_t in [-128, 127] with sum_t d_t 256^(3-t) == I exactly;
* I 2^-s is within 2^-30 of the row maximum (plus the fp32 rounding of the
  scaling multiply, 2^-24 of the element) of x';
* a 32-element group's integer sum of int8 weights times digits stays below
  2^24 in magnitude, so its fp32 conversion is exact.
The kernel's own results are checked against the oracle by the GPU tests."""
import numpy as np
import pytest

BIAS = 0x80808080


def digit_exponent(bound):
    """s with bound * 2^s in [2^29, 2^30), clamped to [-126, 126]; 0 for a
    zero, infinite or NaN bound (read from the binary32 exponent field)."""
    b = np.float32(bound)
    ef = (int(b.view(np.uint32)) >> 23) & 0xFF
    if not (b > 0) or ef == 0xFF:
        return 0
    e = 29 - (ef - 127)
    return max(-126, min(126, e))


def perm(s0, s1, sel):
    """v_perm_b32: byte i of the result is byte sel_i of {s1 (0..3), s0 (4..7)},
    0 for selector 0x0c."""
    src = [(s1 >> (8 * i)) & 255 for i in range(4)] + [(s0 >> (8 * i)) & 255 for i in range(4)]
    out = 0
    for i in range(4):
        k = (sel >> (8 * i)) & 255
        out |= (0 if k == 0x0C else src[k]) << (8 * i)
    return out


def transpose_bytes(j0, j1, j2, j3):
    p_lo, p_hi = perm(j1, j0, 0x05010400), perm(j1, j0, 0x07030602)
    q_lo, q_hi = perm(j3, j2, 0x05010400), perm(j3, j2, 0x07030602)
    return [perm(q_lo, p_lo, 0x05040100), perm(q_lo, p_lo, 0x07060302),
            perm(q_hi, p_hi, 0x05040100), perm(q_hi, p_hi, 0x07060302)]


def encode_chunk(v8, cs):
    """8 staged values of one row -> 4 digit planes of 8 int8 (digit 0 first)."""
    prod = (np.asarray(v8, np.float32) * np.float32(cs)).astype(np.float32)
    I = np.rint(prod).astype(np.int64)           # round half to even, as v_rndne_f32
    assert np.all(np.abs(I) < 2 ** 31)
    J = [(int(i) + BIAS) % (1 << 32) for i in I]
    assert all(0 <= (int(i) + BIAS) < (1 << 32) for i in I)
    lo, hi = transpose_bytes(*J[:4]), transpose_bytes(*J[4:])
    planes = np.zeros((4, 8), np.int64)
    for t in range(4):
        words = (lo[3 - t] ^ BIAS, hi[3 - t] ^ BIAS)
        for e in range(8):
            byte = (words[e // 4] >> (8 * (e % 4))) & 255
            planes[t, e] = byte - 256 if byte >= 128 else byte
    return I, planes


def rows(seed):
    r = np.random.default_rng(seed)
    out = [r.standard_normal(256).astype(np.float32),
           (r.standard_normal(256) * 1e-30).astype(np.float32),
           np.zeros(256, np.float32),
           r.integers(-8, 9, 256).astype(np.float32)]
    x = r.standard_normal(256).astype(np.float32)
    x[[3, 77, 200]] = [1e4, -2e4, 3e3]            # outlier channels
    out.append(x)
    x = r.standard_normal(256).astype(np.float32)
    x[5] = np.float32(2.0 ** 30) * 0.999999       # a maximum just below a binade
    out.append(x)
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("inv_sqrt_n", [1.0, float(np.float32(1 / np.sqrt(128)))])
def test_digits_give_the_integer_back(seed, inv_sqrt_n):
    for staged in rows(seed):
        bound = np.float32(np.max(np.abs(staged)) * np.float32(inv_sqrt_n))
        s = digit_exponent(bound)
        cs = np.float32(np.ldexp(np.float32(inv_sqrt_n), s))
        if bound > 0 and s < 126:
            assert 2.0 ** 29 <= float(bound) * 2.0 ** s < 2.0 ** 30
        xp = staged.astype(np.float64) * float(inv_sqrt_n)      # x' itself
        for c in range(0, 256, 8):
            I, planes = encode_chunk(staged[c:c + 8], cs)
            assert planes.min() >= -128 and planes.max() <= 127
            back = sum(planes[t] * 256 ** (3 - t) for t in range(4))
            assert np.array_equal(back, I)
            err = np.abs(I * 2.0 ** -s - xp[c:c + 8])
            lim = 2.0 ** -30 * float(np.max(np.abs(xp))) * 1.0001 + 2.0 ** -24 * np.abs(xp[c:c + 8])
            if s < 126:
                assert np.all(err <= lim + 1e-300)


def test_group_sums_convert_exactly():
    # the largest |sum over 32 of w * d| with int8 weights and digits
    worst = 32 * 127 * 128
    assert worst < 2 ** 24
    r = np.random.default_rng(9)
    w = r.integers(-127, 128, (1000, 32))
    d = r.integers(-128, 128, (1000, 32))
    sums = (w * d).sum(axis=1)
    assert np.all(np.abs(sums) <= worst)
    assert np.all(sums.astype(np.float32).astype(np.int64) == sums)


def test_exponent_clamps():
    assert digit_exponent(0.0) == 0 and digit_exponent(np.inf) == 0 and digit_exponent(np.nan) == 0
    assert digit_exponent(1.0) == 29
    assert digit_exponent(2.0 ** -120) == 126          # clamped: 2^-120 * 2^126 = 2^6
    assert digit_exponent(np.float32(3.0e38)) == 29 - 127
