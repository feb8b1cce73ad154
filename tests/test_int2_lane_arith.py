"""The integer algebra of the INT2 (SUM) scan's lane arithmetic, emulated on the CPU in plain Python.

The 2-bit key format (include/prism.h: 32-bit word w of a row holds dims 16w .. 16w + 15, dim
16w + 4j + i in bits 8i + 2j) is read by the scan with the masks w & 0x33333333 and
(w >> 2) & 0x33333333, which put eight codes b in [0, 3] into the eight 4-bit fields of a word; the
group's summed query code of a dim, |qs| <= 15 * 127, is split into three signed base-16 digits
qs = 256 d2 + 16 d1 + d0 (each in [-8, 7]) packed into 4-bit fields in the same order, and a signed
8 x 4-bit dot product (v_dot8_i32_i4) accumulates each digit vector.  This file checks, against a
direct integer dot product, that the decomposition is exact and that the field order of the packed
digits matches the order in which the masks lay out the codes, and that the digit sums give the
-3 * sum(q) correction of the levels c = 2b - 3.  It checks the algebra only; the parity tests check
the kernel itself against the oracle."""
import random


def s4(x):
    """Signed value of a 4-bit field."""
    x &= 0xF
    return x - 16 if x >= 8 else x


def dot8_i4(a, b, c):
    """Signed 8 x 4-bit dot product of two 32-bit words, accumulated into c."""
    return c + sum(s4(a >> (4 * k)) * s4(b >> (4 * k)) for k in range(8))


def digits(q):
    d0 = ((q + 8) & 15) - 8
    r1 = (q - d0) >> 4
    d1 = ((r1 + 8) & 15) - 8
    return d0, d1, (r1 - d1) >> 4


def pack_codes(b):
    """Four 32-bit words of one lane's 64 dims in the 2-bit key format."""
    words = []
    for m in range(4):
        w = 0
        for j in range(4):
            for i in range(4):
                w |= int(b[16 * m + 4 * j + i]) << (8 * i + 2 * j)
        words.append(w)
    return words


def pack_digits(dn):
    """The eight nibble words of one digit vector over 64 dims: nibble k of word 2m holds dim
    16m + 8 (k & 1) + (k >> 1), of word 2m + 1 dim 16m + 4 + 8 (k & 1) + (k >> 1)."""
    out = []
    for m in range(4):
        by = [dn[16 * m + t] & 0xFF for t in range(16)]
        x = [by[4 * r] | by[4 * r + 1] << 8 | by[4 * r + 2] << 16 | by[4 * r + 3] << 24 for r in range(4)]
        out.append((x[0] & 0x0F0F0F0F) | ((x[2] & 0x0F0F0F0F) << 4))
        out.append((x[1] & 0x0F0F0F0F) | ((x[3] & 0x0F0F0F0F) << 4))
    return out


def lane_dot(qs, b):
    words = pack_codes(b)
    dig = list(zip(*[digits(q) for q in qs]))
    qn = [pack_digits(list(dig[n])) for n in range(3)]
    acc = [0, 0, 0]
    for m in range(4):
        lo, hi = words[m] & 0x33333333, (words[m] >> 2) & 0x33333333
        for n in range(3):
            acc[n] = dot8_i4(qn[n][2 * m], lo, acc[n])
            acc[n] = dot8_i4(qn[n][2 * m + 1], hi, acc[n])
    dot_b = 256 * acc[2] + 16 * acc[1] + acc[0]
    sums = [sum(dot8_i4(w, 0x11111111, 0) for w in qn[n]) for n in range(3)]
    return dot_b, 256 * sums[2] + 16 * sums[1] + sums[0]


def test_digit_decomposition_exact_over_the_range():
    for q in range(-15 * 127, 15 * 127 + 1):
        d = digits(q)
        assert all(-8 <= x <= 7 for x in d)
        assert 256 * d[2] + 16 * d[1] + d[0] == q


def test_lane_dot_matches_direct_dot():
    rng = random.Random(7)
    for trial in range(400):
        G = rng.randint(1, 15)
        if trial % 4 == 0:  # the extremes: every dim at +-127 G
            qs = [rng.choice((-1, 1)) * 127 * G for _ in range(64)]
        else:
            qs = [sum(rng.randint(-127, 127) for _ in range(G)) for _ in range(64)]
        b = [rng.randint(0, 3) for _ in range(64)]
        dot_b, qsum = lane_dot(qs, b)
        assert dot_b == sum(q * x for q, x in zip(qs, b))
        assert qsum == sum(qs)
        # the levels c = 2 b - 3 of the key format: the lane's contribution before the lane-group sum
        assert 2 * dot_b - 3 * qsum == sum(q * (2 * x - 3) for q, x in zip(qs, b))


def test_a_swapped_field_order_is_caught():
    """Packing the digits in plain dim order (not the masks' order) must fail the dot product."""
    rng = random.Random(3)
    qs = [sum(rng.randint(-127, 127) for _ in range(4)) for _ in range(64)]
    b = [rng.randint(0, 3) for _ in range(64)]
    words = pack_codes(b)
    dig = list(zip(*[digits(q) for q in qs]))
    acc = [0, 0, 0]
    for m in range(4):
        lo, hi = words[m] & 0x33333333, (words[m] >> 2) & 0x33333333
        for n in range(3):
            plain = [sum((dig[n][16 * m + 8 * h + k] & 0xF) << (4 * k) for k in range(8)) for h in range(2)]
            acc[n] = dot8_i4(plain[0], lo, acc[n])
            acc[n] = dot8_i4(plain[1], hi, acc[n])
    assert 256 * acc[2] + 16 * acc[1] + acc[0] != sum(q * x for q, x in zip(qs, b))
