"""Pins of the oracle's decode-to-bf16 (precisit "pack-unpack-run" README,
codec.py description: decoding gives back c * s; screen.py description: the
decoder hands the selected weights back as bf16).

The expected values come from definitions written here independently of the
oracle: the base-3 digits of a byte from integer division, the product c * s
as an exact Fraction, and the nearest bf16 (ties to the even significand)
found by comparing exact distances to the neighbouring bf16 values."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def f16_value(bits: int) -> Fraction:
    sign = -1 if bits & 0x8000 else 1
    e, m = (bits >> 10) & 0x1F, bits & 0x3FF
    if e == 0:
        return sign * Fraction(m, 1 << 24)
    return sign * Fraction(1024 + m, 1 << 10) * (Fraction(2) ** (e - 15))


def bf16_value(bits: int) -> Fraction:
    sign = -1 if bits & 0x8000 else 1
    e, m = (bits >> 7) & 0xFF, bits & 0x7F
    if e == 0:
        return sign * Fraction(m, 1 << 7) * (Fraction(2) ** -126)
    return sign * Fraction(128 + m, 1 << 7) * (Fraction(2) ** (e - 127))


def nearest_bf16(v: Fraction, negative_zero: bool) -> int:
    """Nearest bf16 bit pattern to v (finite, inside the normal range), ties
    to the even significand; a zero keeps the given sign."""
    if v == 0:
        return 0x8000 if negative_zero else 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    best = None
    for e in range(1, 255):
        lo = Fraction(2) ** (e - 127)
        if not (lo <= a < 2 * lo):
            continue
        step = lo / 128
        k = int(a / step)                       # a in [k step, (k+1) step)
        for cand in (k, k + 1):
            d = abs(a - cand * step)
            key = (d, cand % 2)                 # nearer first, then even
            if best is None or key < best[0]:
                best = (key, cand, e)
    _, cand, e = best
    if cand == 256:
        cand, e = 128, e + 1
    return sign | (e << 7) | (cand - 128)


def encode(codes):
    """Bytes of a run of codes, five base-3 digits a byte, first lowest."""
    out = []
    for b in range(0, len(codes), 5):
        v = 0
        for i, c in enumerate(codes[b:b + 5]):
            v += (c + 1) * 3 ** i
        out.append(v)
    return np.array(out, np.uint8)


def expected(codes, sbits):
    s = f16_value(sbits)
    # a zero product takes the XOR of the operands' signs (code 0 counts as +0)
    return [nearest_bf16(c * s, negative_zero=(c == -1) != bool(sbits & 0x8000)) for c in codes]


@pytest.mark.parametrize("sbits", [0x3C00, 0x3C04, 0x3C05, 0x3C0C, 0x3C14, 0x7BFF, 0x0001, 0x03FF,
                                   0x0000, 0x8000, 0xBC00, 0xB555, 0x2E66])
def test_decode_values_match_the_definition(sbits):
    codes = [1, -1, 0, 1, -1]
    w, st = oracle.dequantize(encode(codes).reshape(1, 1), np.array([[sbits]], np.uint16), 1, 5, 5)
    assert st == 0
    assert [int(v) for v in w[0]] == expected(codes, sbits)


def test_printed_roundings():
    """A few results written out: RNE ties go to the even significand."""
    def dec(sbits, c=1):
        w, _ = oracle.dequantize(encode([c] * 5).reshape(1, 1), np.array([[sbits]], np.uint16),
                                 1, 5, 5)
        return int(w[0, 0])
    assert dec(0x3C00) == 0x3F80          # 1.0
    assert dec(0x3C00, -1) == 0xBF80      # -1.0
    assert dec(0x3C04) == 0x3F80          # 1 + 2^-8: a tie, to the even 1.0
    assert dec(0x3C0C) == 0x3F82          # 1 + 3*2^-8: a tie, to the even 1 + 2^-6
    assert dec(0x3C05) == 0x3F81          # above the tie: up
    assert dec(0x7BFF) == 0x4780          # 65504 -> 65536
    assert dec(0x0001) == 0x3380          # 2^-24, exact in bf16
    assert dec(0x0000, -1) == 0x8000      # -1 * +0 = -0
    assert dec(0x3C00, 0) == 0x0000       # 0 * s = +0 for s > 0


def test_random_groups_match_the_definition():
    rng = np.random.default_rng(5)
    N, K, G = 6, 320, 64
    codes = rng.integers(-1, 2, size=(N, K))
    nG, B = K // G, (G + 4) // 5
    packed = np.zeros((N, nG * B), np.uint8)
    for n in range(N):
        for g in range(nG):
            run = list(codes[n, g * G:(g + 1) * G]) + [0] * (5 * B - G)
            packed[n, g * B:(g + 1) * B] = encode(run)
    finite = [b for b in range(0x10000) if ((b >> 10) & 0x1F) != 0x1F]
    scales = rng.choice(finite, size=(N, nG)).astype(np.uint16)
    w, st = oracle.dequantize(packed, scales, N, K, G)
    assert st == 0
    for n in range(N):
        for g in range(nG):
            want = expected(list(codes[n, g * G:(g + 1) * G]), int(scales[n, g]))
            assert [int(v) for v in w[n, g * G:(g + 1) * G]] == want


def test_invalid_bytes_padding_and_nonfinite_scales_are_flagged():
    codes = [1] * 64 + [0]
    packed = encode(codes).reshape(1, -1).copy()
    s = np.array([[0x3C00]], np.uint16)
    w, st = oracle.dequantize(packed, s, 1, 64, 64)
    assert st == 0 and all(int(v) == 0x3F80 for v in w[0])
    bad = packed.copy()
    bad[0, 3] = 250
    w, st = oracle.dequantize(bad, s, 1, 64, 64)
    assert st == oracle.INVALID_BYTE
    assert all(int(v) == 0 for v in w[0, 15:20])            # that byte's codes read as 0
    assert all(int(v) == 0x3F80 for v in w[0, :15])
    pad = encode(codes[:64] + [1]).reshape(1, -1)            # padding trit holds code +1
    _, st = oracle.dequantize(pad, s, 1, 64, 64)
    assert st == oracle.BAD_PADDING
    _, st = oracle.dequantize(packed, np.array([[0x7C00]], np.uint16), 1, 64, 64)
    assert st == oracle.NONFINITE


def test_a_changed_code_byte_changes_the_reconstruction():
    """precisit README, test_codec.py description: a changed valid code byte
    must change the reconstruction (nonzero scale)."""
    rng = np.random.default_rng(9)
    codes = list(rng.integers(-1, 2, size=64)) + [0]
    packed = encode(codes).reshape(1, -1)
    s = np.array([[0x2E66]], np.uint16)
    w0, _ = oracle.dequantize(packed, s, 1, 64, 64)
    for b in range(packed.shape[1]):
        for v in (0, 121, 242):
            if v == packed[0, b] or (b == packed.shape[1] - 1 and v // 81 != 1):
                continue  # same byte, or a non-canonical padding trit
            q = packed.copy()
            q[0, b] = v
            w1, st = oracle.dequantize(q, s, 1, 64, 64)
            assert st == 0
            assert not np.array_equal(w0, w1), (b, v)
