"""Exact rational arithmetic used to pin the oracle on tiny inputs.

Nothing here uses binary floating point: values are ``fractions.Fraction``
and every rounding step is written from its definition (round to nearest,
ties to even, on the binary32 grid with subnormals, or on the E4M3FN grid of
the OCP OFP8 format).  It is a brute-force check of the quantisation formulas
of TeleFuser "Quantization" ("Core ideas" for INT8, "Scaled FP8 checkpoints:
W8A8" for FP8), independent of the oracle's C code.
"""
from fractions import Fraction


def bf16_bits_to_fraction(h: int) -> Fraction:
    s = -1 if (h >> 15) & 1 else 1
    e = (h >> 7) & 0xFF
    m = h & 0x7F
    assert e != 0xFF, "finite inputs only"
    if e == 0:
        return s * Fraction(m, 1 << 7) * Fraction(1, 1 << 126)
    return s * (1 + Fraction(m, 1 << 7)) * (Fraction(2) ** (e - 127))


def _floor_log2(v: Fraction) -> int:
    # largest e with 2^e <= v  (v > 0)
    e = v.numerator.bit_length() - v.denominator.bit_length()
    while Fraction(2) ** e > v:
        e -= 1
    while Fraction(2) ** (e + 1) <= v:
        e += 1
    return e


def _round_half_even_int(v: Fraction) -> int:
    return round(v)  # Fraction.__round__ rounds half to even


def round_to_binary32(v: Fraction) -> Fraction:
    """Round-to-nearest-even onto the binary32 grid (subnormals kept)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = max(_floor_log2(a), -126)
    ulp = Fraction(2) ** (e - 23)
    n = _round_half_even_int(a / ulp)
    r = n * ulp
    assert r < Fraction(2) ** 128, "overflow is out of contract"
    return sign * r


def e4m3fn_values():
    """Values of codes 0x00..0x7E from the OCP definition."""
    vals = []
    for c in range(127):
        e, m = c >> 3, c & 7
        if e == 0:
            vals.append(Fraction(m, 8) * Fraction(1, 64))
        else:
            vals.append((1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return vals


_E4 = e4m3fn_values()


def e4m3fn_encode_exact(t: Fraction, negative_zero: bool = False) -> int:
    """Nearest E4M3FN code, ties to the even code, saturating at 448."""
    neg = t < 0 or (t == 0 and negative_zero)
    a = abs(t)
    best, bestd = 0, None
    for c, v in enumerate(_E4):
        d = abs(a - v)
        if bestd is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    return best | (0x80 if neg else 0)


def quantize_row_exact(xbits, qtype: str, qmax: float):
    """(scale as Fraction, codes) for one row of BF16 bit patterns."""
    xs = [bf16_bits_to_fraction(int(h)) for h in xbits]
    negz = [(int(h) >> 15) & 1 == 1 for h in xbits]
    amax = max(abs(v) for v in xs)
    s = round_to_binary32(amax / Fraction(qmax))
    codes = []
    for v, nz in zip(xs, negz):
        if s == 0:
            t, tneg0 = Fraction(0), nz
        else:
            t = round_to_binary32(v / s)
            tneg0 = v < 0 or (v == 0 and nz)
        if qtype == "fp8":
            q = Fraction(qmax)
            t = min(max(t, -q), q)
            codes.append(e4m3fn_encode_exact(t, negative_zero=(t == 0 and tneg0)))
        else:
            r = _round_half_even_int(t)
            r = min(max(r, -128), 127)
            codes.append(r & 0xFF)
    return s, codes
