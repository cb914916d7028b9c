"""Pins for the oracle's MXFP4 path (CPU only).

TeleFuser "Quantization" (converter section: MXFP4/6/8 use 32-value blocks
with E8M0 scales).  The block rule is the OCP Microscaling (MX) v1.0 one for
E2M1 elements -- shared exponent floor(log2(amax)) - 2, clamped to
[-127, 127]; elements v / 2^shared clamped to +-6 and rounded to the nearest
E2M1 value (0, 0.5, 1, 1.5, 2, 3, 4, 6), ties to the even code -- since the
pages print no rule of their own.  Expected values are worked by hand from
that rule or computed with exact rationals, never taken from the oracle.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as orc
import synth

pytestmark = pytest.mark.filterwarnings("ignore")

MAG = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
       Fraction(4), Fraction(6)]


def bf16(values):
    return synth.to_bf16_bits(np.asarray(values, dtype=np.float32))


def block(values):
    v = list(values) + [0.0] * (32 - len(values))
    return bf16([v])


def unpack(q):
    """Packed bytes [R, C/2] -> codes [R, C] (lower index in the low nibble)."""
    q = np.asarray(q, dtype=np.uint8)
    out = np.empty((q.shape[0], q.shape[1] * 2), np.uint8)
    out[:, 0::2] = q & 15
    out[:, 1::2] = q >> 4
    return out


def exact_e2m1(t: Fraction, neg: bool) -> int:
    """Nearest E2M1 code by exact rationals, saturating at 6, ties to even."""
    a = min(abs(t), Fraction(6))
    best = min(range(8), key=lambda c: (abs(a - MAG[c]), c & 1))
    return best | (8 if neg else 0)


def test_worked_block():
    # amax 6: floor(log2 6) = 2 -> shared 0 -> E8M0 127, X = 1.
    # 1.25 ties 1 (code 2) / 1.5 (3) -> 1; 1.75 ties 1.5 / 2 (4) -> 2;
    # 0.25 ties 0 / 0.5 -> 0; 5 ties 4 (6) / 6 (7) -> 4; 2.5 ties 2 / 3 -> 2
    q, s = orc.quantize_mx4(block([6.0, -3.0, 1.25, 1.75, 0.25, 0.3125, 5.0, 5.5, -0.0, 2.5]))
    assert s.tolist() == [[127]]
    want = [7, 8 | 5, 2, 4, 0, 1, 6, 7, 8, 4]
    assert unpack(q)[0, :10].tolist() == want
    assert q[0, 0] == (7 | ((8 | 5) << 4))          # element 0 in the low nibble
    assert (unpack(q)[0, 10:] == 0).all()


def test_saturation_and_scaling():
    # amax 7.5: floor(log2) = 2 -> E8M0 127: 7.5 -> 6 (saturated), 7 -> 6, -6.5 -> -6
    q, s = orc.quantize_mx4(block([7.5, 7.0, -6.5]))
    assert s.tolist() == [[127]] and unpack(q)[0, :3].tolist() == [7, 7, 15]
    # amax 0.75: floor(log2) = -1 -> shared -3 -> E8M0 124, X = 1/8:
    # 0.75 * 8 = 6 -> 7; 0.1 * 8 = 0.8 -> 1 (code 2); 0.03125 * 8 = 0.25 -> 0
    q, s = orc.quantize_mx4(block([0.75, 0.1, 0.03125, -0.03125]))
    assert s.tolist() == [[124]] and unpack(q)[0, :4].tolist() == [7, 2, 0, 8]


def test_zero_subnormal_and_huge_blocks():
    q, s = orc.quantize_mx4(block([0.0, -0.0]))
    assert s.tolist() == [[0]] and unpack(q)[0, :2].tolist() == [0, 8]
    # 2^-128 (BF16 subnormal): floor(log2) -128 -> shared -130 -> clamped -127
    # (E8M0 0): 2^-128 / 2^-127 = 0.5 -> code 1
    q, s = orc.quantize_mx4(block([2.0 ** -128]))
    assert s.tolist() == [[0]] and unpack(q)[0, 0] == 1
    # 2^120: shared 118 -> E8M0 245; 2^120 / 2^118 = 4 -> code 6
    q, s = orc.quantize_mx4(block([2.0 ** 120, -(2.0 ** 117)]))
    assert s.tolist() == [[245]] and unpack(q)[0, :2].tolist() == [6, 8 | 1]


def test_scale_code_closed_form_every_bf16_amax():
    bits = np.arange(1, 0x7F80, dtype=np.uint32)
    amax = (bits << 16).view(np.float32)
    got = np.array([orc.mx4_scale_code(float(a)) for a in amax], dtype=np.int64)
    want = np.maximum(((bits >> 7) & 0xFF).astype(np.int64) - 2, 0)
    assert np.array_equal(got, want)


def test_e2m1_encoder_against_exact_rationals():
    vals = [Fraction(i, 64) for i in range(0, 9 * 64)] + [Fraction(1, 3), Fraction(7, 3)]
    rng = np.random.default_rng(1)
    vals += [Fraction(float(v)) for v in rng.uniform(0, 8, 2000).astype(np.float32)]
    for v in vals:
        f = float(v)
        assert orc.e2m1_encode(f) == exact_e2m1(v, False), f
        assert orc.e2m1_encode(-f) == exact_e2m1(v, True), -f
    for c in range(16):
        assert Fraction(orc.e2m1_value(c)) == (-MAG[c & 7] if c & 8 else MAG[c & 7])


def test_block_invariants_on_random_rows():
    rng = np.random.default_rng(5)
    x = rng.standard_t(4, (64, 256)).astype(np.float32) * np.exp2(rng.integers(-20, 20, (64, 1)))
    x[rng.random(x.shape) < 0.02] = 0.0
    xb = bf16(x)
    q, s = orc.quantize_mx4(xb)
    codes = unpack(q)
    vals = np.vectorize(orc.e2m1_value)(codes)
    X = np.exp2(s.astype(np.float64) - 127).repeat(32, axis=1)
    xv = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nz = np.abs(xv).reshape(64, -1, 32).max(axis=2) > 0
    top = np.abs(vals).reshape(64, -1, 32).max(axis=2)
    # amax / X lies in [4, 8): the block maximum encodes to 4 or 6
    assert np.isin(top[nz], [4.0, 6.0]).all()
    t = np.abs(xv) / X
    step = np.where(t < 2, 0.5, np.where(t < 4, 1.0, 2.0))
    bound = np.where(t > 6, t - 6, step / 2) * X
    assert (np.abs(xv - vals * X) <= bound * (1 + 1e-12)).all()
    assert (np.sign(vals[vals != 0]) == np.sign(xv[vals != 0])).all()


def _codes(rng, R, K):
    c = rng.integers(0, 16, (R, K)).astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8), c


def test_gemm_reduces_to_plain_dot_with_uniform_scales():
    rng = np.random.default_rng(9)
    M, N, K = 5, 7, 128
    qa, ca = _codes(rng, M, K)
    qb, cb = _codes(rng, N, K)
    ea = np.repeat(rng.integers(110, 140, (M, 1)), K // 32, axis=1).astype(np.uint8)
    eb = np.repeat(rng.integers(110, 140, (N, 1)), K // 32, axis=1).astype(np.uint8)
    y = orc.linear_mx4_ref(qa, ea, qb, eb)
    # integer dot of 2 * value (an integer for every E2M1 code)
    twice = np.array([int(2 * (-MAG[c & 7] if c & 8 else MAG[c & 7])) for c in range(16)])
    d = twice[ca].astype(np.int64) @ twice[cb].astype(np.int64).T / 4.0
    want = d * np.exp2(ea[:, :1].astype(np.float64) - 127) * np.exp2(eb[:, 0].astype(np.float64) - 127)
    assert np.array_equal(y, want)


def test_gemm_brute_force_exact_rationals():
    rng = np.random.default_rng(11)
    M, N, K = 3, 4, 96
    qa, ca = _codes(rng, M, K)
    qb, cb = _codes(rng, N, K)
    ea = rng.integers(100, 150, (M, K // 32)).astype(np.uint8)
    eb = rng.integers(100, 150, (N, K // 32)).astype(np.uint8)
    bias = bf16(rng.standard_normal(N))
    y = orc.linear_mx4_ref(qa, ea, qb, eb, bias=bias)
    val = lambda c: -MAG[c & 7] if c & 8 else MAG[c & 7]  # noqa: E731
    for m in range(M):
        for n in range(N):
            acc = sum(val(int(ca[m, k])) * val(int(cb[n, k])) *
                      Fraction(2) ** (int(ea[m, k // 32]) - 127 + int(eb[n, k // 32]) - 127)
                      for k in range(K))
            acc += Fraction(orc.bf16_to_f32(int(bias[n])))
            assert abs(Fraction(y[m, n]) - acc) <= abs(acc) * Fraction(1, 10 ** 12)
