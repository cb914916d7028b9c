"""Pins for the oracle's MXFP8 path (CPU only).

Sources: TeleFuser "Quantization" (converter section: MXFP8 uses 32-value
blocks with E8M0 scales) and TeleFuser "量化" (离线转换).  The block rule is
the OCP Microscaling (MX) v1.0 one -- shared exponent floor(log2(amax)) - 8
for E4M3 elements, clamped to [-127, 127], elements v / 2^shared clamped to
+-448 and encoded E4M3FN round-to-nearest-even -- since the pages print no
rule of their own.  Every expected value below is worked out by hand from
that rule and the E4M3FN definition (1 sign, 4 exponent bits with bias 7, 3
mantissa bits), not produced by the oracle.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as orc
import synth

pytestmark = pytest.mark.filterwarnings("ignore")


def bf16(values):
    return synth.to_bf16_bits(np.asarray(values, dtype=np.float32))


def block(values):
    v = list(values) + [0.0] * (32 - len(values))
    return bf16([v])


def test_worked_block():
    # amax 3.5: floor(log2 3.5) = 1 -> shared exponent -7 -> E8M0 120, X = 2^-7;
    # x * 128 = [448, -224, 128, 56, 0, -0, 2^-3]
    q, s = orc.quantize_mx(block([3.5, -1.75, 1.0, 0.4375, 0.0, -0.0, 2.0 ** -10]))
    assert s.tolist() == [[120]]
    assert q[0, :7].tolist() == [0x7E, 0xF6, 0x70, 0x66, 0x00, 0x80, 0x20]
    assert (q[0, 7:] == 0).all()


def test_saturation_above_448():
    # amax 7.5: floor(log2) = 2 -> E8M0 121, X = 2^-6; 7.5 * 64 = 480 -> 448,
    # 7.0 * 64 = 448, 6.5 * 64 = 416 (exact: 1.625 * 2^8)
    q, s = orc.quantize_mx(block([7.5, 7.0, -6.5]))
    assert s.tolist() == [[121]]
    assert q[0, :3].tolist() == [0x7E, 0x7E, 0xFD]


def test_round_half_to_even():
    # amax 1: E8M0 119, X = 2^-8; 1.0 * 256 = 256 = 2^8 (exponent field 15) -> 0x78;
    # 17 lies halfway between 16 (mantissa 000) and 18 (001) -> 16 = 0x58;
    # 19 between 18 and 20 (010) -> 20 = 0x5A; -17 -> -16 = 0xD8
    q, s = orc.quantize_mx(block([1.0, 17 / 256, 19 / 256, -17 / 256]))
    assert s.tolist() == [[119]]
    assert q[0, :4].tolist() == [0x78, 0x58, 0x5A, 0xD8]
    assert [orc.e4m3fn_value(int(c)) for c in q[0, :4]] == [256.0, 16.0, 20.0, -16.0]


def test_zero_block_and_signed_zero():
    q, s = orc.quantize_mx(block([0.0, -0.0]))
    assert s.tolist() == [[0]]
    assert q[0, 0] == 0x00 and q[0, 1] == 0x80 and (q[0, 2:] == 0).all()


def test_subnormal_and_huge_amax():
    # 2^-130 (a BF16 subnormal): floor(log2) = -130 -> shared -138 -> clamped
    # to -127 (E8M0 0); 2^-130 / 2^-127 = 2^-3 -> 0x20
    q, s = orc.quantize_mx(block([2.0 ** -130]))
    assert s.tolist() == [[0]] and q[0, 0] == 0x20
    # 2^100: shared exponent 92 -> E8M0 219; 2^100 / 2^92 = 256 -> 0x78
    q, s = orc.quantize_mx(block([2.0 ** 100, -(2.0 ** 99)]))
    assert s.tolist() == [[219]] and q[0, :2].tolist() == [0x78, 0xF0]


def test_scale_code_closed_form_every_bf16_amax():
    """E8M0 byte = max(exponent field of the BF16 amax - 8, 0), for every
    positive finite BF16 value (the field is the biased exponent, so a normal
    amax has floor(log2) = field - 127; subnormals have field 0)."""
    bits = np.arange(1, 0x7F80, dtype=np.uint32)          # positive finite BF16
    amax = (bits << 16).view(np.float32)
    got = np.array([orc.mx_scale_code(float(a)) for a in amax], dtype=np.int64)
    want = np.maximum(((bits >> 7) & 0xFF).astype(np.int64) - 8, 0)
    assert np.array_equal(got, want)


def test_block_invariants_on_random_rows():
    rng = np.random.default_rng(5)
    x = rng.standard_t(4, (64, 256)).astype(np.float32) * np.exp2(rng.integers(-20, 20, (64, 1)))
    x[rng.random(x.shape) < 0.02] = 0.0
    xb = bf16(x)
    q, s = orc.quantize_mx(xb)
    xv = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    vals = np.vectorize(orc.e4m3fn_value)(q)
    X = np.exp2(s.astype(np.float64) - 127).repeat(32, axis=1)
    blocks = np.abs(xv).reshape(64, -1, 32).max(axis=2)
    nz = blocks > 0
    # the block maximum lands in [256, 448] (256 <= amax / X < 512, saturated at 448)
    top = np.abs(vals).reshape(64, -1, 32).max(axis=2)
    assert ((top[nz] >= 256) & (top[nz] <= 448)).all()
    # signs survive wherever the code is non-zero
    assert (np.sign(vals[vals != 0]) == np.sign(xv[vals != 0])).all()
    # error: half an E4M3 step of t (step 2^(floor(log2 |t|) - 3), at least
    # 2^-9 in the subnormal range), or the saturation gap above 448
    t = np.abs(xv) / X
    step = np.exp2(np.floor(np.log2(np.maximum(t, 2.0 ** -6))) - 3)
    bound = np.where(t > 448, t - 448, step / 2) * X
    assert (np.abs(xv - vals * X) <= bound * (1 + 1e-12)).all()


def test_gemm_reduces_to_plain_dot_with_uniform_scales():
    """With one E8M0 byte across every block of a row, the MX Linear is the
    plain code dot times 2^(ea + eb - 254)."""
    rng = np.random.default_rng(9)
    M, N, K = 5, 7, 128
    qa = rng.integers(0, 256, (M, K)).astype(np.uint8)
    qb = rng.integers(0, 256, (N, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x12
    qb[(qb & 0x7F) == 0x7F] = 0x34
    ea = np.repeat(rng.integers(110, 140, (M, 1)), K // 32, axis=1).astype(np.uint8)
    eb = np.repeat(rng.integers(110, 140, (N, 1)), K // 32, axis=1).astype(np.uint8)
    y = orc.linear_mx_ref(qa, ea, qb, eb)
    d = orc.dot(qa, qb, "fp8")
    want = d * np.exp2(ea[:, :1].astype(np.float64) - 127) * np.exp2(eb[:, 0].astype(np.float64) - 127)
    assert np.array_equal(y, want)


def test_gemm_brute_force_exact_rationals():
    """Tiny shapes against exact rational arithmetic, block scales varying."""
    rng = np.random.default_rng(11)
    M, N, K = 3, 4, 96
    qa = rng.integers(0, 256, (M, K)).astype(np.uint8)
    qb = rng.integers(0, 256, (N, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x55
    qb[(qb & 0x7F) == 0x7F] = 0x66
    ea = rng.integers(100, 150, (M, K // 32)).astype(np.uint8)
    eb = rng.integers(100, 150, (N, K // 32)).astype(np.uint8)
    bias = bf16(rng.standard_normal(N))
    y = orc.linear_mx_ref(qa, ea, qb, eb, bias=bias)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += (Fraction(orc.e4m3fn_value(int(qa[m, k]))) * Fraction(orc.e4m3fn_value(int(qb[n, k])))
                        * Fraction(2) ** (int(ea[m, k // 32]) - 127 + int(eb[n, k // 32]) - 127))
            acc += Fraction(orc.bf16_to_f32(int(bias[n])))
            assert abs(Fraction(y[m, n]) - acc) <= abs(acc) * Fraction(1, 10 ** 12)
