"""Pins for the oracle's MXFP6 path (CPU only).

TeleFuser "Quantization" (converter section: MXFP4/6/8 use 32-value blocks
with E8M0 scales).  OCP Microscaling (MX) v1.0 rule for the two FP6 element
types: E2M3 (bias 1, largest 7.5) and E3M2 (bias 3, largest 28), shared
exponent floor(log2(amax)) - emax (2 and 4), elements rounded to the
nearest value with ties to the even code and clamped at the largest.  Codes
are a little-endian 6-bit stream per row.  Expected values are worked by
hand or computed with exact rationals, never taken from the oracle.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as orc
import synth

pytestmark = pytest.mark.filterwarnings("ignore")


def grid(fmt):
    """The 32 magnitudes in code order, from the format's definition."""
    eb, mb, bias = (2, 3, 1) if fmt == "e2m3" else (3, 2, 3)
    out = []
    for e in range(1 << eb):
        for m in range(1 << mb):
            if e == 0:
                out.append(Fraction(m, 1 << mb) * Fraction(2) ** (1 - bias))
            else:
                out.append((1 + Fraction(m, 1 << mb)) * Fraction(2) ** (e - bias))
    return out


def exact_encode(fmt, t: Fraction, neg: bool) -> int:
    g = grid(fmt)
    a = min(abs(t), g[-1])
    best = min(range(32), key=lambda c: (abs(a - g[c]), c & 1))
    return best | (32 if neg else 0)


def unpack6(q, K):
    q = np.asarray(q, dtype=np.uint8)
    out = np.zeros((q.shape[0], K), np.uint8)
    for i in range(K):
        bit = 6 * i
        v = q[:, bit >> 3].astype(np.uint32)
        if (bit & 7) > 2:
            v = v | (q[:, (bit >> 3) + 1].astype(np.uint32) << 8)
        out[:, i] = (v >> (bit & 7)) & 63
    return out


def pack6(codes):
    R, K = codes.shape
    q = np.zeros((R, K * 3 // 4), np.uint8)
    for i in range(K):
        bit = 6 * i
        v = codes[:, i].astype(np.uint32) << (bit & 7)
        q[:, bit >> 3] |= (v & 255).astype(np.uint8)
        if (bit & 7) > 2:
            q[:, (bit >> 3) + 1] |= (v >> 8).astype(np.uint8)
    return q


def bf16(values):
    return synth.to_bf16_bits(np.asarray(values, dtype=np.float32))


def block(values):
    v = list(values) + [0.0] * (32 - len(values))
    return bf16([v])


def test_value_tables():
    for fmt in ("e2m3", "e3m2"):
        g = grid(fmt)
        assert all(g[i] < g[i + 1] for i in range(31))
        for c in range(64):
            want = -g[c & 31] if c & 32 else g[c & 31]
            assert Fraction(orc.fp6_value(fmt, c)) == want
    assert grid("e2m3")[31] == Fraction(15, 2) and grid("e2m3")[1] == Fraction(1, 8)
    assert grid("e3m2")[31] == 28 and grid("e3m2")[1] == Fraction(1, 16)


def test_worked_blocks_and_packing():
    # E2M3, amax 7.5: shared 0 (E8M0 127).  0.0625 ties 0 / 0.125 -> 0;
    # 0.1875 ties 0.125 (code 1) / 0.25 (2) -> 2; 1.0625 ties 1 (8) / 1.125 (9)
    # -> 8; 3.125 ties 3 (20) / 3.25 (21) -> 20; -7.90625 -> -7.5 (saturated)
    q, s = orc.quantize_mx6(block([7.5, 0.0625, 0.1875, 1.0625, 3.125, -7.9, -0.0]), "e2m3")
    assert s.tolist() == [[127]]
    c = unpack6(q, 32)[0]
    assert c[:7].tolist() == [31, 0, 2, 8, 20, 32 | 31, 32]
    # the stream: byte 0 = c0 | c1 << 6, byte 1 = c1 >> 2 | c2 << 4, byte 2 = c2 >> 4 | c3 << 2
    assert q[0, :3].tolist() == [31 | (0 << 6), 0 | (2 << 4) & 255, (2 >> 4) | (8 << 2)]
    # E3M2, amax 28: shared 0.  0.03125 ties 0 / 1/16 -> 0; 5 -> 1.25 * 4 (code 21);
    # 0.21875 ties 0.1875 (3) / 0.25 (4) -> 4; 30 -> 28 (31)
    q, s = orc.quantize_mx6(block([28.0, 0.03125, 5.0, 0.21875, 30.0]), "e3m2")
    assert s.tolist() == [[127]] and unpack6(q, 32)[0, :5].tolist() == [31, 0, 21, 4, 31]
    # E2M3 with amax 0.75: floor(log2) = -1 -> shared -3 (E8M0 124): 0.75 * 8 = 6 -> code 28
    q, s = orc.quantize_mx6(block([0.75, 0.01]), "e2m3")
    assert s.tolist() == [[124]] and unpack6(q, 32)[0, :2].tolist() == [28, 1]


def test_pack_order_round_trip():
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 64, (3, 64)).astype(np.uint8)
    assert np.array_equal(unpack6(pack6(codes), 64), codes)


@pytest.mark.parametrize("fmt,emax", [("e2m3", 2), ("e3m2", 4)])
def test_scale_code_closed_form_every_bf16_amax(fmt, emax):
    bits = np.arange(1, 0x7F80, dtype=np.uint32)
    amax = (bits << 16).view(np.float32)
    got = np.array([orc.mx6_scale_code(fmt, float(a)) for a in amax], dtype=np.int64)
    want = np.maximum(((bits >> 7) & 0xFF).astype(np.int64) - emax, 0)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_encoder_against_exact_rationals(fmt):
    top = 8 if fmt == "e2m3" else 32
    vals = [Fraction(i, 128) for i in range(0, top * 128 + 64, 3)]
    vals += [(a + b) / 2 for a, b in zip(grid(fmt)[:-1], grid(fmt)[1:])]  # every midpoint
    rng = np.random.default_rng(1)
    vals += [Fraction(float(v)) for v in rng.uniform(0, top, 1500).astype(np.float32)]
    for v in vals:
        f = float(v)
        assert orc.fp6_encode(fmt, f) == exact_encode(fmt, v, False), (fmt, f)
        assert orc.fp6_encode(fmt, -f) == exact_encode(fmt, v, True), (fmt, -f)


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_block_invariants(fmt):
    rng = np.random.default_rng(5)
    x = rng.standard_t(4, (32, 256)).astype(np.float32) * np.exp2(rng.integers(-20, 20, (32, 1)))
    x[rng.random(x.shape) < 0.02] = 0.0
    xb = bf16(x)
    q, s = orc.quantize_mx6(xb, fmt)
    codes = unpack6(q, 256)
    g = [float(v) for v in grid(fmt)]
    vals = np.where(codes & 32, -1.0, 1.0) * np.array(g)[codes & 31]
    X = np.exp2(s.astype(np.float64) - 127).repeat(32, axis=1)
    xv = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    t = np.abs(xv) / X
    # amax / X lies in [2^emax, 2^(emax+1)): the block maximum encodes into
    # the top binade [2^emax, largest]
    top = np.abs(vals).reshape(32, -1, 32).max(axis=2)
    nz = np.abs(xv).reshape(32, -1, 32).max(axis=2) > 0
    emax = 2 if fmt == "e2m3" else 4
    assert ((top[nz] >= 2 ** emax) & (top[nz] <= g[-1])).all()
    # nearest grid value (below the largest): error at most half the gap
    gaps = np.diff(np.array(g))
    idx = np.clip(np.searchsorted(np.array(g), np.minimum(t, g[-1])), 1, 31)
    half = gaps[idx - 1] / 2
    bound = np.where(t > g[-1], t - g[-1], half) * X
    assert (np.abs(xv - vals * X) <= bound * (1 + 1e-12)).all()


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_gemm_brute_force_exact_rationals(fmt):
    rng = np.random.default_rng(11)
    M, N, K = 3, 4, 64
    ca = rng.integers(0, 64, (M, K)).astype(np.uint8)
    cb = rng.integers(0, 64, (N, K)).astype(np.uint8)
    ea = rng.integers(100, 150, (M, K // 32)).astype(np.uint8)
    eb = rng.integers(100, 150, (N, K // 32)).astype(np.uint8)
    bias = bf16(rng.standard_normal(N))
    y = orc.linear_mx6_ref(pack6(ca), ea, pack6(cb), eb, fmt, bias=bias)
    g = grid(fmt)
    val = lambda c: -g[c & 31] if c & 32 else g[c & 31]  # noqa: E731
    for m in range(M):
        for n in range(N):
            acc = sum(val(int(ca[m, k])) * val(int(cb[n, k])) *
                      Fraction(2) ** (int(ea[m, k // 32]) - 127 + int(eb[n, k // 32]) - 127)
                      for k in range(K))
            acc += Fraction(orc.bf16_to_f32(int(bias[n])))
            assert abs(Fraction(y[m, n]) - acc) <= abs(acc) * Fraction(1, 10 ** 12)
