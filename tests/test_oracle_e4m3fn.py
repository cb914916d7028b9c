"""Pins of the oracle's E4M3FN codec (OCP OFP8 E4M3FN, the cast of TeleFuser
"Quantization", section "Scaled FP8 checkpoints: W8A8").

* the closed-form decode table against printed facts of the format and
  against torch's float8_e4m3fn (a library implementation);
* the field-arithmetic encoder against an independent nearest-value search
  encoder on EVERY finite binary32 pattern, and against torch's cast;
* round trips of all 254 finite codes.
"""
import math

import numpy as np
import pytest
import torch


def test_decode_spot_values(orc):
    assert orc.e4m3fn_value(0x7E) == 448.0          # max finite
    assert orc.e4m3fn_value(0xFE) == -448.0
    assert orc.e4m3fn_value(0x01) == 2.0 ** -9      # min subnormal
    assert orc.e4m3fn_value(0x07) == 7 * 2.0 ** -9  # max subnormal
    assert orc.e4m3fn_value(0x08) == 2.0 ** -6      # min normal
    assert orc.e4m3fn_value(0x38) == 1.0            # E = 7, M = 0
    assert orc.e4m3fn_value(0x00) == 0.0 and math.copysign(1, orc.e4m3fn_value(0x00)) > 0
    assert orc.e4m3fn_value(0x80) == 0.0 and math.copysign(1, orc.e4m3fn_value(0x80)) < 0
    assert math.isnan(orc.e4m3fn_value(0x7F)) and math.isnan(orc.e4m3fn_value(0xFF))


def test_decode_table_matches_torch(orc):
    tab = orc.e4m3fn_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(tab), nan)
    assert nan.sum() == 2
    assert np.array_equal(tab[~nan], ref[~nan])
    assert np.array_equal(np.signbit(tab[~nan]), np.signbit(ref[~nan]))
    # strictly increasing magnitudes over the positive codes
    assert np.all(np.diff(tab[:127]) > 0)


def test_round_trip_all_codes(orc):
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        v = orc.e4m3fn_value(c)
        assert orc.e4m3fn_encode(v) == c, hex(c)
        assert orc.e4m3fn_encode_search(v) == c, hex(c)


def test_saturation_and_sign_of_zero(orc):
    for v, c in [(448.0, 0x7E), (464.0, 0x7E), (1e30, 0x7E), (-1e30, 0xFE), (-0.0, 0x80),
                 (0.0, 0x00), (-1e-30, 0x80), (2.0 ** -10, 0x00), (-(2.0 ** -10), 0x80),
                 (3 * 2.0 ** -10, 0x02), (15 * 2.0 ** -10, 0x08)]:
        assert orc.e4m3fn_encode(v) == c, (v, hex(orc.e4m3fn_encode(v)))
        assert orc.e4m3fn_encode_search(v) == c, v


@pytest.mark.slow
def test_encoders_agree_on_every_finite_binary32(orc):
    # both signs of every pattern 0x00000000 .. 0x7F7FFFFF (all finite binary32)
    bad, first = orc.encoder_mismatches(0, 0x7F7FFFFF)
    assert bad == 0, hex(first)


def test_encoder_matches_torch_cast_in_range(orc):
    rng = np.random.default_rng(1)
    # random binary32 bit patterns restricted to |v| <= 448 ...
    bits = rng.integers(0, 0x43E00000 + 1, size=4_000_000, dtype=np.uint32)
    bits |= (rng.integers(0, 2, size=bits.shape, dtype=np.uint32) << 31)
    v = bits.view(np.float32)
    # ... plus every BF16 value in range and every exact midpoint of the grid
    b = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    bv = b.view(np.float32)
    bv = bv[np.isfinite(bv) & (np.abs(bv) <= 448)]
    tab = orc.e4m3fn_table()[:127]
    mids = ((tab[:-1] + tab[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, bv, mids, -mids])
    ours = orc.e4m3fn_encode_array(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref), np.flatnonzero(ours != ref)[:10]


def test_bf16_helpers(orc):
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 0x7F000000, size=200_000, dtype=np.uint32)
    # include exact ties (low 16 bits = 0x8000) with both parities of bit 16
    bits[:1000] = (bits[:1000] & 0xFFFF0000) | 0x8000
    v = bits.view(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([orc.f32_to_bf16(float(x)) for x in v[:20000]], dtype=np.uint16)
    assert np.array_equal(ours, ref[:20000])
    for h in (0x0000, 0x8000, 0x3F80, 0x4078, 0x46FB, 0x7F7F, 0x0001):
        assert orc.bf16_to_f32(h) == float(np.uint32(h << 16).view(np.float32))
