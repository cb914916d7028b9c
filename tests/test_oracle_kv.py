"""Pins for the oracle's FP8 KV cache (CPU only).

TeleFuser "Quantization", "Other quantized data paths" (LiveAct FP8 KV
cache): K/V stored as E4M3FN with one FP32 scale per last-dimension vector,
dequantised to the attention's dtype on load.  Store: against the exact
rational quantisation of each vector (tests/exact_ref.py) and the slot
rules.  Load: every finite code times a spread of scales against the exact
product rounded once to binary32 (exact_ref) and converted by torch.  The
round trip stays within half an E4M3 step.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import exact_ref
import oracle as orc
import synth

pytestmark = pytest.mark.filterwarnings("ignore")


def _kv(rng, T, H, D):
    x = rng.standard_normal((T, H, D)).astype(np.float32) * np.exp2(rng.integers(-8, 8, (T, H, 1)))
    x[rng.random(x.shape) < 0.02] *= 25
    return synth.to_bf16_bits(x.astype(np.float32))


def test_store_vectors_match_exact_quantisation():
    rng = np.random.default_rng(1)
    T, H, D = 3, 4, 64
    kv = _kv(rng, T, H, D)
    kv[1, 2] = 0            # an all-zero vector
    slots = 8
    cache = np.zeros((slots, H, D), np.uint8)
    scale = np.zeros((slots, H), np.float32)
    slot = np.array([5, 0, 2])
    orc.kv_store(kv, slot, cache, scale)
    for t in range(T):
        for h in range(H):
            s_e, q_e = exact_ref.quantize_row_exact([int(b) for b in kv[t, h]], "fp8", 448.0)
            assert Fraction(float(scale[slot[t], h])) == s_e
            assert cache[slot[t], h].tolist() == q_e


def test_store_slot_rules():
    rng = np.random.default_rng(2)
    T, H, D = 6, 2, 32
    kv = _kv(rng, T, H, D)
    cache = np.full((4, H, D), 0xAB, np.uint8)
    scale = np.full((4, H), -1.0, np.float32)
    slot = np.array([3, -1, 4, 1, 2**31 - 1, -2**31])
    orc.kv_store(kv, slot, cache, scale)
    assert (cache[0] == 0xAB).all() and (scale[0] == -1).all()       # never named
    assert (cache[[1, 3]] != 0xAB).any() and (scale[[1, 3]] > 0).all()
    assert (cache[2] == 0xAB).all()
    q, s = orc.quantize_rows(kv[3], "fp8", 448.0)
    assert np.array_equal(cache[1], q) and np.array_equal(scale[1], s)


@pytest.mark.parametrize("out", ["fp32", "bf16", "fp16"])
def test_load_every_code_against_exact_product(out):
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    D = codes.size
    scales = np.array([1.0, 448.0 ** -1, 3.0517578e-05, 0.013671875, 7.1e-3, 2.0 ** -126,
                       1.1754944e-38 * 3, 1e30, 0.333333343], np.float32)
    cache = np.broadcast_to(codes, (scales.size, 1, D)).copy()
    y = orc.kv_load(cache, scales[:, None], np.arange(scales.size), out)
    for i, s in enumerate(scales):
        exact = [exact_ref.round_to_binary32(Fraction(float(s)) * Fraction(orc.e4m3fn_value(int(c))))
                 for c in codes]
        # a zero product keeps the IEEE sign: code 0x80 is -0
        f32 = np.array([float(e) if e != 0 else (-0.0 if c & 0x80 else 0.0)
                        for e, c in zip(exact, codes)], np.float32)
        if out == "fp32":
            want = f32.view(np.uint32)
            got = y[i, 0].view(np.uint32)
        elif out == "bf16":
            want = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            got = y[i, 0]
        else:
            want = torch.from_numpy(f32).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
            got = y[i, 0]
        assert np.array_equal(got, want), (out, float(s))


def test_load_gathers_rows_and_zero_fills_out_of_range():
    rng = np.random.default_rng(3)
    S, H, D = 5, 3, 16
    cache = rng.integers(0, 0x7F, (S, H, D)).astype(np.uint8)
    scale = rng.random((S, H)).astype(np.float32)
    full = orc.kv_load(cache, scale, np.arange(S), "fp32")
    idx = np.array([4, -1, 0, 5, 4, 2**31 - 1])
    y = orc.kv_load(cache, scale, idx, "fp32")
    assert np.array_equal(y[0], full[4]) and np.array_equal(y[2], full[0])
    assert np.array_equal(y[4], full[4])
    assert not y[[1, 3, 5]].any()


def test_round_trip_within_half_a_step():
    rng = np.random.default_rng(4)
    T, H, D = 16, 8, 128
    kv = _kv(rng, T, H, D)
    cache = np.zeros((T, H, D), np.uint8)
    scale = np.zeros((T, H), np.float32)
    orc.kv_store(kv, np.arange(T), cache, scale)
    back = orc.kv_load(cache, scale, np.arange(T), "fp32").astype(np.float64)
    x = orc.bf16_bits_to_f64(kv)
    s = scale.astype(np.float64)[:, :, None]
    t = np.abs(x) / np.where(s > 0, s, 1)
    step = np.exp2(np.floor(np.log2(np.maximum(t, 2.0 ** -6))) - 3)
    # half a step of the code grid, plus the binary32 roundings of x/s and s*q
    assert (np.abs(back - x) <= (step / 2) * s * (1 + 2.0 ** -20) + np.abs(x) * 2.0 ** -22).all()
