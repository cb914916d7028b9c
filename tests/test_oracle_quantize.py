"""Pins of the oracle's dynamic absmax quantisers.

TeleFuser "Quantization": "Core ideas" gives s = max|x|/127,
q = clamp(round(x/s), -128, 127); "Scaled FP8 checkpoints: W8A8" gives
s = max|x| / max(E4M3FN), q = cast_E4M3FN(clamp(x/s)); "tf-kernel FP8: online
W8A8" applies it per token.  LightX2V "模型量化技术", "MiniMax-H3 FP8 FP16 累加",
uses scale = max(abs(x))/qmax with reduced qmax 14 / 12 / 7.

Pins: hand-worked rows (tests/golden/quantize_worked.txt); exact rational
brute force on small rows, including rows picked because a reciprocal-multiply
shortcut would change their codes; invariants on the synthetic workloads; the
exhaustive amax sweep; group and block modes reducing to the row mode.
"""
import numpy as np
import pytest
import torch

import synth
from exact_ref import quantize_row_exact
from golden_io import quantize_worked

QMAX_CODE = {448.0: 0x7E, 14.0: 0x56, 12.0: 0x54, 7.0: 0x4E}


def _bf16(vals):
    return synth.to_bf16_bits(np.array(vals, dtype=np.float32))


@pytest.mark.parametrize("case", quantize_worked(), ids=lambda c: c["name"])
def test_worked_examples(orc, case):
    x = _bf16(case["x"]).reshape(1, -1)
    # the fixture values are exact in BF16 (including the sign of zero)
    assert np.array_equal(orc.bf16_bits_to_f64(x).ravel(), np.array(case["x"]))
    assert np.array_equal(np.signbit(orc.bf16_bits_to_f64(x).ravel()),
                          np.signbit(np.array(case["x"])))
    q, s = orc.quantize_rows(x, case["qtype"], case["qmax"])
    assert float(s[0]) == case["scale"]
    assert list(q[0]) == case["codes"], [hex(c) for c in q[0]]


def _rows_where_reciprocal_differs(qmax, qtype, nrows=24, cols=48, seed=5):
    """Random BF16 rows in which x * RN(1/s) and RN(x/s) give different codes
    for at least one element (found with numpy float32 + torch's cast)."""
    rng = np.random.default_rng(seed)
    picked = []
    tries = 0
    while len(picked) < nrows and tries < 400:
        tries += 1
        x = synth.to_bf16_bits((rng.standard_normal((4096, cols)) *
                                np.exp2(rng.integers(-20, 20, (4096, 1)))).astype(np.float32))
        xf = (x.astype(np.uint32) << 16).view(np.float32)
        amax = np.abs(xf).max(axis=1, keepdims=True)
        s = amax / np.float32(qmax)
        t_div = np.clip(xf / s, -qmax, qmax)
        t_rcp = np.clip(xf * (np.float32(1) / s), -qmax, qmax)
        if qtype == "fp8":
            cd = torch.from_numpy(t_div).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            cr = torch.from_numpy(t_rcp).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        else:
            cd, cr = np.rint(t_div), np.rint(t_rcp)
        bad = np.flatnonzero((cd != cr).any(axis=1))
        for r in bad[: nrows - len(picked)]:
            picked.append(x[r])
    assert len(picked) == nrows, "search for division-sensitive rows failed"
    return np.stack(picked)


@pytest.mark.parametrize("qtype,qmax", [("fp8", 448.0), ("fp8", 14.0), ("fp8", 7.0),
                                        ("int8", 127.0)])
def test_exact_rational_brute_force(orc, qtype, qmax):
    rng = np.random.default_rng(3)
    rows = [synth.to_bf16_bits((rng.standard_normal((6, 40)) *
                                np.exp2(rng.integers(-30, 30, (6, 1)))).astype(np.float32))]
    rows.append(_rows_where_reciprocal_differs(qmax, qtype, cols=40))
    # a row with a subnormal BF16 amax (the scale is then a binary32 subnormal)
    tiny = np.array([[1, 0x8003, 2, 0x0005, 0x8000, 0]], dtype=np.uint16)
    rows.append(np.repeat(tiny, 1, axis=0).repeat(8, axis=1)[:, :40])
    rows.append(np.zeros((1, 40), dtype=np.uint16) | np.uint16(0x8000))  # all -0
    x = np.concatenate(rows)
    q, s = orc.quantize_rows(x, qtype, qmax)
    for r in range(x.shape[0]):
        se, ce = quantize_row_exact(x[r], qtype, qmax)
        assert float(s[r]) == float(se), r
        assert list(q[r]) == ce, (r, [hex(a) for a in q[r]], [hex(a) for a in ce])


@pytest.mark.parametrize("qmax", [448.0, 14.0, 12.0, 7.0, 127.0])
def test_amax_sweep_hits_qmax_code(orc, qmax):
    """Every positive finite BF16 amax value: the amax element itself must
    land exactly on qmax's code (|q| <= qmax and max|q| = qmax)."""
    h = np.arange(1, 0x7F80, dtype=np.uint16)  # all positive finite BF16
    x = np.stack([h, h | np.uint16(0x8000)], axis=1)  # row [amax, -amax]
    qtype = "int8" if qmax == 127.0 else "fp8"
    q, s = orc.quantize_rows(x, qtype, qmax)
    if qtype == "int8":
        assert np.all(q[:, 0].view(np.int8) == 127) and np.all(q[:, 1].view(np.int8) == -127)
    else:
        assert np.all(q[:, 0] == QMAX_CODE[qmax]) and np.all(q[:, 1] == (QMAX_CODE[qmax] | 0x80))
    amax = (h.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(s, amax / np.float32(qmax))  # numpy binary32 division
    assert np.all(s > 0)


def _invariants(orc, xbits, q, s, qtype, qmax):
    xf = orc.bf16_bits_to_f64(xbits)
    tab = orc.e4m3fn_table()
    vals = tab[q] if qtype == "fp8" else q.view(np.int8).astype(np.float64)
    amax = np.abs(xf).max(axis=1)
    # s == RN(amax / qmax) in binary32
    assert np.array_equal(s, (amax.astype(np.float32) / np.float32(qmax)))
    assert np.all(np.abs(vals) <= qmax)
    nz = amax > 0
    assert np.all(np.abs(vals[nz]).max(axis=1) == qmax)
    # sign(q) == sign(x) where q != 0
    m = vals != 0
    assert np.all(np.sign(vals[m]) == np.sign(xf[m]))
    # dequantisation error bound: half a grid step of the code's binade
    sd = s.astype(np.float64)[:, None]
    err = np.abs(xf - sd * vals)
    if qtype == "int8":
        bound = sd * (0.5 + 2.0 ** -16)
    else:
        t = np.abs(xf) / np.where(sd > 0, sd, 1)
        step = np.where(t < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(t, 2.0 ** -6))) - 3))
        bound = sd * step / 2 * (1 + 2.0 ** -16)
    assert np.all(err <= bound + 1e-300)


@pytest.mark.parametrize("name,kw", [("c1_tiny_fp8", {}), ("c2_int8", dict(M=256, K=384, N=64)),
                                     ("c3_image_dit", dict(M=200, N=64)),
                                     ("c4_video_dit", dict(M=96, K=512, N=64, n_down=32))])
def test_invariants_on_workload_inputs(orc, name, kw):
    d = synth.make(name, **kw)
    wl = d["spec"]
    for qmax in wl.act_qmax:
        q, s = orc.quantize_rows(d["x"], wl.qtype, qmax)
        _invariants(orc, d["x"], q, s, wl.qtype, qmax)
    qw, sw = orc.quantize_rows(d["w"], wl.qtype, wl.w_qmax)
    _invariants(orc, d["w"], qw, sw, wl.qtype, wl.w_qmax)


def test_group_mode_is_row_mode_per_slice(orc):
    d = synth.make("c5_block_fp8", M=64, K=640, N=128)
    q, s = orc.quantize_rows(d["x"], "fp8", 448.0, group=128)
    assert s.shape == (64, 5)
    for g in range(5):
        qg, sg = orc.quantize_rows(np.ascontiguousarray(d["x"][:, g * 128:(g + 1) * 128]), "fp8", 448.0)
        assert np.array_equal(q[:, g * 128:(g + 1) * 128], qg)
        assert np.array_equal(s[:, g], sg)
    # with one group spanning the row, group mode is row mode exactly
    q1, s1 = orc.quantize_rows(d["x"][:, :128].copy(), "fp8", 448.0, group=128)
    q0, s0 = orc.quantize_rows(d["x"][:, :128].copy(), "fp8", 448.0)
    assert np.array_equal(q1, q0) and np.array_equal(s1[:, 0], s0)


def test_block_mode_reduces_to_per_channel(orc):
    """When every row of a 128-row band has the same absmax in every 128-col
    block, the 128x128 block scales equal the per-channel scales and the codes
    agree bit for bit."""
    rng = np.random.default_rng(7)
    n, k = 256, 384
    w = np.clip((rng.standard_normal((n, k)) * 0.02).astype(np.float32), -0.05, 0.05)
    r = np.arange(n)
    for kb in range(k // 128):
        # row r of band b gets +-peak(b, kb) once inside column block kb; every
        # other entry is below 0.05 < peak, so row and block absmax coincide
        peak = (0.0625 * (1 + r // 128 + 2 * kb)).astype(np.float32)
        w[r, kb * 128 + (r * 37) % 128] = peak * np.where(r % 2, 1, -1)
    wb = synth.to_bf16_bits(w)
    qb, sb = orc.quantize_blocks(wb, "fp8", 448.0, 128)
    # per-channel, per 128-column slice
    for kb in range(k // 128):
        sl = np.ascontiguousarray(wb[:, kb * 128:(kb + 1) * 128])
        qc, sc = orc.quantize_rows(sl, "fp8", 448.0)
        assert np.array_equal(qb[:, kb * 128:(kb + 1) * 128], qc)
        assert np.array_equal(np.repeat(sb[:, kb], 128), sc)


def test_block_scales_are_block_absmax(orc):
    d = synth.make("c5_block_fp8", M=8, K=256, N=384)
    q, s = orc.quantize_blocks(d["w"], "fp8", 448.0, 128)
    wf = orc.bf16_bits_to_f64(d["w"])
    for i in range(3):
        for j in range(2):
            amax = np.abs(wf[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]).max()
            assert s[i, j] == np.float32(amax) / np.float32(448.0)
            blk = q[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            assert np.any((blk & 0x7F) == 0x7E)
