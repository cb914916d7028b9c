"""Pins of the oracle's scaled-GEMM references.

The Linear output is the product of the dequantised operands, x_hat = s q
(TeleFuser "Quantization", "Core ideas"), so y[m, n] = s_row[m] s_col[n]
sum_k q_x[m,k] q_w[n,k]; tf_kernel.fp8_scaled_mm returns BF16 ("tf-kernel
FP8: online W8A8").  Block-scaled FP8 (LightX2V "模型量化技术", table "量化模式",
fp8-b128-deepgemm; vLLM-Omni "FP8 Quantization", "Parameters",
weight_block_size) applies one scale per K-block.

Pins: hand-worked outputs (tests/golden/gemm_worked.txt); integer brute force
on tiny shapes (E4M3FN values times 2^9 are integers); numpy binary64 matmul
of independently decoded operands (torch's float8 decode) on non-square
shapes, which fails for a transposed or mis-indexed operand; block mode
reducing to the row mode; GELU-tanh against torch and its odd-part identity;
the fixed INT8 BF16 epilogue against numpy binary32 steps; E_max / E_rel on
known vectors.
"""
import math

import numpy as np
import pytest
import torch

import synth
from golden_io import gemm_worked


def _torch_decode(codes: np.ndarray, qtype: str) -> np.ndarray:
    if qtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(
            torch.float64).numpy()
    return np.ascontiguousarray(codes).view(np.int8).astype(np.float64)


@pytest.mark.parametrize("case", gemm_worked(), ids=lambda c: c["name"])
def test_worked_examples(orc, case):
    qmax = 448.0 if case["qtype"] == "fp8" else 127.0
    x = synth.to_bf16_bits(np.array([case["x"]], dtype=np.float32))
    w = synth.to_bf16_bits(np.array([case["w"]], dtype=np.float32))
    qx, sx = orc.quantize_rows(x, case["qtype"], qmax)
    qw, sw = orc.quantize_rows(w, case["qtype"], qmax)
    assert float(sx[0]) == case["sx"] and float(sw[0]) == case["sw"]
    assert list(qx[0]) == case["xcodes"] and list(qw[0]) == case["wcodes"]
    assert orc.dot(qx, qw, case["qtype"])[0, 0] == case["dot"]
    y = orc.linear_ref(qx, sx, qw, sw, case["qtype"])
    assert y[0, 0] == case["y"]
    assert orc.f32_to_bf16(float(y[0, 0])) == case["ybits"]
    if case["qtype"] == "int8":
        acc, yb = orc.int8_linear(qx, sx, qw, sw)
        assert acc[0, 0] == case["dot"] and yb[0, 0] == case["ybits"]


def _random_codes(rng, shape, qtype):
    if qtype == "fp8":
        c = rng.integers(0, 256, size=shape, dtype=np.uint8)
        c[(c & 0x7F) == 0x7F] = 0x7E  # no NaN codes
        return c
    return rng.integers(-128, 128, size=shape, dtype=np.int8).view(np.uint8)


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
def test_dot_integer_brute_force_tiny(orc, qtype):
    rng = np.random.default_rng(11)
    for (M, N, K) in [(1, 1, 1), (3, 5, 7), (16, 9, 256), (7, 16, 100)]:
        a = _random_codes(rng, (M, K), qtype)
        b = _random_codes(rng, (N, K), qtype)
        scale = 512 if qtype == "fp8" else 1  # E4M3FN values * 2^9 are integers
        ai = [[int(round(v * scale)) for v in row] for row in _torch_decode(a, qtype)]
        bi = [[int(round(v * scale)) for v in row] for row in _torch_decode(b, qtype)]
        got = orc.dot(a, b, qtype)
        for m in range(M):
            for n in range(N):
                exact = sum(ai[m][k] * bi[n][k] for k in range(K))
                assert got[m, n] * scale * scale == exact


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
def test_linear_matches_numpy_dequantised_product(orc, qtype):
    rng = np.random.default_rng(12)
    M, N, K = 37, 23, 160
    a = _random_codes(rng, (M, K), qtype)
    b = _random_codes(rng, (N, K), qtype)
    sa = rng.uniform(0.001, 0.1, M).astype(np.float32)
    sb = rng.uniform(0.001, 0.1, N).astype(np.float32)
    A, B = _torch_decode(a, qtype), _torch_decode(b, qtype)
    dot_np = A @ B.T  # binary64; exact by the bound on the products
    assert np.array_equal(orc.dot(a, b, qtype), dot_np)
    y_np = dot_np * sa.astype(np.float64)[:, None] * sb.astype(np.float64)[None, :]
    y = orc.linear_ref(a, sa, b, sb, qtype)
    assert np.allclose(y, y_np, rtol=1e-15, atol=0)
    # selected rows, out of order
    rows = np.array([36, 0, 5, 5, 17])
    assert np.array_equal(orc.linear_ref(a, sa, b, sb, qtype, rows=rows), y[rows])
    # bias and GELU follow the scaling
    bias = synth.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    yb = orc.linear_ref(a, sa, b, sb, qtype, bias=bias, gelu=True)
    h = y_np + orc.bf16_bits_to_f64(bias)[None, :]
    ref = torch.nn.functional.gelu(torch.from_numpy(h), approximate="tanh").numpy()
    assert np.allclose(yb, ref, rtol=1e-13, atol=1e-300)


def test_exact_dot_at_long_k(orc):
    """K = 13824 (the down projection): binary64 sums of E4M3FN products are
    exact in any order, so the oracle equals integer arithmetic."""
    rng = np.random.default_rng(13)
    K = 13824
    a = _random_codes(rng, (2, K), "fp8")
    b = _random_codes(rng, (3, K), "fp8")
    A = np.rint(_torch_decode(a, "fp8") * 512).astype(np.int64)
    B = np.rint(_torch_decode(b, "fp8") * 512).astype(np.int64)
    exact = A @ B.T  # int64, |sum| < 2^53
    got = orc.dot(a, b, "fp8")
    assert np.array_equal((got * 512 * 512).astype(np.int64), exact)
    assert np.all(np.abs(got * 262144) < 2.0 ** 53)


def test_block_mode_reduces_to_row_mode(orc):
    rng = np.random.default_rng(14)
    M, N, K = 9, 256, 384
    a = _random_codes(rng, (M, K), "fp8")
    b = _random_codes(rng, (N, K), "fp8")
    sa = rng.uniform(0.01, 0.1, M).astype(np.float32)
    sb = rng.uniform(0.01, 0.1, N // 128).astype(np.float32)
    # block scales constant along K reduce to per-row / per-128-channel scales
    sa_blk = np.repeat(sa[:, None], K // 128, axis=1)
    sb_blk = np.repeat(sb[:, None], K // 128, axis=1)
    yb = orc.linear_ref(a, sa_blk, b, sb_blk, "fp8", scale_block=128)
    yr = orc.linear_ref(a, sa, b, np.repeat(sb, 128), "fp8")
    # sums of per-block terms may cancel: compare on the scale of the outputs
    assert np.allclose(yb, yr, rtol=1e-13, atol=1e-13 * np.abs(yr).max())
    # general block scales: numpy per-K-block sum
    sa_g = rng.uniform(0.01, 0.1, (M, K // 128)).astype(np.float32)
    sb_g = rng.uniform(0.01, 0.1, (N // 128, K // 128)).astype(np.float32)
    A, B = _torch_decode(a, "fp8"), _torch_decode(b, "fp8")
    ref = np.zeros((M, N))
    for kb in range(K // 128):
        p = A[:, kb * 128:(kb + 1) * 128] @ B[:, kb * 128:(kb + 1) * 128].T
        ref += sa_g[:, kb].astype(np.float64)[:, None] * np.repeat(sb_g[:, kb], 128)[None, :] * p
    yg = orc.linear_ref(a, sa_g, b, sb_g, "fp8", scale_block=128)
    assert np.allclose(yg, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())


def test_gelu_tanh(orc):
    assert orc.gelu_tanh(0.0) == 0.0
    for h in (-9.0, -3.2, -1.0, -0.1, 0.37, 1.0, 2.5, 8.0):
        # odd part of the tanh form: gelu(h) - gelu(-h) = h
        assert abs(orc.gelu_tanh(h) - orc.gelu_tanh(-h) - h) <= 1e-15 * max(1.0, abs(h))
        ref = torch.nn.functional.gelu(torch.tensor(h, dtype=torch.float64), approximate="tanh")
        assert abs(orc.gelu_tanh(h) - float(ref)) <= 1e-15 * max(1.0, abs(h))
        # within the tanh approximation's distance of the erf definition
        exact = 0.5 * h * (1 + math.erf(h / math.sqrt(2)))
        assert abs(orc.gelu_tanh(h) - exact) < 1e-3
    assert abs(orc.gelu_tanh(1.0) - 0.8411919906082768) < 1e-15


def test_int8_epilogue_fixed_order(orc):
    rng = np.random.default_rng(15)
    M, N, K = 19, 33, 96
    a = _random_codes(rng, (M, K), "int8")
    b = _random_codes(rng, (N, K), "int8")
    sa = rng.uniform(0.001, 0.2, M).astype(np.float32)
    sb = rng.uniform(0.001, 0.2, N).astype(np.float32)
    acc, y = orc.int8_linear(a, sa, b, sb)
    A = a.view(np.int8).astype(np.int64)
    B = b.view(np.int8).astype(np.int64)
    assert np.array_equal(acc, A @ B.T)
    f = (A @ B.T).astype(np.float32) * sa[:, None]   # numpy binary32 steps
    f = f * sb[None, :]
    ref = synth.to_bf16_bits(f)
    assert np.array_equal(y, ref)
    bias = synth.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    _, yb = orc.int8_linear(a, sa, b, sb, bias=bias)
    fb = f + orc.bf16_bits_to_f64(bias).astype(np.float32)[None, :]
    assert np.array_equal(yb, synth.to_bf16_bits(fb))


def test_error_measures(orc):
    y = np.array([3.0, -4.0, 0.0])
    yq = np.array([3.0, -4.0, 0.5])
    emax, erel = orc.error_measures(yq, y)
    assert emax == 0.5 and erel == 0.1


def _fp8_operands(rng, M, N, K, orc, qtype="fp8", wscale=0.02):
    x = synth.to_bf16_bits((rng.standard_normal((M, K)) *
                            np.exp2(rng.integers(-8, 8, (M, 1)))).astype(np.float32))
    w = synth.to_bf16_bits((wscale * rng.standard_normal((N, K))).astype(np.float32))
    qmax = 448.0 if qtype == "fp8" else 127.0
    return orc.quantize_rows(x, qtype, qmax), orc.quantize_rows(w, qtype, qmax)


@pytest.mark.parametrize("M,N,K", [(1, 8, 16), (7, 40, 96), (33, 130, 520), (5, 24, 13824)])
@pytest.mark.parametrize("gelu", [False, True])
def test_fast_linear_ref_bit_equal_to_loop_version(orc, M, N, K, gelu):
    """The BLAS-formed reference equals the loop reference bit for bit (the
    exact-dot property), with and without bias and GELU, on all rows and on a
    row selection; K = 13 824 is the video-DiT down projection."""
    rng = np.random.default_rng(M * 1000 + K + gelu)
    (qa, sa), (qb, sb) = _fp8_operands(rng, M, N, K, orc)
    bias = synth.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    for b in (None, bias):
        ref = orc.linear_ref(qa, sa, qb, sb, "fp8", bias=b, gelu=gelu)
        fast = orc.linear_ref_fast(qa, sa, qb, sb, "fp8", bias=b, gelu=gelu)
        assert np.array_equal(ref.view(np.uint64), fast.view(np.uint64))
    rows = rng.integers(0, M, 5)
    ref = orc.linear_ref(qa, sa, qb, sb, "fp8", gelu=gelu, rows=rows)
    fast = orc.linear_ref_fast(qa, sa, qb, sb, "fp8", gelu=gelu, rows=rows)
    assert np.array_equal(ref.view(np.uint64), fast.view(np.uint64))


@pytest.mark.parametrize("M,N,K", [(3, 128, 128), (9, 256, 640)])
def test_fast_linear_ref_block_mode_bit_equal(orc, M, N, K):
    rng = np.random.default_rng(N + K)
    x = synth.to_bf16_bits((rng.standard_normal((M, K)) *
                            np.exp2(rng.integers(-6, 6, (M, K // 128)).repeat(128, 1))
                            ).astype(np.float32))
    w = synth.to_bf16_bits((0.02 * rng.standard_normal((N, K))).astype(np.float32))
    qa, sa = orc.quantize_rows(x, "fp8", 448.0, 128)
    qb, sb = orc.quantize_blocks(w, "fp8", 448.0, 128)
    bias = synth.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    for gelu in (False, True):
        ref = orc.linear_ref(qa, sa, qb, sb, "fp8", 128, bias=bias, gelu=gelu)
        fast = orc.linear_ref_fast(qa, sa, qb, sb, "fp8", 128, bias=bias, gelu=gelu)
        assert np.array_equal(ref.view(np.uint64), fast.view(np.uint64))


@pytest.mark.parametrize("M,N,K", [(4, 16, 32), (17, 72, 3072)])
def test_fast_int8_linear_equal_to_loop_version(orc, M, N, K):
    rng = np.random.default_rng(M + N + K)
    (qa, sa), (qb, sb) = _fp8_operands(rng, M, N, K, orc, "int8")
    bias = synth.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    for b in (None, bias):
        acc, y = orc.int8_linear(qa, sa, qb, sb, bias=b)
        acc_f, y_f = orc.int8_linear_fast(qa, sa, qb, sb, bias=b)
        assert np.array_equal(acc, acc_f) and np.array_equal(y, y_f)
    rows = np.array([M - 1, 0, M // 2])
    acc, y = orc.int8_linear(qa, sa, qb, sb, rows=rows)
    acc_f, y_f = orc.int8_linear_fast(qa, sa, qb, sb, rows=rows)
    assert np.array_equal(acc, acc_f) and np.array_equal(y, y_f)
    # extreme codes at the INT32 bound: K = 131056 rows of -128 / 127 sums
    qa2 = np.full((1, 131056), -128, dtype=np.int8).view(np.uint8)
    qb2 = np.full((2, 131056), -128, dtype=np.int8)
    qb2[1] = 127
    one = np.ones(1, np.float32)
    acc_f, _ = orc.int8_linear_fast(qa2, one, qb2.view(np.uint8), np.ones(2, np.float32))
    assert acc_f.tolist() == [[128 * 128 * 131056, -128 * 127 * 131056]]
