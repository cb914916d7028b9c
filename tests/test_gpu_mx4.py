"""GPU parity of the MXFP4 path against the oracle.

MXFP4 = E2M1 elements (two per byte, lower index in the low nibble) with one
E8M0 scale per 32 elements along K (TeleFuser "Quantization", converter
section; OCP MX v1.0 block rule, as the oracle states).  Quantisation: packed
codes and scale bytes bit for bit.  GEMM: BF16 outputs within
2^-7 |y_ref| + 1e-3 max_row|y_ref| of the oracle's binary64 sum over the
same codes.  Inputs vary their magnitude from one 32-block to the next, so a
scale applied to the wrong block fails the check.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from gpu_util import (assert_fp8_tolerance, dev_bf16, dev_u8, every_bf16_blocks, host_bits,
                      mx_grouped, mx_ungrouped, needs_gpu, say)

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module")
def tfq():
    import int8_w8a8_quantized_amd as m

    return m


def _blocky(rng, rows, cols, sigma=1.0, spread=6):
    x = rng.standard_normal((rows, cols)) * sigma
    gain = np.exp2(rng.integers(-spread, spread + 1, (rows, cols // 32))).repeat(32, axis=1)
    x = x * gain
    x[rng.random((rows, cols)) < 0.01] *= 16
    return synth.to_bf16_bits(x.astype(np.float32))


def test_quantize_mxfp4_every_bf16_value(tfq):
    """Every finite BF16 value, both signs, through the quantiser under the
    shared exponents -127 (the E8M0 byte 0), -126, -20, -1, 0, 1, 20 and
    125: codes and scale bytes bit for bit against the oracle (this pins the
    hardware's scaled E2M1 conversion, saturation and ties included)."""
    xb = every_bf16_blocks(2, [-127, -126, -20, -1, 0, 1, 20, 125])
    say(f"mxfp4 every bf16 value rows={xb.shape[0]} cols={xb.shape[1]}")
    q, s = tfq.tfq_quantize_mxfp4(dev_bf16(xb))
    torch.cuda.synchronize()
    q_e, s_e = orc.quantize_mx4(xb)
    assert np.array_equal(mx_ungrouped(host_bits(s)), s_e)
    assert np.array_equal(host_bits(q), q_e)


@pytest.mark.parametrize("rows,cols", [(1, 128), (300, 1152), (7, 13824), (64, 8192 + 128)])
def test_quantize_mxfp4_bit_exact(tfq, rows, cols):
    rng = np.random.default_rng(rows * 37 + cols)
    xb = _blocky(rng, rows, cols)
    say(f"quantize_mxfp4 rows={rows} cols={cols}")
    q, s = tfq.tfq_quantize_mxfp4(dev_bf16(xb))
    torch.cuda.synchronize()
    qe, se = orc.quantize_mx4(xb)
    assert np.array_equal(mx_ungrouped(host_bits(s)), se)
    assert np.array_equal(host_bits(q), qe)


def test_quantize_mxfp4_special_values_and_stride(tfq):
    """Ties at every grid midpoint, saturation, zero / signed-zero, subnormal
    and huge blocks, through a row stride larger than the row."""
    rng = np.random.default_rng(3)
    rows, cols, ld = 40, 384, 512
    x = rng.standard_normal((rows, ld)).astype(np.float32)
    x[0, :32] = 0.0
    x[1, :32] = -0.0
    x[2, :32] = np.float32(2.0 ** -130) * rng.integers(-3, 4, 32)
    x[3, :32] = rng.standard_normal(32) * 2.0 ** 120
    # amax 6 (X = 1): every midpoint of the E2M1 grid and both signs
    mids = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.9, 0.1]
    x[4, :20] = mids + [-m for m in mids]
    x[5, :4] = [7.5, 7.0, -6.5, 1.0]
    x[6] *= 2.0 ** -126
    xb = synth.to_bf16_bits(x)
    xd = dev_bf16(xb)[:, :cols]
    say(f"quantize_mxfp4 special rows={rows} cols={cols} ld={ld}")
    q, s = tfq.tfq_quantize_mxfp4(xd)
    torch.cuda.synchronize()
    qe, se = orc.quantize_mx4(xb[:, :cols])
    assert np.array_equal(mx_ungrouped(host_bits(s)), se)
    assert np.array_equal(host_bits(q), qe)


def _operands(seed, M, N, K):
    rng = np.random.default_rng(seed)
    xb = _blocky(rng, M, K)
    wb = _blocky(rng, N, K, sigma=0.02, spread=3)
    qa, sa = orc.quantize_mx4(xb)
    qb, sb = orc.quantize_mx4(wb)
    bias = synth.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    return xb, wb, qa, sa, qb, sb, bias


@pytest.mark.parametrize("M,N,K", [(1, 8, 128), (300, 520, 384), (257, 264, 1152), (513, 768, 2048),
                                   (64, 2048, 256), (130, 136, 640),
                                   (258, 136, 640), (259, 264, 384)])
def test_mxfp4_gemm(tfq, M, N, K):
    _, _, qa, sa, qb, sb, bias = _operands(M + 3 * N + K, M, N, K)
    a, b = dev_u8(qa), dev_u8(qb)
    sad, sbd = dev_u8(mx_grouped(sa)), dev_u8(mx_grouped(sb))
    for use_bias, epi in [(False, None), (True, None), (True, "gelu_tanh")]:
        say(f"scaled_mm_mxfp4 M={M} N={N} K={K} bias={use_bias} epi={epi}")
        y = tfq.tfq_scaled_mm_mxfp4(a, sad, b, sbd, dev_bf16(bias) if use_bias else None, epi)
        torch.cuda.synchronize()
        ref = orc.linear_mx4_ref(qa, sa, qb, sb, bias=bias if use_bias else None,
                                 gelu=epi is not None)
        assert_fp8_tolerance(host_bits(y), ref, f"mx4 M={M} N={N} K={K} bias={use_bias} epi={epi}")


def test_mxfp4_single_block_scales(tfq):
    """Each activation row has one non-zero 32-element block: a scale taken
    from the wrong block, row or operand shows up as a wrong power of two."""
    M, N, K = 256, 256, 512
    rng = np.random.default_rng(21)
    codes = np.zeros((M, K), np.uint8)
    kb_a = rng.integers(0, K // 32, M)
    for m in range(M):
        codes[m, kb_a[m] * 32:(kb_a[m] + 1) * 32] = rng.integers(1, 8, 32) | (rng.integers(0, 2, 32) << 3)
    qa = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    cb = rng.integers(0, 16, (N, K)).astype(np.uint8)
    qb = (cb[:, 0::2] | (cb[:, 1::2] << 4)).astype(np.uint8)
    sa = rng.integers(110, 140, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(110, 140, (N, K // 32)).astype(np.uint8)
    say(f"scaled_mm_mxfp4 single-block M={M} N={N} K={K}")
    y = tfq.tfq_scaled_mm_mxfp4(dev_u8(qa), dev_u8(mx_grouped(sa)), dev_u8(qb), dev_u8(mx_grouped(sb)))
    torch.cuda.synchronize()
    ref = orc.linear_mx4_ref(qa, sa, qb, sb)
    assert_fp8_tolerance(host_bits(y), ref, "mx4 single-block")


def test_mxfp4_quantize_then_gemm_end_to_end(tfq):
    M, N, K = 333, 264, 640
    xb, wb, _, _, _, _, bias = _operands(17, M, N, K)
    say(f"mx4 end-to-end M={M} N={N} K={K}")
    qa, sa = tfq.tfq_quantize_mxfp4(dev_bf16(xb))
    qb, sb = tfq.tfq_quantize_mxfp4(dev_bf16(wb))
    y = tfq.tfq_scaled_mm_mxfp4(qa, sa, qb, sb, dev_bf16(bias), "gelu_tanh")
    torch.cuda.synchronize()
    qa_e, sa_e = orc.quantize_mx4(xb)
    qb_e, sb_e = orc.quantize_mx4(wb)
    assert np.array_equal(host_bits(qa), qa_e) and np.array_equal(mx_ungrouped(host_bits(sa)), sa_e)
    assert np.array_equal(host_bits(qb), qb_e) and np.array_equal(mx_ungrouped(host_bits(sb)), sb_e)
    ref = orc.linear_mx4_ref(qa_e, sa_e, qb_e, sb_e, bias=bias, gelu=True)
    assert_fp8_tolerance(host_bits(y), ref, "mx4 end-to-end")


def test_mxfp4_big_shape_sampled_rows(tfq):
    M, N, K = 4100, 4104, 1280
    _, _, qa, sa, qb, sb, _ = _operands(99, M, N, K)
    say(f"scaled_mm_mxfp4 big M={M} N={N} K={K}")
    y = tfq.tfq_scaled_mm_mxfp4(dev_u8(qa), dev_u8(mx_grouped(sa)), dev_u8(qb), dev_u8(mx_grouped(sb)))
    torch.cuda.synchronize()
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(M - 8, M),
                                     rng.choice(np.arange(8, M - 8), 16, replace=False)]))
    ref = orc.linear_mx4_ref(qa, sa, qb, sb, rows=rows)
    assert_fp8_tolerance(host_bits(y)[rows], ref, "mx4 big")


@pytest.mark.parametrize("qtype", ["mxfp8", "mxfp4"])
def test_quant_linear_mx_modes(tfq, qtype):
    """QuantLinear in the MX modes equals quantise + GEMM through the entry
    points, and keeps its quantised weight."""
    M, N, K = 200, 264, 512
    rng = np.random.default_rng(4)
    xb = _blocky(rng, M, K)
    wb = _blocky(rng, N, K, sigma=0.02, spread=3)
    bias = synth.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    say(f"QuantLinear {qtype} M={M} N={N} K={K}")
    lin = tfq.QuantLinear(dev_bf16(wb), dev_bf16(bias), qtype=qtype, epi="gelu_tanh")
    y1 = lin(dev_bf16(xb))
    wq = lin.w_q
    y2 = lin(dev_bf16(xb))
    quant = tfq.tfq_quantize_mx if qtype == "mxfp8" else tfq.tfq_quantize_mxfp4
    mm = tfq.tfq_scaled_mm_mxfp8 if qtype == "mxfp8" else tfq.tfq_scaled_mm_mxfp4
    qa, sa = quant(dev_bf16(xb))
    qb, sb = quant(dev_bf16(wb))
    y3 = mm(qa, sa, qb, sb, dev_bf16(bias), "gelu_tanh")
    torch.cuda.synchronize()
    assert lin.w_q is wq
    assert torch.equal(y1, y2) and torch.equal(y1, y3)


def test_mxfp4_tuned_config_same_bits(tfq):
    """The tuned launch configuration of an MXFP4 GEMM gives the default
    configuration's bits and is recorded under the MXFP4 kind."""
    M, N, K = 700, 1024, 1024
    _, _, qa, sa, qb, sb, bias = _operands(31, M, N, K)
    a, b = dev_u8(qa), dev_u8(qb)
    sad, sbd = dev_u8(mx_grouped(sa)), dev_u8(mx_grouped(sb))
    say(f"autotune mxfp4 M={M} N={N} K={K}")
    y0 = tfq.tfq_scaled_mm_mxfp4(a, sad, b, sbd, dev_bf16(bias), "gelu_tanh")
    tfq.tfq_autotune_clear()
    try:
        tfq.tfq_set_autotune(1)
        y1 = tfq.tfq_scaled_mm_mxfp4(a, sad, b, sbd, dev_bf16(bias), "gelu_tanh")
        y2 = tfq.tfq_scaled_mm_mxfp4(a, sad, b, sbd, dev_bf16(bias), "gelu_tanh")
        torch.cuda.synchronize()
        cfg = tfq.tfq_autotune_lookup("mxfp4", M, N, K, "gelu_tanh")
    finally:
        tfq.tfq_set_autotune(0)
        tfq.tfq_autotune_clear()
    assert torch.equal(y0, y1) and torch.equal(y0, y2)
    assert cfg is not None and cfg[0] == 0 and cfg[1] in (1, 2, 4, 8)
