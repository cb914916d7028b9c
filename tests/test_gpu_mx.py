"""GPU parity of the MXFP8 path against the oracle.

MXFP8 = E4M3FN elements with one E8M0 scale per 32 consecutive elements along
K (TeleFuser "Quantization", converter section; block rule of the OCP MX v1.0
format, as the oracle states).  Quantisation: codes and scale bytes bit for
bit.  GEMM: BF16 outputs within 2^-7 |y_ref| + 1e-3 max_row|y_ref| of the
oracle's binary64 sum over the same quantised operands.  Inputs vary their
magnitude from one 32-block to the next, so a scale applied to the wrong
block fails the check.  The oracle keeps scales as [rows, cols/32]; the
library stores them as [cols/128, rows, 4] (the four block scales of a
128-wide K group together, in the byte order 0, 2, 1, 3, group-major):
`grouped` and `ungrouped` convert.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from gpu_util import (assert_fp8_tolerance, dev_bf16, dev_u8, host_bits, mx_grouped,
                      mx_ungrouped, needs_gpu, say)

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module")
def tfq():
    import int8_w8a8_quantized_amd as m

    return m


grouped, ungrouped = mx_grouped, mx_ungrouped


def _blocky(rng, rows, cols, sigma=1.0, spread=6):
    """Normal values with a random power-of-two gain per 32-element block."""
    x = rng.standard_normal((rows, cols)) * sigma
    gain = np.exp2(rng.integers(-spread, spread + 1, (rows, cols // 32))).repeat(32, axis=1)
    x = x * gain
    x[rng.random((rows, cols)) < 0.01] *= 16
    return synth.to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("rows,cols", [(1, 128), (300, 1152), (7, 13824), (64, 8192 + 128)])
def test_quantize_mx_bit_exact(tfq, rows, cols):
    rng = np.random.default_rng(rows * 31 + cols)
    xb = _blocky(rng, rows, cols)
    say(f"quantize_mx rows={rows} cols={cols}")
    q, s = tfq.tfq_quantize_mx(dev_bf16(xb))
    torch.cuda.synchronize()
    qe, se = orc.quantize_mx(xb)
    assert np.array_equal(ungrouped(host_bits(s)), se)
    assert np.array_equal(host_bits(q), qe)


def test_quantize_mx_special_blocks_and_stride(tfq):
    """Zero and signed-zero blocks, BF16 subnormals (scale byte 0), huge
    magnitudes, values that saturate at 448 and ties, read through a row
    stride larger than the row."""
    rng = np.random.default_rng(3)
    rows, cols, ld = 40, 384, 512
    x = rng.standard_normal((rows, ld)).astype(np.float32)
    x[0, :32] = 0.0
    x[1, :32] = -0.0
    x[2, :32] = np.float32(2.0 ** -130) * rng.integers(-3, 4, 32)
    x[3, :32] = rng.standard_normal(32) * 2.0 ** 120
    x[4, :4] = [7.5, 7.0, -6.5, 1.0]
    x[5, :4] = [1.0, 17 / 256, 19 / 256, -17 / 256]
    x[6] *= 2.0 ** -126
    xb = synth.to_bf16_bits(x)
    xd = dev_bf16(xb)[:, :cols]
    assert xd.stride(0) == ld
    say(f"quantize_mx special rows={rows} cols={cols} ld={ld}")
    q, s = tfq.tfq_quantize_mx(xd)
    torch.cuda.synchronize()
    qe, se = orc.quantize_mx(xb[:, :cols])
    assert np.array_equal(ungrouped(host_bits(s)), se)
    assert np.array_equal(host_bits(q), qe)


def _mx_operands(seed, M, N, K):
    rng = np.random.default_rng(seed)
    xb = _blocky(rng, M, K)
    wb = _blocky(rng, N, K, sigma=0.02, spread=3)
    qa, sa = orc.quantize_mx(xb)
    qb, sb = orc.quantize_mx(wb)
    bias = synth.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    return xb, wb, qa, sa, qb, sb, bias


@pytest.mark.parametrize("M,N,K", [(1, 8, 128), (300, 520, 384), (257, 264, 1152), (513, 768, 2048),
                                   (64, 2048, 256),
                                   (258, 136, 640), (259, 264, 384)])
def test_mxfp8_gemm(tfq, M, N, K):
    _, _, qa, sa, qb, sb, bias = _mx_operands(M + 2 * N + K, M, N, K)
    a, b, sad, sbd = dev_u8(qa), dev_u8(qb), dev_u8(grouped(sa)), dev_u8(grouped(sb))
    for use_bias, epi in [(False, None), (True, None), (True, "gelu_tanh")]:
        say(f"scaled_mm_mxfp8 M={M} N={N} K={K} bias={use_bias} epi={epi}")
        y = tfq.tfq_scaled_mm_mxfp8(a, sad, b, sbd, dev_bf16(bias) if use_bias else None, epi)
        torch.cuda.synchronize()
        ref = orc.linear_mx_ref(qa, sa, qb, sb, bias=bias if use_bias else None,
                                gelu=epi is not None)
        assert_fp8_tolerance(host_bits(y), ref, f"mx M={M} N={N} K={K} bias={use_bias} epi={epi}")


def test_mxfp8_single_block_scales(tfq):
    """Each activation row has one non-zero K block: its outputs are that
    block's dot times 2^(ea + eb - 254), so a scale taken from the wrong block,
    row or operand shows up as a wrong power of two."""
    M, N, K = 256, 256, 512
    rng = np.random.default_rng(21)
    qa = np.zeros((M, K), np.uint8)
    qb = np.zeros((N, K), np.uint8)
    kb_a = rng.integers(0, K // 32, M)
    for m in range(M):
        qa[m, kb_a[m] * 32:(kb_a[m] + 1) * 32] = rng.integers(0x30, 0x50, 32)
    qb[:] = rng.integers(0x30, 0x50, (N, K)) | (rng.integers(0, 2, (N, K)) << 7)
    sa = rng.integers(110, 140, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(110, 140, (N, K // 32)).astype(np.uint8)
    say(f"scaled_mm_mxfp8 single-block M={M} N={N} K={K}")
    y = tfq.tfq_scaled_mm_mxfp8(dev_u8(qa), dev_u8(grouped(sa)), dev_u8(qb), dev_u8(grouped(sb)))
    torch.cuda.synchronize()
    ref = orc.linear_mx_ref(qa, sa, qb, sb)
    assert_fp8_tolerance(host_bits(y), ref, "mx single-block")


def test_mxfp8_quantize_then_gemm_end_to_end(tfq):
    """Activations and weights quantised on the GPU (bit-exact with the
    oracle), then the MXFP8 GEMM with bias and GELU."""
    M, N, K = 333, 264, 640
    xb, wb, _, _, _, _, bias = _mx_operands(17, M, N, K)
    say(f"mx end-to-end M={M} N={N} K={K}")
    qa, sa = tfq.tfq_quantize_mx(dev_bf16(xb))
    qb, sb = tfq.tfq_quantize_mx(dev_bf16(wb))
    y = tfq.tfq_scaled_mm_mxfp8(qa, sa, qb, sb, dev_bf16(bias), "gelu_tanh")
    torch.cuda.synchronize()
    qa_e, sa_e = orc.quantize_mx(xb)
    qb_e, sb_e = orc.quantize_mx(wb)
    assert np.array_equal(host_bits(qa), qa_e) and np.array_equal(ungrouped(host_bits(sa)), sa_e)
    assert np.array_equal(host_bits(qb), qb_e) and np.array_equal(ungrouped(host_bits(sb)), sb_e)
    ref = orc.linear_mx_ref(qa_e, sa_e, qb_e, sb_e, bias=bias, gelu=True)
    assert_fp8_tolerance(host_bits(y), ref, "mx end-to-end")


def test_mxfp8_big_shape_sampled_rows(tfq):
    """More 256x256 tiles than CUs with ragged M and N tails; sampled rows
    against the oracle."""
    M, N, K = 4100, 4104, 1280
    _, _, qa, sa, qb, sb, _ = _mx_operands(99, M, N, K)
    say(f"scaled_mm_mxfp8 big M={M} N={N} K={K}")
    y = tfq.tfq_scaled_mm_mxfp8(dev_u8(qa), dev_u8(grouped(sa)), dev_u8(qb), dev_u8(grouped(sb)))
    torch.cuda.synchronize()
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(M - 8, M),
                                     rng.choice(np.arange(8, M - 8), 16, replace=False)]))
    ref = orc.linear_mx_ref(qa, sa, qb, sb, rows=rows)
    assert_fp8_tolerance(host_bits(y)[rows], ref, "mx big")
