"""GPU parity of the scaled GEMMs and the fused Linear against the oracle.

FP8 BF16 outputs: max|y - y_ref| <= 2^-7 |y_ref| + 1e-3 max_row|y_ref| with
y_ref the same quantised operands summed exactly in binary64; INT8: INT32
accumulators and the fixed-order BF16 outputs bit for bit (TeleFuser
"Quantization", "tf-kernel FP8: online W8A8" and "Core ideas"; LightX2V
"模型量化技术", table "量化模式", fp8-b128-deepgemm for block mode).
Shapes span several 256x256 tiles with ragged M, N and K tails.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from gpu_util import (assert_fp8_tolerance, dev_bf16, dev_f32, dev_u8, host_bits, needs_gpu,
                      say)

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module")
def tfq():
    import int8_w8a8_quantized_amd as m

    return m


def _operands(seed, M, N, K, qtype, x_scale=1.0):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((M, K)) * x_scale).astype(np.float32)
    x[rng.random((M, K)) < 0.01] *= 20
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    xb, wb = synth.to_bf16_bits(x), synth.to_bf16_bits(w)
    qmax = 448.0 if qtype == "fp8" else 127.0
    qa, sa = orc.quantize_rows(xb, qtype, qmax)
    qb, sb = orc.quantize_rows(wb, qtype, qmax)
    bias = synth.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    return xb, wb, qa, sa, qb, sb, bias


FP8_SHAPES = [(1, 8, 16), (300, 520, 384), (257, 264, 272), (513, 768, 1024), (64, 2048, 128),
              (1000, 136, 3088)]


@pytest.mark.parametrize("M,N,K", FP8_SHAPES)
def test_fp8_gemm(tfq, M, N, K):
    _, _, qa, sa, qb, sb, bias = _operands(M + N + K, M, N, K, "fp8")
    a, b = dev_u8(qa), dev_u8(qb)
    sad, sbd = dev_f32(sa), dev_f32(sb)
    for use_bias, epi in [(False, None), (True, None), (True, "gelu_tanh"), (False, "gelu_tanh")]:
        say(f"scaled_mm_fp8 M={M} N={N} K={K} bias={use_bias} epi={epi}")
        bd = dev_bf16(bias) if use_bias else None
        y = tfq.tfq_scaled_mm_fp8(a, sad, b, sbd, 0, bd, epi)
        torch.cuda.synchronize()
        ref = orc.linear_ref(qa, sa, qb, sb, "fp8", bias=bias if use_bias else None,
                             gelu=epi is not None)
        assert_fp8_tolerance(host_bits(y), ref, f"M={M} N={N} K={K} bias={use_bias} epi={epi}")


@pytest.mark.parametrize("M,N,K", [(1, 8, 16), (300, 520, 384), (257, 264, 272), (130, 1024, 2064)])
def test_int8_gemm_bit_exact(tfq, M, N, K):
    _, _, qa, sa, qb, sb, bias = _operands(M * 3 + N + K, M, N, K, "int8")
    a, b = dev_u8(qa, torch.int8), dev_u8(qb, torch.int8)
    sad, sbd = dev_f32(sa), dev_f32(sb)
    say(f"scaled_mm_int8 M={M} N={N} K={K} y+acc")
    y, acc = tfq.tfq_scaled_mm_int8(a, sad, b, sbd, None, None, True, True)
    torch.cuda.synchronize()
    acc_e, y_e = orc.int8_linear(qa, sa, qb, sb)
    assert np.array_equal(host_bits(acc).astype(np.int64), acc_e)
    assert np.array_equal(host_bits(y), y_e)
    say(f"scaled_mm_int8 M={M} N={N} K={K} bias, y only / acc only")
    y2, _ = tfq.tfq_scaled_mm_int8(a, sad, b, sbd, dev_bf16(bias), None, True, False)
    _, acc2 = tfq.tfq_scaled_mm_int8(a, sad, b, sbd, None, None, False, True)
    torch.cuda.synchronize()
    _, y2_e = orc.int8_linear(qa, sa, qb, sb, bias=bias, want_acc=False)
    assert np.array_equal(host_bits(y2), y2_e)
    assert np.array_equal(host_bits(acc2).astype(np.int64), acc_e)
    say(f"scaled_mm_int8 M={M} N={N} K={K} gelu")
    y3, _ = tfq.tfq_scaled_mm_int8(a, sad, b, sbd, dev_bf16(bias), "gelu_tanh", True, False)
    torch.cuda.synchronize()
    ref = orc.linear_ref(qa, sa, qb, sb, "int8", bias=bias, gelu=True)
    assert_fp8_tolerance(host_bits(y3), ref, "int8 gelu")


def test_int8_extreme_accumulators(tfq):
    """All codes -128/127 at the largest K: INT32 sums near the overflow bound."""
    M, N, K = 16, 64, 131056
    say(f"scaled_mm_int8 extreme M={M} N={N} K={K}")
    qa = np.full((M, K), -128, dtype=np.int8)
    qa[1::2] = 127
    qb = np.full((N, K), -128, dtype=np.int8)
    qb[::3] = 127
    sa = np.ones(M, np.float32)
    sb = np.ones(N, np.float32)
    y, acc = tfq.tfq_scaled_mm_int8(dev_u8(qa.view(np.uint8), torch.int8), dev_f32(sa),
                                    dev_u8(qb.view(np.uint8), torch.int8), dev_f32(sb),
                                    want_y=True, want_acc=True)
    torch.cuda.synchronize()
    acc_e, y_e = orc.int8_linear(qa.view(np.uint8), sa, qb.view(np.uint8), sb)
    assert np.array_equal(host_bits(acc).astype(np.int64), acc_e)
    assert np.array_equal(host_bits(y), y_e)


@pytest.mark.parametrize("M,N,K", [(200, 256, 384), (384, 640, 1280), (129, 128, 128)])
def test_fp8_block_scaled(tfq, M, N, K):
    rng = np.random.default_rng(M + N + K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[rng.random((M, K)) < 0.01] *= 20
    x *= np.exp2(rng.integers(-4, 4, (1, K // 128))).repeat(128, axis=1).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    xb, wb = synth.to_bf16_bits(x), synth.to_bf16_bits(w)
    say(f"block-scaled fp8 M={M} N={N} K={K}")
    xd, wd = dev_bf16(xb), dev_bf16(wb)
    qa, sa = tfq.tfq_quantize_rows(xd, "fp8", 448.0, 128)
    qb, sb = tfq.tfq_quantize_weight_per_channel(wd, "fp8", 448.0, 128)
    y = tfq.tfq_scaled_mm_fp8(qa, sa, qb, sb, 128)
    torch.cuda.synchronize()
    qa_e, sa_e = orc.quantize_rows(xb, "fp8", 448.0, 128)
    qb_e, sb_e = orc.quantize_blocks(wb, "fp8", 448.0, 128)
    assert np.array_equal(host_bits(qa), qa_e) and np.array_equal(host_bits(sa), sa_e)
    assert np.array_equal(host_bits(qb), qb_e) and np.array_equal(host_bits(sb), sb_e)
    ref = orc.linear_ref(qa_e, sa_e, qb_e, sb_e, "fp8", scale_block=128)
    assert_fp8_tolerance(host_bits(y), ref, f"block M={M} N={N} K={K}")
    # fused path: same kernels, same bits
    y2 = tfq.tfq_quant_linear_fused(xd, qb, sb, "fp8", 448.0, 128)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y2), host_bits(y))


@pytest.mark.parametrize("M,N,K,epi", [(520, 384, 640, "gelu_tanh"), (300, 256, 256, None),
                                       (257, 128, 384, "gelu_tanh")])
def test_fp8_block_scaled_bias_epilogue(tfq, M, N, K, epi):
    """Block mode with a bias (and GELU): several K blocks, fewer blocks than
    the kernel's load pipeline is deep, ragged M."""
    rng = np.random.default_rng(7 * M + N + K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x *= np.exp2(rng.integers(-3, 3, (1, K // 128))).repeat(128, axis=1).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.03).astype(np.float32)
    bias = (rng.standard_normal(N) * 0.5).astype(np.float32)
    xb, wb, bb = synth.to_bf16_bits(x), synth.to_bf16_bits(w), synth.to_bf16_bits(bias)
    say(f"block-scaled fp8 + bias M={M} N={N} K={K} epi={epi}")
    qa, sa = tfq.tfq_quantize_rows(dev_bf16(xb), "fp8", 448.0, 128)
    qb, sb = tfq.tfq_quantize_weight_per_channel(dev_bf16(wb), "fp8", 448.0, 128)
    y = tfq.tfq_scaled_mm_fp8(qa, sa, qb, sb, 128, dev_bf16(bb), epi)
    torch.cuda.synchronize()
    qa_e, sa_e = orc.quantize_rows(xb, "fp8", 448.0, 128)
    qb_e, sb_e = orc.quantize_blocks(wb, "fp8", 448.0, 128)
    ref = orc.linear_ref(qa_e, sa_e, qb_e, sb_e, "fp8", scale_block=128, bias=bb,
                         gelu=epi == "gelu_tanh")
    assert_fp8_tolerance(host_bits(y), ref, f"block+bias M={M} N={N} K={K} epi={epi}")


@pytest.mark.parametrize("qtype,qmax", [("fp8", 448.0), ("fp8", 7.0), ("int8", 127.0)])
def test_fused_linear_matches_two_calls_and_oracle(tfq, qtype, qmax):
    M, N, K = 333, 264, 528
    xb, wb, _, _, _, _, bias = _operands(17, M, N, K, qtype)
    say(f"quant_linear_fused {qtype} qmax={qmax} M={M} N={N} K={K}")
    xd, wd = dev_bf16(xb), dev_bf16(wb)
    wq, ws = tfq.tfq_quantize_weight_per_channel(wd, qtype, 448.0 if qtype == "fp8" else 127.0)
    y = tfq.tfq_quant_linear_fused(xd, wq, ws, qtype, qmax, 0, dev_bf16(bias), None)
    qa, sa = tfq.tfq_quantize_rows(xd, qtype, qmax)
    if qtype == "fp8":
        y2 = tfq.tfq_scaled_mm_fp8(qa, sa, wq, ws, 0, dev_bf16(bias), None)
    else:
        y2, _ = tfq.tfq_scaled_mm_int8(qa, sa, wq, ws, dev_bf16(bias))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y), host_bits(y2))
    qa_e, sa_e = orc.quantize_rows(xb, qtype, qmax)
    qb_e, sb_e = orc.quantize_rows(wb, qtype, 448.0 if qtype == "fp8" else 127.0)
    if qtype == "fp8":
        ref = orc.linear_ref(qa_e, sa_e, qb_e, sb_e, "fp8", bias=bias)
        assert_fp8_tolerance(host_bits(y), ref, "fused fp8")
    else:
        _, y_e = orc.int8_linear(qa_e, sa_e, qb_e, sb_e, bias=bias, want_acc=False)
        assert np.array_equal(host_bits(y), y_e)


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
def test_fused_linear_strided_input_gelu(tfq, qtype):
    """The fused call on a column slice of a wider tensor (row stride ld_x >
    k) with the GELU epilogue equals quantising the same slice and the GEMM
    with GELU; QuantLinear in block mode equals the fused block call."""
    M, N, K, LD = 300, 264, 512, 640
    rng = np.random.default_rng(29)
    x = (rng.standard_normal((M, LD)) * np.exp2(rng.integers(-3, 4, (M, 1)))).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bias = (rng.standard_normal(N) * 0.1).astype(np.float32)
    xb, wb, bb = synth.to_bf16_bits(x), synth.to_bf16_bits(w), synth.to_bf16_bits(bias)
    qmax = 448.0 if qtype == "fp8" else 127.0
    say(f"quant_linear_fused strided {qtype} M={M} N={N} K={K} ld={LD}")
    xd = dev_bf16(xb)[:, :K]
    assert xd.stride(0) == LD
    wq, ws = tfq.tfq_quantize_weight_per_channel(dev_bf16(wb), qtype, qmax)
    y = tfq.tfq_quant_linear_fused(xd, wq, ws, qtype, qmax, 0, dev_bf16(bb), "gelu_tanh")
    qa, sa = tfq.tfq_quantize_rows(xd, qtype, qmax)
    if qtype == "fp8":
        y2 = tfq.tfq_scaled_mm_fp8(qa, sa, wq, ws, 0, dev_bf16(bb), "gelu_tanh")
    else:
        y2, _ = tfq.tfq_scaled_mm_int8(qa, sa, wq, ws, dev_bf16(bb), "gelu_tanh")
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y), host_bits(y2))
    qa_e, sa_e = orc.quantize_rows(np.ascontiguousarray(xb[:, :K]), qtype, qmax)
    qb_e, sb_e = orc.quantize_rows(wb, qtype, qmax)
    assert np.array_equal(host_bits(qa).view(np.uint8), qa_e.view(np.uint8))
    ref = orc.linear_ref(qa_e, sa_e, qb_e, sb_e, qtype, bias=bb, gelu=True)
    assert_fp8_tolerance(host_bits(y), ref, f"fused strided {qtype}")
    if qtype == "fp8":
        # block mode needs N % 128 == 0: the first 256 weight rows
        wd2, bd2 = dev_bf16(np.ascontiguousarray(wb[:256])), dev_bf16(bb[:256])
        lin = tfq.QuantLinear(wd2, bd2, scale_block=128, epi="gelu_tanh")
        yl = lin(xd)
        wqb, wsb = tfq.tfq_quantize_weight_per_channel(wd2, "fp8", 448.0, 128)
        yb = tfq.tfq_quant_linear_fused(xd, wqb, wsb, "fp8", 448.0, 128, bd2, "gelu_tanh")
        torch.cuda.synchronize()
        assert torch.equal(yl, yb)


def test_quant_linear_module_caches_weight(tfq):
    M, N, K = 100, 256, 256
    xb, wb, _, _, _, _, _ = _operands(3, M, N, K, "fp8")
    say("QuantLinear first-use weight cache")
    lin = tfq.QuantLinear(dev_bf16(wb))
    y1 = lin(dev_bf16(xb))
    wq_first = lin.w_q
    y2 = lin(dev_bf16(xb))
    torch.cuda.synchronize()
    assert lin.w_q is wq_first
    assert torch.equal(y1, y2)
    # a changed weight is used only after requantize()
    lin.weight.mul_(2.0)
    y3 = lin(dev_bf16(xb))
    lin.requantize()
    y4 = lin(dev_bf16(xb))
    torch.cuda.synchronize()
    assert torch.equal(y1, y3)
    assert lin.w_q is not wq_first and not torch.equal(y1, y4)


def _sample_rows(M):
    rng = np.random.default_rng(M)
    return np.unique(np.concatenate([np.arange(16), np.arange(M - 16, M),
                                     rng.choice(np.arange(16, M - 16), 16, replace=False)]))


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
def test_big_tile_path_and_kernel_choice_invariance(tfq, qtype):
    """A shape with more 256x256 tiles than CUs (M=4100, N=4104, ragged M, N
    and K tails) runs the 256x256 kernel; its first 256 rows alone run the
    256x128 two-per-CU kernel.  Sampled rows match the oracle and the
    overlapping outputs of the two kernels are bit-identical."""
    M, N, K = 4100, 4104, 336
    _, _, qa, sa, qb, sb, _ = _operands(99, M, N, K, qtype)
    dt = torch.uint8 if qtype == "fp8" else torch.int8
    a, b = dev_u8(qa, dt), dev_u8(qb, dt)
    sad, sbd = dev_f32(sa), dev_f32(sb)
    say(f"big-tile path {qtype} M={M} N={N} K={K}")
    if qtype == "fp8":
        y = tfq.tfq_scaled_mm_fp8(a, sad, b, sbd)
        y_small = tfq.tfq_scaled_mm_fp8(a[:256].contiguous(), sad[:256].contiguous(), b, sbd)
    else:
        y, acc = tfq.tfq_scaled_mm_int8(a, sad, b, sbd, want_y=True, want_acc=True)
        y_small, _ = tfq.tfq_scaled_mm_int8(a[:256].contiguous(), sad[:256].contiguous(), b, sbd)
    torch.cuda.synchronize()
    rows = _sample_rows(M)
    yb = host_bits(y)
    if qtype == "fp8":
        ref = orc.linear_ref(qa, sa, qb, sb, "fp8", rows=rows)
        assert_fp8_tolerance(yb[rows], ref, "big-tile fp8")
    else:
        acc_e, y_e = orc.int8_linear(qa, sa, qb, sb, rows=rows)
        assert np.array_equal(host_bits(acc)[rows].astype(np.int64), acc_e)
        assert np.array_equal(yb[rows], y_e)
    assert np.array_equal(host_bits(y_small), yb[:256])


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
@pytest.mark.parametrize("M,N,K", [(1300, 968, 1040), (257, 200, 3088)])
def test_192_column_tiles(tfq, qtype, M, N, K):
    """The 256x192 tiles pinned through tfq_autotune_set on ragged M, N
    (N % 192 != 0) and K (K % 128 != 0), with bias and (FP8) GELU: against
    the oracle, and bit for bit against the 256x256 tiles."""
    _, _, qa, sa, qb, sb, bias = _operands(M * 7 + N + K, M, N, K, qtype)
    dt = torch.uint8 if qtype == "fp8" else torch.int8
    a, b = dev_u8(qa, dt), dev_u8(qb, dt)
    sad, sbd, bd = dev_f32(sa), dev_f32(sb), dev_bf16(bias)
    epi = "gelu_tanh" if qtype == "fp8" else None
    tfq.tfq_set_autotune(1)
    try:
        outs = {}
        for kern in (2, 0):
            say(f"{qtype} tile width {192 if kern == 2 else 256} M={M} N={N} K={K}")
            tfq.tfq_autotune_set(qtype, M, N, K, kern, 4, epi)
            if qtype == "fp8":
                y = tfq.tfq_scaled_mm_fp8(a, sad, b, sbd, 0, bd, epi)
                acc = None
            else:
                y, acc = tfq.tfq_scaled_mm_int8(a, sad, b, sbd, bd, epi, want_acc=True)
            torch.cuda.synchronize()
            outs[kern] = (host_bits(y), None if acc is None else host_bits(acc))
    finally:
        tfq.tfq_set_autotune(0)
        tfq.tfq_autotune_clear()
    y192, acc192 = outs[2]
    assert np.array_equal(y192, outs[0][0]), "192- and 256-column tiles differ"
    if qtype == "fp8":
        ref = orc.linear_ref_fast(qa, sa, qb, sb, "fp8", bias=bias, gelu=True)
        assert_fp8_tolerance(y192, ref, f"192-column tiles M={M} N={N} K={K}")
    else:
        acc_e, y_e = orc.int8_linear_fast(qa, sa, qb, sb, bias=bias)
        assert np.array_equal(acc192.astype(np.int64), acc_e)
        assert np.array_equal(y192, y_e)
        assert np.array_equal(acc192, outs[0][1])
