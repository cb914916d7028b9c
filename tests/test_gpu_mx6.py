"""GPU parity of the MXFP6 path (E2M3 and E3M2 elements) against the oracle.

MXFP6 = 6-bit elements packed as a little-endian bit stream per row, with one
E8M0 scale per 32 elements along K; the library stores each 128-element
group's 96 bytes group-major ([cols/128, rows, 96]), and these tests move
the oracle's row streams into that layout and back (a byte permutation) (TeleFuser "Quantization", converter
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
                      mx6_grouped, mx6_ungrouped, mx_grouped, mx_ungrouped, needs_gpu, say)

pytestmark = [pytest.mark.gpu, needs_gpu]

FMTS = ["e2m3", "e3m2"]


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


def _pack6(codes):
    """6-bit codes [R, K] -> little-endian bit stream [R, 3K/4] (four codes in three bytes)."""
    c = codes.astype(np.uint32).reshape(codes.shape[0], -1, 4)
    w = c[..., 0] | (c[..., 1] << 6) | (c[..., 2] << 12) | (c[..., 3] << 18)
    out = np.stack([w & 255, (w >> 8) & 255, (w >> 16) & 255], axis=-1)
    return out.reshape(codes.shape[0], -1).astype(np.uint8)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,cols", [(1, 128), (300, 1152), (7, 13824), (64, 8192 + 128)])
def test_quantize_mxfp6_bit_exact(tfq, fmt, rows, cols):
    rng = np.random.default_rng(rows * 37 + cols)
    xb = _blocky(rng, rows, cols)
    say(f"quantize_mxfp6 {fmt} rows={rows} cols={cols}")
    q, s = tfq.tfq_quantize_mxfp6(dev_bf16(xb), fmt)
    torch.cuda.synchronize()
    qe, se = orc.quantize_mx6(xb, fmt)
    assert np.array_equal(mx_ungrouped(host_bits(s)), se)
    assert np.array_equal(mx6_ungrouped(host_bits(q)), qe)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_mxfp6_every_bf16_value(tfq, fmt):
    """Every finite BF16 value, both signs, through the quantiser under
    shared exponents from -127 (the E8M0 byte 0) to the largest the format's
    amax allows: codes and scale bytes bit for bit against the oracle (this
    pins the hardware's scaled 6-bit conversion, saturation and ties
    included)."""
    kemax = 2 if fmt == "e2m3" else 4
    xb = every_bf16_blocks(kemax, [-127, -126, -20, -1, 0, 1, 20, 127 - kemax])
    say(f"mxfp6 {fmt} every bf16 value rows={xb.shape[0]} cols={xb.shape[1]}")
    q, s = tfq.tfq_quantize_mxfp6(dev_bf16(xb), fmt)
    torch.cuda.synchronize()
    q_e, s_e = orc.quantize_mx6(xb, fmt)
    assert np.array_equal(mx_ungrouped(host_bits(s)), s_e)
    assert np.array_equal(mx6_ungrouped(host_bits(q)), q_e)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_mxfp6_special_values_and_stride(tfq, fmt):
    """Ties at every grid midpoint, saturation, zero / signed-zero, subnormal
    and huge blocks, through a row stride larger than the row."""
    rng = np.random.default_rng(3)
    rows, cols, ld = 40, 384, 512
    x = rng.standard_normal((rows, ld)).astype(np.float32)
    x[0, :32] = 0.0
    x[1, :32] = -0.0
    x[2, :32] = np.float32(2.0 ** -130) * rng.integers(-3, 4, 32)
    x[3, :32] = rng.standard_normal(32) * 2.0 ** 120
    # largest value first (X = 1), then every midpoint of the grid in the
    # following blocks, both signs
    eb, mb, bias = (2, 3, 1) if fmt == "e2m3" else (3, 2, 3)
    grid = [(m / (1 << mb)) * 2.0 ** (1 - bias) if e == 0 else (1 + m / (1 << mb)) * 2.0 ** (e - bias)
            for e in range(1 << eb) for m in range(1 << mb)]
    mids = [(a + b) / 2 for a, b in zip(grid[:-1], grid[1:])]
    for r in range(4, 6):
        chunk = mids[(r - 4) * 16:(r - 3) * 16]
        x[r, :32] = 0.0
        x[r, 0] = grid[-1]
        x[r, 1:1 + len(chunk)] = chunk
        x[r, 17:17 + min(len(chunk), 15)] = [-v for v in chunk][:15]
    x[6, :4] = [grid[-1] * 1.06, grid[-1], -grid[-1] * 1.01, 1.0]
    x[7] *= 2.0 ** -126
    xb = synth.to_bf16_bits(x)
    xd = dev_bf16(xb)[:, :cols]
    say(f"quantize_mxfp6 {fmt} special rows={rows} cols={cols} ld={ld}")
    q, s = tfq.tfq_quantize_mxfp6(xd, fmt)
    torch.cuda.synchronize()
    qe, se = orc.quantize_mx6(xb[:, :cols], fmt)
    assert np.array_equal(mx_ungrouped(host_bits(s)), se)
    assert np.array_equal(mx6_ungrouped(host_bits(q)), qe)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,cols", [(37, 384), (17, 128)])
def test_quantize_mxfp6_writes_nothing_past_its_outputs(tfq, fmt, rows, cols):
    """Codes and scales land in views at the front of larger buffers filled
    with a sentinel: a workgroup's last rows (rows not a multiple of 16) must
    not write past either output."""
    rng = np.random.default_rng(rows + cols)
    xb = _blocky(rng, rows, cols)
    nq, ns = cols // 128 * rows * 96, cols // 128 * rows * 4
    qbuf = torch.full((nq + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((ns + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    q = qbuf[:nq].view(cols // 128, rows, 96)
    s = sbuf[:ns].view(cols // 128, rows, 4)
    say(f"quantize_mxfp6 {fmt} guard rows={rows} cols={cols}")
    tfq.tfq_quantize_mxfp6(dev_bf16(xb), fmt, q, s)
    torch.cuda.synchronize()
    assert bool((qbuf[nq:] == 0xA5).all()) and bool((sbuf[ns:] == 0x5A).all())
    qe, se = orc.quantize_mx6(xb, fmt)
    assert np.array_equal(mx6_ungrouped(host_bits(q)), qe)
    assert np.array_equal(mx_ungrouped(host_bits(s)), se)


def _operands(seed, M, N, K, fmt):
    rng = np.random.default_rng(seed)
    xb = _blocky(rng, M, K)
    wb = _blocky(rng, N, K, sigma=0.02, spread=3)
    qa, sa = orc.quantize_mx6(xb, fmt)
    qb, sb = orc.quantize_mx6(wb, fmt)
    bias = synth.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    return xb, wb, qa, sa, qb, sb, bias


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(1, 8, 128), (300, 520, 384), (257, 264, 1152), (513, 768, 2048),
                                   (64, 2048, 256), (130, 136, 640),
                                   (258, 136, 640), (259, 264, 384)])
def test_mxfp6_gemm(tfq, fmt, M, N, K):
    _, _, qa, sa, qb, sb, bias = _operands(M + 3 * N + K, M, N, K, fmt)
    a, b = dev_u8(mx6_grouped(qa)), dev_u8(mx6_grouped(qb))
    sad, sbd = dev_u8(mx_grouped(sa)), dev_u8(mx_grouped(sb))
    for use_bias, epi in [(False, None), (True, None), (True, "gelu_tanh")]:
        say(f"scaled_mm_mxfp6 {fmt} M={M} N={N} K={K} bias={use_bias} epi={epi}")
        y = tfq.tfq_scaled_mm_mxfp6(a, sad, b, sbd, fmt, dev_bf16(bias) if use_bias else None, epi)
        torch.cuda.synchronize()
        ref = orc.linear_mx6_ref(qa, sa, qb, sb, fmt, bias=bias if use_bias else None,
                                 gelu=epi is not None)
        assert_fp8_tolerance(host_bits(y), ref,
                             f"mx6 {fmt} M={M} N={N} K={K} bias={use_bias} epi={epi}")


@pytest.mark.parametrize("fmt", FMTS)
def test_mxfp6_single_block_scales(tfq, fmt):
    """Each activation row has one non-zero 32-element block: a scale or a
    code taken from the wrong block, row or operand shows up in the sum."""
    M, N, K = 256, 256, 512
    rng = np.random.default_rng(21)
    codes = np.zeros((M, K), np.uint8)
    kb_a = rng.integers(0, K // 32, M)
    for m in range(M):
        codes[m, kb_a[m] * 32:(kb_a[m] + 1) * 32] = rng.integers(1, 32, 32) | (rng.integers(0, 2, 32) << 5)
    qa = _pack6(codes)
    qb = _pack6(rng.integers(0, 64, (N, K)).astype(np.uint8))
    sa = rng.integers(110, 140, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(110, 140, (N, K // 32)).astype(np.uint8)
    say(f"scaled_mm_mxfp6 {fmt} single-block M={M} N={N} K={K}")
    y = tfq.tfq_scaled_mm_mxfp6(dev_u8(mx6_grouped(qa)), dev_u8(mx_grouped(sa)),
                                dev_u8(mx6_grouped(qb)), dev_u8(mx_grouped(sb)), fmt)
    torch.cuda.synchronize()
    ref = orc.linear_mx6_ref(qa, sa, qb, sb, fmt)
    assert_fp8_tolerance(host_bits(y), ref, f"mx6 {fmt} single-block")


@pytest.mark.parametrize("fmt", FMTS)
def test_mxfp6_one_hot_codes(tfq, fmt):
    """A single non-zero code per row of A at a distinct K position, B all
    random: output row m is exactly B's column at that position times the
    scales, so any misplaced 6-bit field (stream order, slot, lane half) shows
    as a wrong value, not only a rounding difference."""
    M, N, K = 128, 64, 768
    rng = np.random.default_rng(5)
    codes = np.zeros((M, K), np.uint8)
    pos = rng.permutation(K)[:M]
    codes[np.arange(M), pos] = rng.integers(1, 64, M)
    qa = _pack6(codes)
    qb = _pack6(rng.integers(0, 64, (N, K)).astype(np.uint8))
    sa = np.full((M, K // 32), 127, np.uint8)
    sb = np.full((N, K // 32), 127, np.uint8)
    say(f"scaled_mm_mxfp6 {fmt} one-hot M={M} N={N} K={K}")
    y = tfq.tfq_scaled_mm_mxfp6(dev_u8(mx6_grouped(qa)), dev_u8(mx_grouped(sa)),
                                dev_u8(mx6_grouped(qb)), dev_u8(mx_grouped(sb)), fmt)
    torch.cuda.synchronize()
    ref = orc.linear_mx6_ref(qa, sa, qb, sb, fmt)
    # a product of two 6-bit values fits BF16's 8 significant bits exactly
    got = (host_bits(y).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("fmt", FMTS)
def test_mxfp6_quantize_then_gemm_end_to_end(tfq, fmt):
    M, N, K = 333, 264, 640
    xb, wb, _, _, _, _, bias = _operands(17, M, N, K, fmt)
    say(f"mx6 {fmt} end-to-end M={M} N={N} K={K}")
    qa, sa = tfq.tfq_quantize_mxfp6(dev_bf16(xb), fmt)
    qb, sb = tfq.tfq_quantize_mxfp6(dev_bf16(wb), fmt)
    y = tfq.tfq_scaled_mm_mxfp6(qa, sa, qb, sb, fmt, dev_bf16(bias), "gelu_tanh")
    torch.cuda.synchronize()
    qa_e, sa_e = orc.quantize_mx6(xb, fmt)
    qb_e, sb_e = orc.quantize_mx6(wb, fmt)
    assert np.array_equal(mx6_ungrouped(host_bits(qa)), qa_e)
    assert np.array_equal(mx_ungrouped(host_bits(sa)), sa_e)
    assert np.array_equal(mx6_ungrouped(host_bits(qb)), qb_e)
    assert np.array_equal(mx_ungrouped(host_bits(sb)), sb_e)
    ref = orc.linear_mx6_ref(qa_e, sa_e, qb_e, sb_e, fmt, bias=bias, gelu=True)
    assert_fp8_tolerance(host_bits(y), ref, f"mx6 {fmt} end-to-end")


@pytest.mark.parametrize("fmt", FMTS)
def test_mxfp6_big_shape_sampled_rows(tfq, fmt):
    M, N, K = 4100, 4104, 1280
    _, _, qa, sa, qb, sb, _ = _operands(99, M, N, K, fmt)
    say(f"scaled_mm_mxfp6 {fmt} big M={M} N={N} K={K}")
    y = tfq.tfq_scaled_mm_mxfp6(dev_u8(mx6_grouped(qa)), dev_u8(mx_grouped(sa)),
                                dev_u8(mx6_grouped(qb)), dev_u8(mx_grouped(sb)), fmt)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(M - 8, M),
                                     rng.choice(np.arange(8, M - 8), 16, replace=False)]))
    ref = orc.linear_mx6_ref(qa, sa, qb, sb, fmt, rows=rows)
    assert_fp8_tolerance(host_bits(y)[rows], ref, f"mx6 {fmt} big")


@pytest.mark.parametrize("fmt", FMTS)
def test_mxfp6_quant_linear_and_tuned_config(tfq, fmt):
    """QuantLinear in an MXFP6 mode equals quantise + GEMM through the entry
    points; the tuned launch configuration gives the same bits as the default
    one and is recorded under the format's own kind."""
    M, N, K = 200, 264, 512
    rng = np.random.default_rng(4)
    xb = _blocky(rng, M, K)
    wb = _blocky(rng, N, K, sigma=0.02, spread=3)
    bias = synth.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    say(f"QuantLinear mxfp6_{fmt} M={M} N={N} K={K}")
    lin = tfq.QuantLinear(dev_bf16(wb), dev_bf16(bias), qtype=f"mxfp6_{fmt}", epi="gelu_tanh")
    y1 = lin(dev_bf16(xb))
    wq, act = lin.w_q, lin._act[0]
    y2 = lin(dev_bf16(xb))
    qa, sa = tfq.tfq_quantize_mxfp6(dev_bf16(xb), fmt)
    qb, sb = tfq.tfq_quantize_mxfp6(dev_bf16(wb), fmt)
    y3 = tfq.tfq_scaled_mm_mxfp6(qa, sa, qb, sb, fmt, dev_bf16(bias), "gelu_tanh")
    torch.cuda.synchronize()
    assert lin.w_q is wq and lin._act[0] is act   # same shape: buffers reused
    assert torch.equal(y1, y2) and torch.equal(y1, y3)
    # fewer rows, then the first shape again: new activation buffers, same bits
    y4 = lin(dev_bf16(xb[:77]))
    y5 = lin(dev_bf16(xb))
    torch.cuda.synchronize()
    assert torch.equal(y4, y1[:77]) and torch.equal(y5, y1)
    say(f"autotune mxfp6_{fmt}")
    tfq.tfq_autotune_clear()
    try:
        tfq.tfq_set_autotune(1)
        y4 = tfq.tfq_scaled_mm_mxfp6(qa, sa, qb, sb, fmt, dev_bf16(bias), "gelu_tanh")
        y5 = tfq.tfq_scaled_mm_mxfp6(qa, sa, qb, sb, fmt, dev_bf16(bias), "gelu_tanh")
        torch.cuda.synchronize()
        cfg = tfq.tfq_autotune_lookup(f"mxfp6_{fmt}", M, N, K, "gelu_tanh")
    finally:
        tfq.tfq_set_autotune(0)
        tfq.tfq_autotune_clear()
    assert torch.equal(y3, y4) and torch.equal(y3, y5)
    assert cfg is not None and cfg[0] == 0 and cfg[1] in (1, 2, 4, 8)
