"""GEMMs at the largest K each entry point accepts, so that every 32-bit
buffer offset and record count runs at its bound: FP8 on both kernels
(K = 2^22), MXFP8 (K = 2^22), MXFP4 (K = 2^23) and block-scaled FP8
(K = 2^17).  Codes are random on the
device; outputs are checked on sampled rows x columns against the oracle
(which takes the matching rows of the operands).  MX scales change with the
K block (a different power of two every block), so a misplaced scale word
at a large offset would show.  MXFP6's group-major codes are also checked
past 4 GiB of offset.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from gpu_util import (assert_fp8_tolerance, dev_bf16, host_bits, mx6_ungrouped, mx_grouped,
                      mx_ungrouped, needs_gpu, say)

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module")
def tfq():
    import int8_w8a8_quantized_amd as m

    return m


def _codes(g, rows, cols, fp4=False):
    t = torch.randint(0, 256, (rows, cols), dtype=torch.uint8, device="cuda", generator=g)
    if not fp4:
        t[(t & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    return t


ROWS = np.array([0, 1, 97, 255])


@pytest.mark.parametrize("M,N", [(2048, 2048), (264, 264)])
def test_fp8_max_k(tfq, M, N):
    K = 1 << 22
    g = torch.Generator(device="cuda").manual_seed(1)
    a, b = _codes(g, M, K), _codes(g, N, K)
    sa = torch.rand((M,), device="cuda", generator=g) * 1e-3
    sb = torch.rand((N,), device="cuda", generator=g) * 1e-3
    say(f"fp8 max K: M={M} N={N} K={K}")
    y = tfq.tfq_scaled_mm_fp8(a, sa, b, sb)
    torch.cuda.synchronize()
    cols = np.array([0, 5, 130, N - 1])
    r, c = torch.from_numpy(ROWS), torch.from_numpy(cols)
    ref = orc.linear_ref(host_bits(a[r]), host_bits(sa[r]), host_bits(b[c]), host_bits(sb[c]),
                         "fp8")
    assert_fp8_tolerance(host_bits(y)[ROWS][:, cols], ref, f"fp8 max K {M}x{N}")


def _mx_scale_row(K):
    """One row of E8M0 scales [K/32] that differ per K block: 120 + (block % 15)."""
    return (120 + np.arange(K // 32) % 15).astype(np.uint8)


@pytest.mark.parametrize("fp4", [False, True])
def test_mx_max_k(tfq, fp4):
    M, N = 512, 264
    K = (1 << 23) if fp4 else (1 << 22)
    kb = K // 2 if fp4 else K
    g = torch.Generator(device="cuda").manual_seed(2)
    a, b = _codes(g, M, kb, fp4), _codes(g, N, kb, fp4)
    row = _mx_scale_row(K)
    grouped_row = torch.from_numpy(mx_grouped(row[None, :])).cuda()   # [K/128, 1, 4]
    sa = grouped_row.expand(K // 128, M, 4).contiguous()
    sb = grouped_row.expand(K // 128, N, 4).contiguous()
    say(f"mx max K: fp4={fp4} M={M} N={N} K={K}")
    mm = tfq.tfq_scaled_mm_mxfp4 if fp4 else tfq.tfq_scaled_mm_mxfp8
    y = mm(a, sa, b, sb)
    torch.cuda.synchronize()
    cols = np.array([0, 7, 200, N - 1])
    ref_fn = orc.linear_mx4_ref if fp4 else orc.linear_mx_ref
    r, c = torch.from_numpy(ROWS), torch.from_numpy(cols)
    ref = ref_fn(host_bits(a[r]), np.repeat(row[None, :], ROWS.size, 0), host_bits(b[c]),
                 np.repeat(row[None, :], cols.size, 0))
    assert_fp8_tolerance(host_bits(y)[ROWS][:, cols], ref, f"mx max K fp4={fp4}")


def test_block_scaled_max_k(tfq):
    """Block-scaled FP8 at the largest K (131072: the weight blocks' scale
    row fills its 4 KB of LDS), ragged M, bias and GELU, with row scales and
    weight-block scales that change with every K block."""
    M, N, K = 300, 256, 1 << 17
    g = torch.Generator(device="cuda").manual_seed(3)
    a, b = _codes(g, M, K), _codes(g, N, K)
    kb = torch.arange(K // 128, device="cuda", dtype=torch.float32)
    sa = (torch.rand((M, K // 128), device="cuda", generator=g) + 0.5) * torch.exp2(kb % 7 - 3) * 1e-3
    sb = (torch.rand((N // 128, K // 128), device="cuda", generator=g) + 0.5) * 1e-3
    rng = np.random.default_rng(7)
    bias = synth.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    say(f"block-scaled max K: M={M} N={N} K={K}")
    y = tfq.tfq_scaled_mm_fp8(a, sa, b, sb, 128, dev_bf16(bias), "gelu_tanh")
    torch.cuda.synchronize()
    rows = np.array([0, 1, 150, 255, 256, 299])
    ref = orc.linear_ref(host_bits(a), host_bits(sa), host_bits(b), host_bits(sb), "fp8", 128,
                         bias=bias, gelu=True, rows=rows)
    assert_fp8_tolerance(host_bits(y)[rows], ref, "block-scaled max K")


def test_mx6_max_k(tfq):
    """MXFP6 (E3M2) at the largest K (2^22: 3 MiB code rows)."""
    M, N, K = 512, 264, 1 << 22
    g = torch.Generator(device="cuda").manual_seed(4)
    a = torch.randint(0, 256, (K // 128, M, 96), dtype=torch.uint8, device="cuda", generator=g)
    b = torch.randint(0, 256, (K // 128, N, 96), dtype=torch.uint8, device="cuda", generator=g)
    row = _mx_scale_row(K)
    grouped_row = torch.from_numpy(mx_grouped(row[None, :])).cuda()
    sa = grouped_row.expand(K // 128, M, 4).contiguous()
    sb = grouped_row.expand(K // 128, N, 4).contiguous()
    say(f"mx6 max K: M={M} N={N} K={K}")
    y = tfq.tfq_scaled_mm_mxfp6(a, sa, b, sb, "e3m2")
    torch.cuda.synchronize()
    cols = np.array([0, 7, 200, N - 1])
    r, c = torch.from_numpy(ROWS), torch.from_numpy(cols)
    ref = orc.linear_mx6_ref(mx6_ungrouped(host_bits(a[:, r])), np.repeat(row[None, :], ROWS.size, 0),
                             mx6_ungrouped(host_bits(b[:, c])),
                             np.repeat(row[None, :], cols.size, 0), "e3m2")
    assert_fp8_tolerance(host_bits(y)[ROWS][:, cols], ref, "mx6 max K")


def test_mx6_group_major_past_4gib(tfq):
    """MXFP6 codes of a [50000, 131072] input: the group-major array is 4.9 GB,
    so the last groups' byte offsets ((g rows + r) 96) pass 2^32.  The
    quantiser's codes and scales for sampled rows (the first, one in the
    middle, the last) are bit-exact against the oracle, and the GEMM over
    them (N = 64) is within tolerance on those rows."""
    M, N, K = 50000, 64, 1 << 17
    assert (K // 128 - 1) * M * 96 > 1 << 32
    g = torch.Generator(device="cuda").manual_seed(6)
    x = torch.randn((M, K), dtype=torch.bfloat16, device="cuda", generator=g)
    rng = np.random.default_rng(6)
    wb = synth.to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    say(f"mx6 group-major past 4 GiB: M={M} N={N} K={K}")
    qa, sa = tfq.tfq_quantize_mxfp6(x, "e2m3")
    qb, sb = tfq.tfq_quantize_mxfp6(dev_bf16(wb), "e2m3")
    y = tfq.tfq_scaled_mm_mxfp6(qa, sa, qb, sb, "e2m3")
    torch.cuda.synchronize()
    rows = np.array([0, 24999, M - 1])
    r = torch.from_numpy(rows).cuda()
    xr = host_bits(x[r])
    del x
    qe, se = orc.quantize_mx6(xr, "e2m3")
    assert np.array_equal(mx6_ungrouped(host_bits(qa[:, r])), qe)
    got_s = host_bits(sa[:, r])
    assert np.array_equal(mx_ungrouped(got_s), se)
    qbe, sbe = orc.quantize_mx6(wb, "e2m3")
    ref = orc.linear_mx6_ref(qe, se, qbe, sbe, "e2m3")
    assert_fp8_tolerance(host_bits(y[r]), ref, "mx6 past 4 GiB")
