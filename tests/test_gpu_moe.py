"""GPU parity of the MoE routed W8A8 path against the oracle.

TeleFuser "Quantization", "Other quantized data paths" (LingBot-Video MoE
FP8): routed activations quantised per row, expert weights per output
channel, one scaled matmul per expert.  Gathered quantisation: codes and
scales bit for bit.  Grouped GEMM: within 2^-7 |y_ref| + 1e-3 max_row|y_ref|
of the oracle's binary64 result, and bit-identical to the plain scaled GEMM
for a single group.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from gpu_util import assert_fp8_tolerance, dev_bf16, dev_f32, dev_u8, host_bits, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module")
def tfq():
    import int8_w8a8_quantized_amd as m

    return m


def _x(rng, rows, cols):
    x = (0.5 * rng.standard_normal((rows, cols))).astype(np.float32)
    x[rng.random((rows, cols)) < 0.01] *= 20
    return synth.to_bf16_bits(x)


def _dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("qtype,qmax,group,cols", [("fp8", 448.0, 0, 1024), ("fp8", 448.0, 0, 13824),
                                                   ("fp8", 7.0, 0, 40000), ("int8", 127.0, 0, 5120),
                                                   ("fp8", 448.0, 128, 3072)])
def test_gather_quantize_bit_exact(tfq, qtype, qmax, group, cols):
    """Row-resident, split-row, two-pass and group kernels, through a routed
    index with repeats, a reversed run and out-of-range entries."""
    rng = np.random.default_rng(cols + int(qmax))
    src = 97
    x = _x(rng, src, cols)
    idx = np.concatenate([rng.integers(0, src, 150), np.arange(src - 1, src - 30, -1),
                          [-1, src, 2**31 - 1, -2**31]]).astype(np.int32)
    say(f"quantize_rows_gather {qtype} qmax={qmax} group={group} cols={cols} rows={idx.size}")
    q, s = tfq.tfq_quantize_rows_gather(dev_bf16(x), _dev_i32(idx), qtype, qmax, group)
    torch.cuda.synchronize()
    qe, se = orc.quantize_rows_gather(x, idx, qtype, qmax, group)
    assert np.array_equal(host_bits(q), qe)
    assert np.array_equal(host_bits(s), se)


def test_gather_identity_equals_plain_quantize(tfq):
    rng = np.random.default_rng(8)
    x = dev_bf16(_x(rng, 300, 5120))
    say("quantize_rows_gather identity vs quantize_rows")
    q1, s1 = tfq.tfq_quantize_rows(x, "fp8", 448.0)
    q2, s2 = tfq.tfq_quantize_rows_gather(x, _dev_i32(np.arange(300)), "fp8", 448.0)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)


def _experts(rng, E, N, K):
    w = (rng.standard_normal((E * N, K)) * 0.02).astype(np.float32)
    qb, sb = orc.quantize_rows(synth.to_bf16_bits(w), "fp8", 448.0)
    bias = synth.to_bf16_bits(rng.standard_normal((E, N)).astype(np.float32))
    return qb.reshape(E, N, K), sb.reshape(E, N), bias


@pytest.mark.parametrize("sizes,N,K", [([300, 0, 1, 257, 512, 44], 264, 384),
                                       ([1000], 520, 1040),
                                       ([17, 250, 3, 600], 136, 3088)])
def test_grouped_gemm(tfq, sizes, N, K):
    rng = np.random.default_rng(sum(sizes) + N + K)
    E = len(sizes)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(off[-1])
    qa, sa = orc.quantize_rows(_x(rng, M, K), "fp8", 448.0)
    qb, sb, bias = _experts(rng, E, N, K)
    a, b, sad, sbd, offd = dev_u8(qa), dev_u8(qb), dev_f32(sa), dev_f32(sb), _dev_i32(off)
    for use_bias, epi in [(False, None), (True, "gelu_tanh")]:
        say(f"grouped_scaled_mm_fp8 sizes={sizes} N={N} K={K} bias={use_bias} epi={epi}")
        y = tfq.tfq_grouped_scaled_mm_fp8(a, sad, b, sbd, offd,
                                          dev_bf16(bias) if use_bias else None, epi)
        torch.cuda.synchronize()
        ref = orc.grouped_linear_ref(qa, sa, qb, sb, off, bias=bias if use_bias else None,
                                     gelu=epi is not None)
        assert_fp8_tolerance(host_bits(y), ref, f"grouped sizes={sizes} bias={use_bias} epi={epi}")


def test_single_group_matches_plain_gemm_bits(tfq):
    """One group over all rows runs the same tiles, MFMAs and epilogue as the
    plain 256x256 kernel (a grid with more than 256 tiles), so the bits agree."""
    M, N, K = 4100, 4104, 336
    rng = np.random.default_rng(12)
    qa, sa = orc.quantize_rows(_x(rng, M, K), "fp8", 448.0)
    qb, sb, _ = _experts(rng, 1, N, K)
    a, b, sad, sbd = dev_u8(qa), dev_u8(qb), dev_f32(sa), dev_f32(sb)
    say(f"grouped single group vs scaled_mm_fp8 M={M} N={N} K={K}")
    y1 = tfq.tfq_grouped_scaled_mm_fp8(a, sad, b, sbd, _dev_i32([0, M]))
    y2 = tfq.tfq_scaled_mm_fp8(a, sad, b[0], sbd[0])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_rows_outside_groups_untouched_and_bad_offsets_stay_in_bounds(tfq):
    """Rows before the first and after the last offset keep their contents.
    Decreasing and out-of-range offsets (unspecified results) write nothing
    outside y: a sentinel band after y's rows is unchanged."""
    M, N, K, E = 600, 136, 256, 3
    rng = np.random.default_rng(13)
    qa, sa = orc.quantize_rows(_x(rng, M, K), "fp8", 448.0)
    qb, sb, _ = _experts(rng, E, N, K)
    a, b, sad, sbd = dev_u8(qa), dev_u8(qb), dev_f32(sa), dev_f32(sb)
    sentinel = torch.full((M + 64, N), 7.0, dtype=torch.bfloat16, device="cuda")
    y = sentinel[:M]
    off = np.array([40, 300, 300, 520], dtype=np.int32)
    say("grouped rows outside groups")
    tfq.tfq_grouped_scaled_mm_fp8(a, sad, b, sbd, _dev_i32(off), y=y)
    torch.cuda.synchronize()
    yb = host_bits(sentinel)
    seven = host_bits(torch.tensor([7.0], dtype=torch.bfloat16))[0]
    assert (yb[:40] == seven).all() and (yb[520:] == seven).all()
    ref = orc.grouped_linear_ref(qa, sa, qb, sb, off, rows=np.arange(40, 520))
    assert_fp8_tolerance(yb[40:520], ref, "grouped inner rows")
    for bad in ([0, 500, 100, 600], [-50, 2**30, 10, -7], [600, 0, 0, 0]):
        say(f"grouped invalid offsets {bad}")
        sentinel.fill_(7.0)
        tfq.tfq_grouped_scaled_mm_fp8(a, sad, b, sbd, _dev_i32(bad), y=y)
        torch.cuda.synchronize()
        assert (host_bits(sentinel)[M:] == seven).all()


def test_moe_layer_sampled_rows(tfq):
    """A routed layer end to end: 8 experts, top-2 routing of 16384 tokens
    (ragged expert loads), gather-quantise then the grouped GEMM; sampled rows
    of every expert against the oracle."""
    T, K, N, E, topk = 16384, 5120, 2048, 8, 2
    rng = np.random.default_rng(77)
    x = _x(rng, T, K)
    p = rng.dirichlet(np.full(E, 0.7))
    choice = np.stack([rng.choice(E, 2, replace=False, p=p) for _ in range(T)])
    token = np.repeat(np.arange(T), topk)
    expert = choice.reshape(-1)
    order = np.argsort(expert, kind="stable")
    row_index = token[order].astype(np.int32)
    off = np.concatenate([[0], np.cumsum(np.bincount(expert, minlength=E))]).astype(np.int32)
    qb, sb, bias = _experts(rng, E, N, K)
    say(f"moe layer T={T} K={K} N={N} E={E} top{topk} loads={np.diff(off).tolist()}")
    qa, sa = tfq.tfq_quantize_rows_gather(dev_bf16(x), _dev_i32(row_index), "fp8", 448.0)
    y = tfq.tfq_grouped_scaled_mm_fp8(qa, sa, dev_u8(qb), dev_f32(sb), _dev_i32(off),
                                      dev_bf16(bias), "gelu_tanh")
    torch.cuda.synchronize()
    qa_e, sa_e = orc.quantize_rows_gather(x, row_index, "fp8", 448.0)
    assert np.array_equal(host_bits(qa), qa_e) and np.array_equal(host_bits(sa), sa_e)
    rows = np.unique(np.concatenate([np.concatenate([[o, max(o, e - 1)], rng.integers(o, max(o + 1, e), 4)])
                                     for o, e in zip(off[:-1], off[1:]) if e > o]))
    ref = orc.grouped_linear_ref(qa_e, sa_e, qb, sb, off, bias=bias, gelu=True, rows=rows)
    assert_fp8_tolerance(host_bits(y)[rows], ref, "moe layer")
