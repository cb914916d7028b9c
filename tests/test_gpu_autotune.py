"""GPU checks of the per-shape autotuner (LightX2V "模型量化技术",
"MiniMax-H3 FP8 FP16 累加": tile choices tuned per exact GEMM shape, winner
cached in process).  Every candidate configuration sums in the same order,
so tuned and untuned results must be bit-identical; the winner must be one
of the candidates; a captured stream must not be tuned, and the captured
graph must replay the eager result."""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from gpu_util import assert_fp8_tolerance, dev_bf16, dev_f32, dev_u8, host_bits, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture()
def tfq():
    import int8_w8a8_quantized_amd as m

    m.tfq_autotune_clear()
    yield m
    m.tfq_set_autotune(0)
    m.tfq_autotune_clear()


def _fp8(rng, r, c):
    x = rng.standard_normal((r, c)).astype(np.float32)
    return orc.quantize_rows(synth.to_bf16_bits(x), "fp8", 448.0)


@pytest.mark.parametrize("M,N,K", [(1000, 2048, 1024), (4100, 4104, 336)])
def test_fp8_tuned_equals_default(tfq, M, N, K):
    rng = np.random.default_rng(M + N)
    qa, sa = _fp8(rng, M, K)
    qb, sb = _fp8(rng, N, K)
    a, b, sad, sbd = dev_u8(qa), dev_u8(qb), dev_f32(sa), dev_f32(sb)
    say(f"autotune fp8 M={M} N={N} K={K}")
    y0 = tfq.tfq_scaled_mm_fp8(a, sad, b, sbd, 0, None, "gelu_tanh")
    tfq.tfq_set_autotune(1)
    y1 = tfq.tfq_scaled_mm_fp8(a, sad, b, sbd, 0, None, "gelu_tanh")   # tunes
    y2 = tfq.tfq_scaled_mm_fp8(a, sad, b, sbd, 0, None, "gelu_tanh")   # cached
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(y0, y2)
    cfg = tfq.tfq_autotune_lookup("fp8", M, N, K, "gelu_tanh")
    assert cfg is not None and cfg[0] in (0, 1, 2) and cfg[1] in (1, 2, 4, 8)
    assert tfq.tfq_autotune_lookup("fp8", M, N, K, None) is None   # another key
    # the tuned result against the oracle directly (sampled rows + the ragged tail)
    rows = np.unique(np.concatenate([np.arange(16), np.arange(M - 16, M),
                                     rng.integers(0, M, 32)]))
    ref = orc.linear_ref(qa, sa, qb, sb, "fp8", gelu=True, rows=rows)
    assert_fp8_tolerance(host_bits(y1)[rows], ref, "tuned fp8 + gelu")


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
def test_every_candidate_configuration(tfq, qtype):
    """tfq_autotune_set pins each candidate configuration of a shape in turn
    (256x256 tiles, 256x192 tiles, the two-per-CU 256x128 kernel; every band
    height): every one writes the same bits, which match the oracle.  A
    configuration that is not a candidate is refused."""
    M, N, K = 777, 1000, 1040
    rng = np.random.default_rng(17)
    x = synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = synth.to_bf16_bits((0.02 * rng.standard_normal((N, K))).astype(np.float32))
    qmax = 448.0 if qtype == "fp8" else 127.0
    qa, sa = orc.quantize_rows(x, qtype, qmax)
    qb, sb = orc.quantize_rows(w, qtype, qmax)
    dt = torch.uint8 if qtype == "fp8" else torch.int8
    a, b, sad, sbd = dev_u8(qa, dt), dev_u8(qb, dt), dev_f32(sa), dev_f32(sb)
    kernels = (0, 1, 2)
    epi = "gelu_tanh" if qtype == "fp8" else None  # INT8: the bit-exact BF16 epilogue
    tfq.tfq_set_autotune(1)
    outs = {}
    for kern in kernels:
        for band in (1, 2, 4, 8):
            say(f"pinned config {qtype} kernel={kern} band={band} M={M} N={N} K={K}")
            tfq.tfq_autotune_set(qtype, M, N, K, kern, band, epi)
            assert tfq.tfq_autotune_lookup(qtype, M, N, K, epi) == (kern, band)
            if qtype == "fp8":
                y = tfq.tfq_scaled_mm_fp8(a, sad, b, sbd, 0, None, epi)
                outs[(kern, band)] = (host_bits(y),)
            else:
                y, acc = tfq.tfq_scaled_mm_int8(a, sad, b, sbd, None, epi, want_acc=True)
                outs[(kern, band)] = (host_bits(y), host_bits(acc))
            torch.cuda.synchronize()
    first = next(iter(outs.values()))
    for k, v in outs.items():
        for got, want in zip(v, first):
            assert np.array_equal(got, want), f"configuration {k} differs"
    rows = np.unique(np.concatenate([np.arange(8), np.arange(M - 8, M), rng.integers(0, M, 24)]))
    if qtype == "fp8":
        ref = orc.linear_ref(qa, sa, qb, sb, qtype, gelu=True, rows=rows)
        assert_fp8_tolerance(first[0][rows], ref, "pinned configurations")
    else:
        acc_e, y_e = orc.int8_linear(qa, sa, qb, sb, rows=rows)
        assert np.array_equal(first[1][rows].astype(np.int64), acc_e), "INT32 sums differ"
        assert np.array_equal(first[0][rows], y_e), "INT8 BF16 output differs from the oracle"
    with pytest.raises(tfq.TfqError):
        tfq.tfq_autotune_set(qtype, M, N, K, 7, 4, epi)
    with pytest.raises(tfq.TfqError):
        tfq.tfq_autotune_set(qtype, M, N, K, 2, 3, epi)   # band 3


def test_other_kinds_tuned_equal_default(tfq):
    rng = np.random.default_rng(5)
    M, N, K = 700, 1024, 1024
    # INT8 with raw sums
    xa = synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    xb = synth.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32))
    qa, sa = orc.quantize_rows(xa, "int8", 127.0)
    qb, sb = orc.quantize_rows(xb, "int8", 127.0)
    a, b = dev_u8(qa, torch.int8), dev_u8(qb, torch.int8)
    say("autotune int8 / block / mx / grouped")
    y0, c0 = tfq.tfq_scaled_mm_int8(a, dev_f32(sa), b, dev_f32(sb), want_acc=True)
    # block-scaled FP8
    xd, wd = dev_bf16(xa), dev_bf16(xb)
    qa8, sa8 = tfq.tfq_quantize_rows(xd, "fp8", 448.0, 128)
    qw8, sw8 = tfq.tfq_quantize_weight_per_channel(wd, "fp8", 448.0, 128)
    yb0 = tfq.tfq_scaled_mm_fp8(qa8, sa8, qw8, sw8, 128)
    # MXFP8
    qam, sam = tfq.tfq_quantize_mx(xd)
    qwm, swm = tfq.tfq_quantize_mx(wd)
    ym0 = tfq.tfq_scaled_mm_mxfp8(qam, sam, qwm, swm)
    # grouped FP8 (2 experts)
    qf, sf = tfq.tfq_quantize_rows(xd, "fp8", 448.0)
    qe, se = tfq.tfq_quantize_weight_per_channel(wd, "fp8", 448.0)
    qe2, se2 = torch.stack([qe, qe.flip(0)]), torch.stack([se, se.flip(0)])
    off = torch.tensor([0, 300, M], dtype=torch.int32, device="cuda")
    yg0 = tfq.tfq_grouped_scaled_mm_fp8(qf, sf, qe2, se2, off)
    tfq.tfq_set_autotune(1)
    y1, c1 = tfq.tfq_scaled_mm_int8(a, dev_f32(sa), b, dev_f32(sb), want_acc=True)
    yb1 = tfq.tfq_scaled_mm_fp8(qa8, sa8, qw8, sw8, 128)
    ym1 = tfq.tfq_scaled_mm_mxfp8(qam, sam, qwm, swm)
    yg1 = tfq.tfq_grouped_scaled_mm_fp8(qf, sf, qe2, se2, off)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(c0, c1)
    assert torch.equal(yb0, yb1) and torch.equal(ym0, ym1) and torch.equal(yg0, yg1)
    for kind, groups in (("int8", 0), ("fp8_block", 0), ("mxfp8", 0), ("grouped_fp8", 2)):
        cfg = tfq.tfq_autotune_lookup(kind, M, N, K, None, groups)
        assert cfg is not None and cfg[1] in (1, 2, 4, 8), kind
        if kind != "int8":
            assert cfg[0] == 0, kind   # only the 256x256 kernel serves these


def test_captured_stream_is_not_tuned_and_replays_match(tfq):
    M, N, K = 512, 768, 640
    rng = np.random.default_rng(9)
    qa, sa = _fp8(rng, M, K)
    qb, sb = _fp8(rng, N, K)
    a, b, sad, sbd = dev_u8(qa), dev_u8(qb), dev_f32(sa), dev_f32(sb)
    y_eager = tfq.tfq_scaled_mm_fp8(a, sad, b, sbd)
    torch.cuda.synchronize()
    tfq.tfq_set_autotune(1)
    y = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    g = torch.cuda.CUDAGraph()
    say("autotune under graph capture")
    with torch.cuda.graph(g):
        tfq.tfq_scaled_mm_fp8(a, sad, b, sbd, y=y)
    torch.cuda.synchronize()
    assert tfq.tfq_autotune_lookup("fp8", M, N, K) is None
    for r in range(3):
        y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), r
