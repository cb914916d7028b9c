"""Seeded random shapes through the per-channel FP8 and INT8 GEMMs, the
block-scaled FP8 GEMM, the grouped (routed) FP8 GEMM, the fused Linear and
the MXFP8 / MXFP4 / MXFP6 quantise + GEMM pairs, against the oracle.

Each case draws M, N and K (ragged against the 256-row, 256- and 192-column
tiles and the 128-byte K stages) and per-row magnitudes spread over
2^-6 .. 2^6 from its own seed, with a bias or none and GELU-tanh or none
set per case so that every mode meets each of them; three size
classes put the default launch configuration on each kernel (under 64
256x256 tiles: the two-per-CU kernel; from 64 tiles: the 256x256 or the
256x192 tiles).  The GPU's quantiser output is checked bit for bit against
the oracle's (TeleFuser "Quantization", "Scaled FP8 checkpoints: W8A8"),
then the GEMM on the oracle's codes: INT8 sums and plain BF16 outputs bit
for bit, FP8 (and INT8 with GELU) within the FP8 tolerance of the exact
binary64 reference (TeleFuser "Quantization", "tf-kernel FP8: online W8A8";
LightX2V "模型量化技术", table "量化模式", fp8-b128-deepgemm for the block
mode; TeleFuser "Quantization", "Other quantized data paths" for the routed
rows).
"""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from gpu_util import (assert_fp8_tolerance, dev_bf16, dev_f32, dev_u8, host_bits, mx6_ungrouped,
                      mx_ungrouped, needs_gpu, say)

pytestmark = [pytest.mark.gpu, needs_gpu]

# (M range, N range, K range) per size class; N and K are drawn as multiples
# of the step given with them
CLASSES = {
    "small": ((1, 520), (8, 768, 8), (16, 1536, 16)),      # <= 9 256x256 tiles
    "mid": ((1800, 2600), (1840, 2640, 8), (128, 1024, 16)),  # 64..121 tiles
    "large": ((5200, 6200), (4400, 5600, 8), (64, 400, 16)),  # 378..550 tiles
}
BLOCK_CLASSES = {
    "small": ((1, 520), (128, 768, 128), (128, 768, 128)),
    "mid": ((1800, 2600), (1920, 2560, 128), (128, 640, 128)),
    "large": ((5200, 6200), (4480, 5632, 128), (128, 384, 128)),
}


@pytest.fixture(scope="module")
def tfq():
    import int8_w8a8_quantized_amd as m

    m.tfq_set_autotune(0)
    return m


def _pick(rng, lo, hi, step=1):
    return int(rng.integers(lo // step, hi // step + 1)) * step


def _shape(rng, classes, cls):
    (m0, m1), (n0, n1, ns), (k0, k1, ks) = classes[cls]
    return _pick(rng, m0, m1), _pick(rng, n0, n1, ns), _pick(rng, k0, k1, ks)


def _inputs(rng, M, N, K):
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[rng.random((M, K)) < 0.01] *= 20
    x *= np.exp2(rng.integers(-6, 7, (M, 1))).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bias = (rng.standard_normal(N) * 0.5).astype(np.float32)
    return synth.to_bf16_bits(x), synth.to_bf16_bits(w), synth.to_bf16_bits(bias)


SEEDS = {"small": 101, "mid": 202, "large": 303}
G_ = "gelu_tanh"
# (bias, epilogue) of each case, so that every mode meets both epilogues and
# both bias cases across its size classes
OPTIONS = {
    ("fp8", "small"): (True, G_), ("fp8", "mid"): (False, G_), ("fp8", "large"): (True, None),
    ("int8", "small"): (False, None), ("int8", "mid"): (True, None), ("int8", "large"): (True, G_),
    ("block", "small"): (True, G_), ("block", "mid"): (False, None), ("block", "large"): (True, G_),
    ("grouped", "small"): (True, G_), ("grouped", "mid"): (False, None),
    ("fused", "fp8"): (True, G_), ("fused", "int8"): (True, None),
    ("mxfp8", "small"): (True, None), ("mxfp8", "mid"): (False, G_),
    ("mxfp4", "small"): (False, G_), ("mxfp4", "mid"): (True, None),
    ("e2m3", "small"): (True, G_), ("e2m3", "mid"): (False, None),
    ("e3m2", "small"): (False, None), ("e3m2", "mid"): (True, G_),
}
MX_CLASSES = {
    "small": ((1, 520), (8, 768, 8), (128, 1536, 128)),
    "mid": ((1800, 2600), (1840, 2640, 8), (128, 768, 128)),
}


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
@pytest.mark.parametrize("cls", list(CLASSES))
def test_per_channel(tfq, qtype, cls):
    rng = np.random.default_rng(SEEDS[cls] + (7 if qtype == "int8" else 0))
    M, N, K = _shape(rng, CLASSES, cls)
    use_bias, epi = OPTIONS[(qtype, cls)]
    xb, wb, bb = _inputs(rng, M, N, K)
    qmax = 448.0 if qtype == "fp8" else 127.0
    say(f"random per-channel {qtype} {cls} M={M} N={N} K={K} bias={use_bias} epi={epi}")
    qa, sa = tfq.tfq_quantize_rows(dev_bf16(xb), qtype, qmax)
    qb, sb = tfq.tfq_quantize_weight_per_channel(dev_bf16(wb), qtype, qmax)
    qa_e, sa_e = orc.quantize_rows(xb, qtype, qmax)
    qb_e, sb_e = orc.quantize_rows(wb, qtype, qmax)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(qa), qa_e) and np.array_equal(host_bits(sa), sa_e)
    assert np.array_equal(host_bits(qb), qb_e) and np.array_equal(host_bits(sb), sb_e)
    bd = dev_bf16(bb) if use_bias else None
    bias = bb if use_bias else None
    if qtype == "fp8":
        y = tfq.tfq_scaled_mm_fp8(qa, sa, qb, sb, 0, bd, epi)
    else:
        y, acc = tfq.tfq_scaled_mm_int8(qa, sa, qb, sb, bd, epi, want_acc=True)
    torch.cuda.synchronize()
    if qtype == "int8":
        acc_e, y_e = orc.int8_linear_fast(qa_e, sa_e, qb_e, sb_e, bias=bias)
        assert np.array_equal(host_bits(acc).astype(np.int64), acc_e), "INT32 sums differ"
        if epi is None:
            assert np.array_equal(host_bits(y), y_e), "INT8 BF16 outputs differ"
            return
    ref = orc.linear_ref_fast(qa_e, sa_e, qb_e, sb_e, qtype, bias=bias, gelu=epi is not None)
    assert_fp8_tolerance(host_bits(y), ref, f"{qtype} {cls} M={M} N={N} K={K}")


@pytest.mark.parametrize("cls", list(BLOCK_CLASSES))
def test_block_scaled(tfq, cls):
    rng = np.random.default_rng(SEEDS[cls] + 13)
    M, N, K = _shape(rng, BLOCK_CLASSES, cls)
    use_bias, epi = OPTIONS[("block", cls)]
    xb, wb, bb = _inputs(rng, M, N, K)
    say(f"random block-scaled fp8 {cls} M={M} N={N} K={K} bias={use_bias} epi={epi}")
    qa, sa = tfq.tfq_quantize_rows(dev_bf16(xb), "fp8", 448.0, 128)
    qb, sb = tfq.tfq_quantize_weight_per_channel(dev_bf16(wb), "fp8", 448.0, 128)
    qa_e, sa_e = orc.quantize_rows(xb, "fp8", 448.0, 128)
    qb_e, sb_e = orc.quantize_blocks(wb, "fp8", 448.0, 128)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(qa), qa_e) and np.array_equal(host_bits(sa), sa_e)
    assert np.array_equal(host_bits(qb), qb_e) and np.array_equal(host_bits(sb), sb_e)
    y = tfq.tfq_scaled_mm_fp8(qa, sa, qb, sb, 128, dev_bf16(bb) if use_bias else None, epi)
    torch.cuda.synchronize()
    ref = orc.linear_ref_fast(qa_e, sa_e, qb_e, sb_e, "fp8", scale_block=128,
                              bias=bb if use_bias else None, gelu=epi is not None)
    assert_fp8_tolerance(host_bits(y), ref, f"block {cls} M={M} N={N} K={K}")


@pytest.mark.parametrize("cls", ["small", "mid"])
def test_grouped(tfq, cls):
    """Routed rows: random group sizes, some groups empty, the last group
    ending before M (rows past it are left as they were)."""
    rng = np.random.default_rng(SEEDS[cls] + 29)
    M, N, K = _shape(rng, CLASSES, cls)
    G = int(rng.integers(2, 9))
    use_bias, epi = OPTIONS[("grouped", cls)]
    xb, _, _ = _inputs(rng, M, N, K)
    w = (rng.standard_normal((G, N, K)) * 0.02).astype(np.float32)
    wb = synth.to_bf16_bits(w)
    bb = synth.to_bf16_bits((rng.standard_normal((G, N)) * 0.5).astype(np.float32))
    cuts = np.sort(rng.integers(0, M + 1, G - 1))
    end = int(rng.integers(max(int(cuts[-1]), M - M // 8), M + 1))
    off = np.concatenate([[0], cuts, [end]]).astype(np.int32)
    off[rng.integers(1, G)] = off[rng.integers(0, G)]  # (may empty a group)
    off = np.maximum.accumulate(off).astype(np.int32)
    say(f"random grouped fp8 {cls} M={M} N={N} K={K} G={G} off={off.tolist()} "
        f"bias={use_bias} epi={epi}")
    qa_e, sa_e = orc.quantize_rows(xb, "fp8", 448.0)
    qe = np.stack([orc.quantize_rows(wb[g], "fp8", 448.0)[0] for g in range(G)])
    se = np.stack([orc.quantize_rows(wb[g], "fp8", 448.0)[1] for g in range(G)])
    y = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    y = tfq.tfq_grouped_scaled_mm_fp8(dev_u8(qa_e), dev_f32(sa_e), dev_u8(qe), dev_f32(se),
                                      torch.from_numpy(off).cuda(),
                                      dev_bf16(bb) if use_bias else None, epi, y)
    torch.cuda.synchronize()
    yb = host_bits(y)
    for g in range(G):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi == lo:
            continue
        ref = orc.linear_ref_fast(qa_e[lo:hi], sa_e[lo:hi], qe[g], se[g], "fp8",
                                  bias=bb[g] if use_bias else None, gelu=epi is not None)
        assert_fp8_tolerance(yb[lo:hi], ref, f"grouped {cls} group {g} rows {lo}..{hi}")
    assert not yb[int(off[-1]):].any(), "rows past the last group were written"


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
def test_fused_strided(tfq, qtype):
    """The fused Linear on a column slice (ld_x > K) of a random shape equals
    the oracle's quantisation and Linear."""
    rng = np.random.default_rng(404 + (1 if qtype == "int8" else 0))
    M, N, K = _shape(rng, CLASSES, "mid")
    LD = K + _pick(rng, 8, 256, 8)
    use_bias, epi = OPTIONS[("fused", qtype)]
    xw, wb, bb = _inputs(rng, M, N, LD)
    wb = np.ascontiguousarray(wb[:, :K])
    qmax = 448.0 if qtype == "fp8" else 127.0
    say(f"random fused {qtype} M={M} N={N} K={K} ld={LD} bias={use_bias} epi={epi}")
    xd = dev_bf16(xw)[:, :K]
    wq, ws = tfq.tfq_quantize_weight_per_channel(dev_bf16(wb), qtype, qmax)
    y = tfq.tfq_quant_linear_fused(xd, wq, ws, qtype, qmax, 0, dev_bf16(bb) if use_bias else None,
                                   epi)
    torch.cuda.synchronize()
    qa_e, sa_e = orc.quantize_rows(np.ascontiguousarray(xw[:, :K]), qtype, qmax)
    qb_e, sb_e = orc.quantize_rows(wb, qtype, qmax)
    bias = bb if use_bias else None
    if qtype == "int8" and epi is None:
        _, y_e = orc.int8_linear_fast(qa_e, sa_e, qb_e, sb_e, bias=bias)
        assert np.array_equal(host_bits(y), y_e)
    else:
        ref = orc.linear_ref_fast(qa_e, sa_e, qb_e, sb_e, qtype, bias=bias, gelu=epi is not None)
        assert_fp8_tolerance(host_bits(y), ref, f"fused {qtype} M={M} N={N} K={K}")


@pytest.mark.parametrize("kind", ["mxfp8", "mxfp4", "e2m3", "e3m2"])
@pytest.mark.parametrize("cls", list(MX_CLASSES))
def test_mx(tfq, kind, cls):
    """MX quantise + GEMM on random shapes, with magnitudes that change by up
    to 2^+-6 from one 32-element block to the next (a scale applied to the
    wrong block fails): codes and E8M0 scales bit-exact, then the GEMM on
    the GPU's codes within the FP8 tolerance (TeleFuser "Quantization",
    "Offline conversion": 32-value blocks with E8M0 scales).  The mid class
    is checked on the first and last 8 rows and one row of every 256-row
    tile."""
    rng = np.random.default_rng(SEEDS[cls] + 31 + ["mxfp8", "mxfp4", "e2m3", "e3m2"].index(kind))
    M, N, K = _shape(rng, MX_CLASSES, cls)
    use_bias, epi = OPTIONS[(kind, cls)]

    def blocky(rows, sigma):
        x = rng.standard_normal((rows, K)) * sigma
        x *= np.exp2(rng.integers(-6, 7, (rows, K // 32))).repeat(32, axis=1)
        return synth.to_bf16_bits(x.astype(np.float32))

    xb, wb = blocky(M, 1.0), blocky(N, 0.02)
    bb = synth.to_bf16_bits((rng.standard_normal(N) * 0.5).astype(np.float32))
    say(f"random {kind} {cls} M={M} N={N} K={K} bias={use_bias} epi={epi}")
    bd, bias, gelu = (dev_bf16(bb) if use_bias else None), (bb if use_bias else None), epi is not None
    if kind == "mxfp8":
        qa, sa = tfq.tfq_quantize_mx(dev_bf16(xb))
        qb, sb = tfq.tfq_quantize_mx(dev_bf16(wb))
        y = tfq.tfq_scaled_mm_mxfp8(qa, sa, qb, sb, bd, epi)
        (qa_e, sa_e), (qb_e, sb_e) = orc.quantize_mx(xb), orc.quantize_mx(wb)
        codes = host_bits
    elif kind == "mxfp4":
        qa, sa = tfq.tfq_quantize_mxfp4(dev_bf16(xb))
        qb, sb = tfq.tfq_quantize_mxfp4(dev_bf16(wb))
        y = tfq.tfq_scaled_mm_mxfp4(qa, sa, qb, sb, bd, epi)
        (qa_e, sa_e), (qb_e, sb_e) = orc.quantize_mx4(xb), orc.quantize_mx4(wb)
        codes = host_bits
    else:
        qa, sa = tfq.tfq_quantize_mxfp6(dev_bf16(xb), kind)
        qb, sb = tfq.tfq_quantize_mxfp6(dev_bf16(wb), kind)
        y = tfq.tfq_scaled_mm_mxfp6(qa, sa, qb, sb, kind, bd, epi)
        (qa_e, sa_e), (qb_e, sb_e) = orc.quantize_mx6(xb, kind), orc.quantize_mx6(wb, kind)

        def codes(t):
            return mx6_ungrouped(host_bits(t))
    torch.cuda.synchronize()
    assert np.array_equal(codes(qa), qa_e) and np.array_equal(mx_ungrouped(host_bits(sa)), sa_e)
    assert np.array_equal(codes(qb), qb_e) and np.array_equal(mx_ungrouped(host_bits(sb)), sb_e)
    rows = None
    if cls != "small":
        rows = np.unique(np.concatenate([np.arange(8), np.arange(M - 8, M),
                                         np.arange(0, M, 256) + rng.integers(0, 256, (M + 255) // 256)]))
        rows = rows[rows < M]
    if kind == "mxfp8":
        ref = orc.linear_mx_ref(qa_e, sa_e, qb_e, sb_e, bias=bias, gelu=gelu, rows=rows)
    elif kind == "mxfp4":
        ref = orc.linear_mx4_ref(qa_e, sa_e, qb_e, sb_e, bias=bias, gelu=gelu, rows=rows)
    else:
        ref = orc.linear_mx6_ref(qa_e, sa_e, qb_e, sb_e, kind, bias=bias, gelu=gelu, rows=rows)
    yb = host_bits(y)
    assert_fp8_tolerance(yb if rows is None else yb[rows], ref, f"{kind} {cls} M={M} N={N} K={K}")
