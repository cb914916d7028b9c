"""GPU parity at the five workloads' full sizes, in the launch configuration
bench.py times.

Quantisation parity is full-size and bit-exact (codes and scales).  GEMM
outputs of c1, c2, c3 and c5 are checked in full against the oracle's
BLAS-formed exact references (linear_ref_fast / int8_linear_fast, pinned bit
for bit to the loop versions): INT8 bit-exact, FP8 within max|y - y_ref| <=
2^-7 |y_ref| + 1e-3 max_row|y_ref|.  The c4 FFN pair (2 x 10.7 TFLOP per
qmax) is checked on one seeded row of every 256-row tile plus the first and
last 16 rows (the ragged last tile included).  In the FFN pair the second
quantisation is checked on the GPU's own G (so tolerance in the first GEMM
cannot compound into the bit-exact check), and the down GEMM reference uses
those codes.

Sources: TeleFuser "Quantization", "tf-kernel FP8: online W8A8", "Scaled FP8
checkpoints: W8A8", "Core ideas", "Validation" (E_max / E_rel, reported only);
LightX2V "模型量化技术", table "量化模式" and "MiniMax-H3 FP8 FP16 累加".
"""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from gpu_util import (assert_fp8_tolerance, bf16_to_f64, dev_bf16, host_bits, needs_gpu, say)

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module")
def tfq():
    import int8_w8a8_quantized_amd as m

    return m


def sample_rows(M, seed=0):
    """The first and last 16 rows and one seeded row in every 256-row tile."""
    rng = np.random.default_rng(seed + M)
    per_tile = [t + int(rng.integers(0, min(256, M - t))) for t in range(0, M, 256)]
    return np.unique(np.concatenate([np.arange(min(16, M)), np.arange(max(0, M - 16), M),
                                     np.asarray(per_tile, dtype=np.int64)])).astype(np.int64)


def _quant_parity(tfq, xd, xbits, qtype, qmax, group=0, what=""):
    say(f"{what}: quantize_rows {qtype} qmax={qmax} group={group} shape={tuple(xbits.shape)}")
    q, s = tfq.tfq_quantize_rows(xd, qtype, qmax, group)
    torch.cuda.synchronize()
    qe, se = orc.quantize_rows(xbits, qtype, qmax, group)
    assert np.array_equal(host_bits(s).view(np.uint32), se.view(np.uint32)), f"{what} scales"
    assert np.array_equal(host_bits(q), qe), f"{what} codes"
    return q, s, qe, se


def test_c1_tiny_fp8_full(tfq):
    d = synth.make("c1_tiny_fp8")
    xd, wd = dev_bf16(d["x"]), dev_bf16(d["w"])
    wq, ws = tfq.tfq_quantize_weight_per_channel(wd, "fp8", 448.0)
    qe_w, se_w = orc.quantize_rows(d["w"], "fp8", 448.0)
    assert np.array_equal(host_bits(wq), qe_w) and np.array_equal(host_bits(ws), se_w)
    _, _, qe, se = _quant_parity(tfq, xd, d["x"], "fp8", 448.0, what="c1")
    say("c1: quant_linear_fused 128x256 . 512x256")
    y = tfq.tfq_quant_linear_fused(xd, wq, ws, "fp8", 448.0)
    torch.cuda.synchronize()
    ref = orc.linear_ref(qe, se, qe_w, se_w, "fp8")
    assert_fp8_tolerance(host_bits(y), ref, "c1 full")


def test_c2_int8(tfq):
    d = synth.make("c2_int8")
    xd, wd = dev_bf16(d["x"]), dev_bf16(d["w"])
    qa, sa, qe, se = _quant_parity(tfq, xd, d["x"], "int8", 127.0, what="c2 X")
    qw, sw, qe_w, se_w = _quant_parity(tfq, wd, d["w"], "int8", 127.0, what="c2 W")
    say("c2: scaled_mm_int8 4096x3072x3072")
    y, acc = tfq.tfq_scaled_mm_int8(qa, sa, qw, sw, None, None, True, True)
    torch.cuda.synchronize()
    # every one of the 4096 x 3072 outputs, bit-exact
    acc_e, y_e = orc.int8_linear_fast(qe, se, qe_w, se_w)
    assert np.array_equal(host_bits(acc).astype(np.int64), acc_e), "c2 INT32 sums"
    assert np.array_equal(host_bits(y), y_e), "c2 BF16 outputs"
    say("c2: quant_linear_fused int8")
    y2 = tfq.tfq_quant_linear_fused(xd, qw, sw, "int8", 127.0)
    torch.cuda.synchronize()
    assert torch.equal(y2, y)


def test_c3_image_dit(tfq):
    d = synth.make("c3_image_dit")
    xd, wd = dev_bf16(d["x"]), dev_bf16(d["w"])
    _, _, qe, se = _quant_parity(tfq, xd, d["x"], "fp8", 448.0, what="c3 X")
    wq, ws, qe_w, se_w = _quant_parity(tfq, wd, d["w"], "fp8", 448.0, what="c3 W")
    say("c3: quant_linear_fused 7145x3072 . 12288x3072")
    y = tfq.tfq_quant_linear_fused(xd, wq, ws, "fp8", 448.0)
    torch.cuda.synchronize()
    # every output against the exact binary64 reference
    ref_all = orc.linear_ref_fast(qe, se, qe_w, se_w, "fp8")
    yb_all = host_bits(y)
    r = assert_fp8_tolerance(yb_all, ref_all, "c3 full")
    del ref_all
    rows = sample_rows(d["spec"].M)
    yb = yb_all[rows]
    # operator error against the unquantised BF16 product (report only)
    true = bf16_to_f64(d["x"][rows]) @ bf16_to_f64(d["w"]).T
    emax, erel = orc.error_measures(bf16_to_f64(yb), true)
    print(f"c3: max err/allowance {r:.3f}; vs unquantised BF16 GEMM: E_max {emax:.4g} "
          f"E_rel {erel:.4g}")


@pytest.fixture(scope="module")
def c4():
    return synth.make("c4_video_dit")


@pytest.mark.parametrize("qmax", [448.0, 14.0, 7.0])
def test_c4_video_dit_ffn_pair(tfq, c4, qmax):
    d = c4
    M, K, N, N2 = d["spec"].M, d["spec"].K, d["spec"].N, d["spec"].n_down
    xd = dev_bf16(d["x"])
    wq_up, ws_up = tfq.tfq_quantize_weight_per_channel(dev_bf16(d["w"]), "fp8", 448.0)
    wq_dn, ws_dn = tfq.tfq_quantize_weight_per_channel(dev_bf16(d["w_down"]), "fp8", 448.0)
    rows = sample_rows(M)
    qx, sx, qe_x, se_x = _quant_parity(tfq, xd, d["x"], "fp8", qmax, what=f"c4 X qmax={qmax}")
    say(f"c4 qmax={qmax}: up GEMM + GELU {M}x{N}x{K}")
    g = tfq.tfq_scaled_mm_fp8(qx, sx, wq_up, ws_up, 0, None, "gelu_tanh")
    torch.cuda.synchronize()
    qe_up, se_up = orc.quantize_rows(d["w"], "fp8", 448.0)
    ref_g = orc.linear_ref_fast(qe_x, se_x, qe_up, se_up, "fp8", gelu=True, rows=rows)
    gb = host_bits(g)
    assert_fp8_tolerance(gb[rows], ref_g, f"c4 up+gelu qmax={qmax}")
    del qx
    # second quantisation on the GPU's own G, full size, bit-exact
    qg, sg, qe_g, se_g = _quant_parity(tfq, g, gb, "fp8", qmax, what=f"c4 G qmax={qmax}")
    del gb, g
    say(f"c4 qmax={qmax}: down GEMM {M}x{N2}x{N}")
    y = tfq.tfq_scaled_mm_fp8(qg, sg, wq_dn, ws_dn, 0, None, None)
    torch.cuda.synchronize()
    qe_dn, se_dn = orc.quantize_rows(d["w_down"], "fp8", 448.0)
    ref_y = orc.linear_ref_fast(np.ascontiguousarray(qe_g[rows]), se_g[rows], qe_dn, se_dn, "fp8")
    assert_fp8_tolerance(host_bits(y)[rows], ref_y, f"c4 down qmax={qmax}")
    assert host_bits(qg).shape == (M, N)


def test_c5_block_fp8(tfq):
    d = synth.make("c5_block_fp8")
    xd, wd = dev_bf16(d["x"]), dev_bf16(d["w"])
    qa, sa, qe, se = _quant_parity(tfq, xd, d["x"], "fp8", 448.0, group=128, what="c5 X groups")
    say("c5: weight 128x128 blocks")
    qw, sw = tfq.tfq_quantize_weight_per_channel(wd, "fp8", 448.0, 128)
    torch.cuda.synchronize()
    qe_w, se_w = orc.quantize_blocks(d["w"], "fp8", 448.0, 128)
    assert np.array_equal(host_bits(qw), qe_w) and np.array_equal(host_bits(sw), se_w)
    say("c5: block-scaled GEMM 8192x5120x5120")
    y = tfq.tfq_scaled_mm_fp8(qa, sa, qw, sw, 128)
    torch.cuda.synchronize()
    ref = orc.linear_ref_fast(qe, se, qe_w, se_w, "fp8", scale_block=128)
    assert_fp8_tolerance(host_bits(y), ref, "c5 full")
