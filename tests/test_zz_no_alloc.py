"""The allocation-free fused Linear (tfq_quant_linear_fused_noalloc), through
the C ABI, against the workspace entry point tfq_quant_linear_fused: the same
kernels, so the same bits, and within the FP8 tolerance of the oracle
(TeleFuser "Quantization", "tf-kernel FP8: online W8A8").  Two calls in a
row, the second smaller, so the second runs over the first's leftovers in
the shared device scratch; then a call over the scratch limit is refused."""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from gpu_util import assert_fp8_tolerance, dev_bf16, host_bits, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module")
def tfq():
    import int8_w8a8_quantized_amd as m

    return m


def _case(tfq, seed, M, K, N, qtype, block=0, with_bias=False):
    rng = np.random.default_rng(seed)
    x = synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32) *
                           np.exp2(rng.integers(-6, 6, (M, 1))).astype(np.float32))
    w = synth.to_bf16_bits((0.02 * rng.standard_normal((N, K))).astype(np.float32))
    b = synth.to_bf16_bits(rng.standard_normal(N).astype(np.float32)) if with_bias else None
    qmax = 448.0 if qtype == "fp8" else 127.0
    xd, wd = dev_bf16(x), dev_bf16(w)
    bd = None if b is None else dev_bf16(b)
    wq, ws = tfq.tfq_quantize_weight_per_channel(wd, qtype, qmax, block)
    return x, w, b, xd, wd, bd, wq, ws, qmax


@pytest.mark.parametrize("qtype,block", [("fp8", 0), ("int8", 0), ("fp8", 128)])
def test_noalloc_matches_workspace_entry_point(tfq, qtype, block):
    outs = []
    for call, (M, K, N) in enumerate([(4100, 3072, 1536), (1000, 1024, 520)]):
        if block == 128:
            N = N // 128 * 128
        x, w, b, xd, wd, bd, wq, ws, qmax = _case(tfq, 100 * call + len(qtype) + block, M, K, N,
                                                   qtype, block, with_bias=call == 1)
        epi = "gelu_tanh" if call == 0 and qtype == "fp8" else None
        say(f"noalloc fused {qtype} block={block} call={call} M={M} K={K} N={N} epi={epi}")
        y_ref = tfq.tfq_quant_linear_fused(xd, wq, ws, qtype, qmax, block, bd, epi)
        y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
        tfq.tfq_quant_linear_fused_noalloc(xd, wq, ws, y, qtype, qmax, block, bd, epi)
        torch.cuda.synchronize()
        yb = host_bits(y)
        assert np.array_equal(yb, host_bits(y_ref)), f"call {call}: differs from the workspace call"
        rows = np.unique(np.concatenate([np.arange(8), np.arange(M - 8, M),
                                         np.random.default_rng(call).integers(0, M, 24)]))
        qa, sa = orc.quantize_rows(x, qtype, qmax, block)
        qw, sw = (orc.quantize_rows(w, qtype, qmax) if block == 0
                  else orc.quantize_blocks(w, qtype, qmax, block))
        if qtype == "fp8":
            ref = orc.linear_ref(qa, sa, qw, sw, "fp8", block, bias=b, gelu=epi is not None,
                                 rows=rows)
            assert_fp8_tolerance(yb[rows], ref, f"noalloc call {call}")
        else:
            _, y_e = orc.int8_linear(qa, sa, qw, sw, bias=b, rows=rows, want_acc=False)
            assert np.array_equal(yb[rows], y_e), f"noalloc INT8 call {call}"
        outs.append(yb)
    assert len(outs) == 2


def test_noalloc_refuses_inputs_beyond_its_scratch(tfq):
    M, K, N = 16384, 5120, 256  # 80 MiB of codes > 64 MiB
    assert tfq.tfq_quant_linear_workspace_bytes(M, K, "fp8", 0) > tfq.NOALLOC_WORKSPACE_BYTES
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
    ws = torch.ones((N,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    say("noalloc over the scratch limit")
    with pytest.raises(tfq.TfqError, match="WORKSPACE_TOO_SMALL"):
        tfq.tfq_quant_linear_fused_noalloc(x, wq, ws, y, "fp8", 448.0)
