"""Calls on a stream other than torch's current one: the tensors a wrapper
allocates itself (outputs, the fused Linear's workspace) must belong to the
caller's stream, so that torch's caching allocator cannot hand their memory
to work on the current stream while the kernels still read or write it."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev_bf16, host_bits, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module")
def tfq():
    import int8_w8a8_quantized_amd as m

    return m


def test_fused_linear_on_side_stream(tfq):
    """The fused Linear on a side stream with its workspace allocated inside
    the call; right after it returns, the current stream allocates blocks of
    the workspace's and output's sizes and overwrites them.  The result must
    equal the same call on the current stream bit for bit."""
    d = synth.make("c3_image_dit", M=4096, K=3072, N=12288)
    M, K = d["x"].shape
    say(f"fused linear side stream M={M} K={K} N={d['w'].shape[0]}")
    x, w = dev_bf16(d["x"]), dev_bf16(d["w"])
    wq, ws = tfq.tfq_quantize_weight_per_channel(w, "fp8", 448.0)
    ref = tfq.tfq_quant_linear_fused(x, wq, ws, "fp8", 448.0)
    torch.cuda.synchronize()
    ref_bits = host_bits(ref)
    need = tfq.tfq_quant_linear_workspace_bytes(M, K, "fp8", 0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        y = tfq.tfq_quant_linear_fused(x, wq, ws, "fp8", 448.0, stream=side)
        # the current stream is idle: these fills start at once, while the
        # side stream's kernels may still use their blocks if they were shared
        junk = [torch.empty(max(need, 1), dtype=torch.uint8, device="cuda").fill_(0x7E)
                for _ in range(4)]
        junk_y = torch.empty_like(ref).fill_(1.0)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(y), ref_bits), f"side-stream result differs (rep {rep})"
        del y, junk, junk_y


def test_quantize_and_gemm_outputs_on_side_stream(tfq):
    """Outputs allocated by tfq_quantize_rows and tfq_scaled_mm_fp8 on a side
    stream are not reused by the current stream while in flight."""
    d = synth.make("c3_image_dit", M=2048, K=3072, N=4096)
    x, w = dev_bf16(d["x"]), dev_bf16(d["w"])
    say("quantize_rows + scaled_mm_fp8 side stream 2048x3072x4096")
    wq, ws = tfq.tfq_quantize_weight_per_channel(w, "fp8", 448.0)
    qa, sa = tfq.tfq_quantize_rows(x, "fp8", 448.0)
    ref = tfq.tfq_scaled_mm_fp8(qa, sa, wq, ws)
    torch.cuda.synchronize()
    ref_q, ref_y = host_bits(qa), host_bits(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    q2, s2 = tfq.tfq_quantize_rows(x, "fp8", 448.0, stream=side)
    y2 = tfq.tfq_scaled_mm_fp8(q2, s2, wq, ws, stream=side)
    junk = [torch.empty_like(ref).fill_(-2.0), torch.empty_like(qa).fill_(0x11)]
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(q2), ref_q)
    assert np.array_equal(host_bits(y2), ref_y)
    del junk
