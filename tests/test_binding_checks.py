"""Host checks of the Python binding's argument validation (no GPU).

Every entry checks its tensors before their pointers reach the library:
element type, shape (K of both GEMM operands, scale and output sizes), row
or whole contiguity, and device memory.  A wrong tensor would otherwise be
reinterpreted by the kernels, or read past its end.  The checks run in that
order, so host tensors reach every one of them here.
"""
import pytest
import torch

import int8_w8a8_quantized_amd as tfq

bf16 = torch.bfloat16


def _raises(name, fn, *a, **kw):
    with pytest.raises((TypeError, ValueError), match=name):
        fn(*a, **kw)


def test_quantize_rows_checks():
    x = torch.zeros(4, 256, dtype=bf16)
    _raises("x", tfq.tfq_quantize_rows, x.float())                    # dtype
    _raises("x", tfq.tfq_quantize_rows, x[None])                      # 3-D
    _raises("x", tfq.tfq_quantize_rows, torch.zeros(4, 512, dtype=bf16)[:, ::2])  # strided columns
    _raises("GPU memory", tfq.tfq_quantize_rows, x)                   # host tensor
    _raises("q_out", tfq.tfq_quantize_rows, x, q_out=torch.zeros(4, 128, dtype=torch.uint8))
    _raises("q_out", tfq.tfq_quantize_rows, x, q_out=torch.zeros(4, 256, dtype=torch.int16))
    _raises("scale_out", tfq.tfq_quantize_rows, x, "fp8", 448.0, 128,
            scale_out=torch.zeros(4, dtype=torch.float32))            # groups need [rows, cols/128]
    _raises("row_index", tfq.tfq_quantize_rows_gather, x, torch.zeros(3, dtype=torch.int64))
    _raises("w", tfq.tfq_quantize_weight_per_channel, x.half())


def test_gemm_checks():
    a = torch.zeros(64, 256, dtype=torch.uint8)
    b = torch.zeros(32, 256, dtype=torch.uint8)
    sa, sb = torch.ones(64), torch.ones(32)
    _raises("b_q", tfq.tfq_scaled_mm_fp8, a, sa, torch.zeros(32, 128, dtype=torch.uint8), sb)  # K
    _raises("a_q", tfq.tfq_scaled_mm_fp8, a.float(), sa, b, sb)
    _raises("a_scale", tfq.tfq_scaled_mm_fp8, a, torch.ones(63), b, sb)
    _raises("b_scale", tfq.tfq_scaled_mm_fp8, a, sa, b, sb.double())
    _raises("b_scale", tfq.tfq_scaled_mm_fp8, a, torch.ones(64, 2), b, torch.ones(32), 128)
    _raises("bias", tfq.tfq_scaled_mm_fp8, a, sa, b, sb, 0, torch.zeros(31, dtype=bf16))
    _raises("y", tfq.tfq_scaled_mm_fp8, a, sa, b, sb, y=torch.zeros(64, 32))
    _raises("b_q", tfq.tfq_scaled_mm_fp8, a, sa, b.t(), sb)           # transposed view: K differs
    _raises("a_q", tfq.tfq_scaled_mm_fp8, torch.zeros(256, 64, dtype=torch.uint8).t(), sa,
            torch.zeros(32, 64, dtype=torch.uint8), sb)              # not contiguous
    _raises("GPU memory", tfq.tfq_scaled_mm_fp8, a, sa, b, sb)
    _raises("acc", tfq.tfq_scaled_mm_int8, a.view(torch.int8), sa, b.view(torch.int8), sb,
            want_acc=True, acc=torch.zeros(64, 32, dtype=torch.int64))
    e = torch.zeros(2, 32, 256, dtype=torch.uint8)
    off = torch.zeros(3, dtype=torch.int32)
    _raises("group_offsets", tfq.tfq_grouped_scaled_mm_fp8, a, sa, e, torch.ones(2, 32), off[:2])
    _raises("b_scale", tfq.tfq_grouped_scaled_mm_fp8, a, sa, e, torch.ones(32), off)
    _raises("w_q", tfq.tfq_quant_linear_fused, torch.zeros(64, 256, dtype=bf16),
            torch.zeros(32, 255, dtype=torch.uint8), sb)


def test_mx_checks():
    x = torch.zeros(8, 256, dtype=bf16)
    _raises("scale_out", tfq.tfq_quantize_mx, x, scale_out=torch.zeros(2, 8, 3, dtype=torch.uint8))
    _raises("q_out", tfq.tfq_quantize_mxfp4, x, q_out=torch.zeros(8, 256, dtype=torch.uint8))
    _raises("fmt", tfq.tfq_quantize_mxfp6, x, "e5m2")
    a, b = torch.zeros(2, 8, 96, dtype=torch.uint8), torch.zeros(2, 16, 96, dtype=torch.uint8)
    sa, sb = torch.zeros(2, 8, 4, dtype=torch.uint8), torch.zeros(2, 16, 4, dtype=torch.uint8)
    _raises("q_out", tfq.tfq_quantize_mxfp6, x, q_out=torch.zeros(8, 192, dtype=torch.uint8))
    _raises("a_scale", tfq.tfq_scaled_mm_mxfp6, a, sb, b, sb)
    _raises("fmt", tfq.tfq_scaled_mm_mxfp6, a, sa, b, sb, "e4m3")
    _raises("a_q", tfq.tfq_scaled_mm_mxfp6, torch.zeros(8, 192, dtype=torch.uint8), sa,
            torch.zeros(16, 192, dtype=torch.uint8), sb)
    _raises("b_q", tfq.tfq_scaled_mm_mxfp6, a, sa, torch.zeros(3, 16, 96, dtype=torch.uint8), sb)
    _raises("GPU memory", tfq.tfq_scaled_mm_mxfp6, a, sa, b, sb)
    _raises("b_scale", tfq.tfq_scaled_mm_mxfp8, torch.zeros(8, 256, dtype=torch.uint8), sa,
            torch.zeros(16, 256, dtype=torch.uint8), sa)
    _raises("b_q", tfq.tfq_scaled_mm_mxfp4, torch.zeros(8, 128, dtype=torch.uint8), sa,
            torch.zeros(16, 128, dtype=torch.int8), sb)


def test_kv_and_encoder_checks():
    kv = torch.zeros(4, 2, 128, dtype=bf16)
    cache = torch.zeros(10, 2, 128, dtype=torch.uint8)
    cs = torch.zeros(10, 2)
    slot = torch.zeros(4, dtype=torch.int32)
    _raises("kv", tfq.tfq_kv_cache_store, kv.transpose(1, 2).contiguous().transpose(1, 2), slot,
            cache, cs)                                                # head_dim not contiguous
    _raises("slot_index", tfq.tfq_kv_cache_store, kv, slot.long(), cache, cs)
    _raises("cache_scale", tfq.tfq_kv_cache_store, kv, slot, cache, torch.zeros(10, 3))
    _raises("GPU memory", tfq.tfq_kv_cache_store, kv, slot, cache, cs)
    _raises("out", tfq.tfq_kv_cache_load, cache, cs, slot, out=torch.zeros(4, 2, 128, dtype=torch.int8))
    _raises("out", tfq.tfq_kv_cache_load, cache, cs, slot, out=torch.zeros(4, 2, 64, dtype=bf16))
    _raises("x", tfq.tfq_e4m3fn_encode_f32, torch.zeros(8, dtype=bf16))
    _raises("q", tfq.tfq_e4m3fn_encode_f32, torch.zeros(8), torch.zeros(4, dtype=torch.uint8))
