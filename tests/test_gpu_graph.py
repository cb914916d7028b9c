"""GPU check that the library's entry points run inside a captured HIP graph.

One graph holds a pass over every compute entry point on fixed buffers:
* the FFN pair: per-token FP8 quantisation of X, up GEMM + GELU,
  quantisation of G, down GEMM;
* the fused Linear, and the INT8 and block-scaled FP8 Linears;
* the MXFP8, MXFP6 and MXFP4 quantise + GEMM pairs;
* the per-channel weight quantiser;
* the routed quantisation with the grouped GEMM;
* the FP8 KV-cache store and load, and the E4M3FN encoder.

The graph is replayed three times on fresh inputs, with eager calls and
synchronisations between the replays.  Each replay must equal the same calls
made eagerly, bit for bit: every kernel is deterministic.  That the eager
results agree with the oracle is what the other GPU tests check."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev_bf16, dev_f32, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]

M, K, NU, ND = 700, 640, 1536, 640      # ragged M (not a multiple of 256)
R = 900                                 # routed rows, in 3 expert groups
TOKENS, HEADS, HD, SLOTS = 300, 4, 128, 512


def _bf16(rng, shape, std):
    return dev_bf16(synth.to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32)))


def _inputs(seed):
    """What changes between replays: the activations, the KV vectors, a
    weight for the weight quantiser and the encoder's float input."""
    rng = np.random.default_rng(seed)
    return {"x": _bf16(rng, (M, K), 2.0), "kv": _bf16(rng, (TOKENS, HEADS, HD), 1.0),
            "w": _bf16(rng, (NU, K), 0.05),
            "f32": dev_f32((rng.standard_normal(4096) * 100).astype(np.float32))}


def _fixed(tfq):
    """Weights, routing and cache slots that every pass shares."""
    rng = np.random.default_rng(77)
    w_up, w_dn = _bf16(rng, (NU, K), 0.05), _bf16(rng, (ND, NU), 0.03)
    f = {"bu": _bf16(rng, (NU,), 0.1)}
    f["wu_q"], f["wu_s"] = tfq.tfq_quantize_weight_per_channel(w_up, "fp8")
    f["wd_q"], f["wd_s"] = tfq.tfq_quantize_weight_per_channel(w_dn, "fp8")
    f["wu_q8"], f["wu_s8"] = tfq.tfq_quantize_weight_per_channel(w_up, "int8", 127.0)
    f["wu_qb"], f["wu_sb"] = tfq.tfq_quantize_weight_per_channel(w_up, "fp8", 448.0, 128)
    f["m8q"], f["m8s"] = tfq.tfq_quantize_mx(w_up)
    f["m6q"], f["m6s"] = tfq.tfq_quantize_mxfp6(w_up, "e3m2")
    f["m4q"], f["m4s"] = tfq.tfq_quantize_mxfp4(w_up)
    experts = [tfq.tfq_quantize_weight_per_channel(_bf16(rng, (NU, K), 0.05), "fp8") for _ in range(3)]
    f["ex_q"] = torch.stack([q for q, _ in experts])
    f["ex_s"] = torch.stack([s for _, s in experts])
    f["route"] = torch.from_numpy(rng.integers(0, M, R).astype(np.int32)).cuda()
    f["goff"] = torch.tensor([0, 250, 600, R], dtype=torch.int32).cuda()
    slots = rng.permutation(SLOTS)[:TOKENS].astype(np.int32)
    f["slot"] = torch.from_numpy(slots).cuda()
    f["load"] = torch.from_numpy(slots[::-1].copy()).cuda()
    torch.cuda.synchronize()
    return f


def _alloc(tfq):
    d = "cuda"
    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    e = lambda shape, dt: torch.zeros(shape, dtype=dt, device=d)
    return {
        "qx": e((M, K), u8), "sx": e((M,), f32), "g": e((M, NU), bf), "qg": e((M, NU), u8),
        "sg": e((M,), f32), "y": e((M, ND), bf),
        "y_fused": e((M, NU), bf), "ws": e((tfq.tfq_quant_linear_workspace_bytes(M, K),), u8),
        "qx8": e((M, K), torch.int8), "sx8": e((M,), f32), "y8": e((M, NU), bf),
        "qxb": e((M, K), u8), "sxb": e((M, K // 128), f32), "yb": e((M, NU), bf),
        "qm8": e((M, K), u8), "sm8": e((K // 128, M, 4), u8), "ym8": e((M, NU), bf),
        "qm6": e((K // 128, M, 96), u8), "sm6": e((K // 128, M, 4), u8), "ym6": e((M, NU), bf),
        "qm4": e((M, K // 2), u8), "sm4": e((K // 128, M, 4), u8), "ym4": e((M, NU), bf),
        "wq": e((NU, K), u8), "wqs": e((NU,), f32),
        "qr": e((R, K), u8), "sr": e((R,), f32), "yr": e((R, NU), bf),
        "cache": e((SLOTS, HEADS, HD), u8), "cache_s": e((SLOTS, HEADS), f32),
        "kv_out": e((TOKENS, HEADS, HD), bf), "enc": e((4096,), u8),
    }


def _pass(t, f, i, o):
    """One call of every compute entry point, inputs i, outputs o."""
    x = i["x"]
    t.tfq_quantize_rows(x, "fp8", 448.0, 0, o["qx"], o["sx"])
    t.tfq_scaled_mm_fp8(o["qx"], o["sx"], f["wu_q"], f["wu_s"], 0, f["bu"], "gelu_tanh", o["g"])
    t.tfq_quantize_rows(o["g"], "fp8", 448.0, 0, o["qg"], o["sg"])
    t.tfq_scaled_mm_fp8(o["qg"], o["sg"], f["wd_q"], f["wd_s"], 0, None, None, o["y"])
    t.tfq_quant_linear_fused(x, f["wu_q"], f["wu_s"], "fp8", 448.0, 0, None, "gelu_tanh",
                             o["y_fused"], o["ws"])
    t.tfq_quantize_rows(x, "int8", 127.0, 0, o["qx8"], o["sx8"])
    t.tfq_scaled_mm_int8(o["qx8"], o["sx8"], f["wu_q8"], f["wu_s8"], None, None, True, False,
                         o["y8"])
    t.tfq_quantize_rows(x, "fp8", 448.0, 128, o["qxb"], o["sxb"])
    t.tfq_scaled_mm_fp8(o["qxb"], o["sxb"], f["wu_qb"], f["wu_sb"], 128, None, None, o["yb"])
    t.tfq_quantize_mx(x, o["qm8"], o["sm8"])
    t.tfq_scaled_mm_mxfp8(o["qm8"], o["sm8"], f["m8q"], f["m8s"], None, "gelu_tanh", o["ym8"])
    t.tfq_quantize_mxfp6(x, "e3m2", o["qm6"], o["sm6"])
    t.tfq_scaled_mm_mxfp6(o["qm6"], o["sm6"], f["m6q"], f["m6s"], "e3m2", None, None, o["ym6"])
    t.tfq_quantize_mxfp4(x, o["qm4"], o["sm4"])
    t.tfq_scaled_mm_mxfp4(o["qm4"], o["sm4"], f["m4q"], f["m4s"], f["bu"], None, o["ym4"])
    t.tfq_quantize_weight_per_channel(i["w"], "fp8", 448.0, 0, o["wq"], o["wqs"])
    t.tfq_quantize_rows_gather(x, f["route"], "fp8", 448.0, 0, o["qr"], o["sr"])
    t.tfq_grouped_scaled_mm_fp8(o["qr"], o["sr"], f["ex_q"], f["ex_s"], f["goff"], None,
                                "gelu_tanh", o["yr"])
    t.tfq_kv_cache_store(i["kv"], f["slot"], o["cache"], o["cache_s"])
    t.tfq_kv_cache_load(o["cache"], o["cache_s"], f["load"], torch.bfloat16, o["kv_out"])
    t.tfq_e4m3fn_encode_f32(i["f32"], o["enc"])


def test_every_entry_point_replays_in_a_graph():
    import int8_w8a8_quantized_amd as tfq

    tfq.tfq_set_autotune(0)
    say(f"graph of every entry point, M={M} K={K} N_up={NU} N_down={ND}")
    f = _fixed(tfq)
    i_static, o_static = _inputs(1), _alloc(tfq)
    _pass(tfq, f, i_static, o_static)          # first launches outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _pass(tfq, f, i_static, o_static)
    torch.cuda.synchronize()
    prev = None
    for r in range(3):
        say(f"graph replay {r}")
        fresh = _inputs(100 + r)
        ref = _alloc(tfq)
        _pass(tfq, f, fresh, ref)               # eager work between the replays
        torch.cuda.synchronize()
        for k, v in fresh.items():
            i_static[k].copy_(v)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(o_static[k].view(torch.uint8), ref[k].view(torch.uint8)), (r, k)
        # each replay computed from its own inputs
        if prev is not None:
            assert not torch.equal(o_static["y"], prev), r
        prev = o_static["y"].clone()
