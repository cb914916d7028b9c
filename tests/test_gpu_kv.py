"""GPU parity of the FP8 KV cache against the oracle.

TeleFuser "Quantization", "Other quantized data paths" (LiveAct FP8 KV
cache).  Store: cache codes and scales bit for bit, slots that are not named
(or out of range) untouched.  Load: BF16 / FP16 / FP32 outputs bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from gpu_util import dev_bf16, host_bits, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]

DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


@pytest.fixture(scope="module")
def tfq():
    import int8_w8a8_quantized_amd as m

    return m


def _kv(rng, T, W):
    x = rng.standard_normal((T, W)).astype(np.float32) * np.exp2(rng.integers(-10, 10, (T, 1)))
    x[rng.random(x.shape) < 0.02] *= 25
    return synth.to_bf16_bits(x.astype(np.float32))


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _bits(y):
    """Raw bits of a device tensor: uint16 for BF16 / FP16, uint32 for FP32."""
    y = y.detach().contiguous().cpu()
    if y.dtype == torch.float32:
        return y.numpy().view(np.uint32)
    return y.view(torch.int16).numpy().view(np.uint16)


def _same(got, want, what):
    """Bit equality; on failure name the first differing elements."""
    got = np.ascontiguousarray(got).reshape(-1)
    want = np.ascontiguousarray(want).reshape(-1)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {got.size} differ; first: " +
                           ", ".join(f"[{i}] got {int(got[i]):#x} want {int(want[i]):#x}"
                                     for i in bad[:6]))


@pytest.mark.parametrize("T,H,D,extra", [(37, 8, 128, 0), (100, 40, 128, 3 * 40 * 128),
                                         (5, 3, 64, 8), (9, 2, 96, 0), (11, 1, 512, 0),
                                         (64, 4, 8, 0), (20, 6, 256, 1536)])
def test_store_then_load_bit_exact(tfq, T, H, D, extra):
    """Tokens land in a permuted subset of slots (some tokens map outside the
    cache); the token stride may exceed heads * head_dim (K inside a fused
    QKV row)."""
    rng = np.random.default_rng(T * 7 + H + D)
    W = H * D + extra
    x = _kv(rng, T, W)
    x[0, :D] = 0                                   # an all-zero vector
    if H > 1:
        x[1 % T, D:2 * D] = 0x0001                 # every element the smallest BF16 subnormal
    S = T + 13
    slot = rng.permutation(S)[:T].astype(np.int64)
    slot[rng.random(T) < 0.1] = -1
    slot[-1] = S                                    # out of range
    kv = dev_bf16(x)[:, :H * D].view(T, H, D) if extra == 0 else \
        torch.as_strided(dev_bf16(x), (T, H, D), (W, D, 1))
    cache = torch.full((S, H, D), 0xAB, dtype=torch.uint8, device="cuda")
    scale = torch.full((S, H), -1.0, dtype=torch.float32, device="cuda")
    say(f"kv_cache_store T={T} H={H} D={D} ld={W}")
    tfq.tfq_kv_cache_store(kv, _i32(slot), cache, scale)
    torch.cuda.synchronize()
    cache_e = np.full((S, H, D), 0xAB, np.uint8)
    scale_e = np.full((S, H), -1.0, np.float32)
    orc.kv_store(x[:, :H * D].reshape(T, H, D), slot, cache_e, scale_e)
    assert np.array_equal(host_bits(cache), cache_e)
    assert np.array_equal(host_bits(scale).view(np.uint32), scale_e.view(np.uint32))
    idx = np.concatenate([rng.integers(0, S, 30), [-5, S, 2**31 - 1]])
    for out in ("bf16", "fp16", "fp32"):
        say(f"kv_cache_load {out} n={idx.size} H={H} D={D}")
        y = tfq.tfq_kv_cache_load(cache, scale, _i32(idx), DT[out])
        torch.cuda.synchronize()
        want = orc.kv_load(cache_e, scale_e, idx, out)
        if out == "fp32":
            want = want.view(np.uint32)
        _same(_bits(y), want, out)


def test_load_every_code_and_extreme_scales(tfq):
    """All finite codes times scales from binary32 subnormals to 1e30, in every
    output type (products that round to subnormals, to BF16/FP16 overflow
    and to zero included)."""
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    D = 256  # 254 finite codes, padded with zeros
    row = np.zeros(D, np.uint8)
    row[:codes.size] = codes
    scales = np.array([1.0, 1 / 448, 3.0517578e-05, 2.0 ** -126, 2.0 ** -140, 1e-20, 7.1e-3,
                       1e30, 65504 / 448, 0.333333343], np.float32)
    S = scales.size
    cache_e = np.broadcast_to(row, (S, 1, D)).copy()
    scale_e = scales[:, None].copy()
    cache = torch.from_numpy(cache_e).cuda()
    scale = torch.from_numpy(scale_e).cuda()
    for out in ("bf16", "fp16", "fp32"):
        say(f"kv_cache_load all codes {out}")
        y = tfq.tfq_kv_cache_load(cache, scale, _i32(np.arange(S)), DT[out])
        torch.cuda.synchronize()
        want = orc.kv_load(cache_e, scale_e, np.arange(S), out)
        if out == "fp32":
            want = want.view(np.uint32)
        _same(_bits(y), want, out)


def test_video_dit_attention_cache_sampled(tfq):
    """A video-DiT-sized K cache: 75600 tokens x 40 heads x 128, stored in
    reverse slot order, then loaded in a random order; sampled tokens checked."""
    T, H, D = 75600, 40, 128
    g = torch.Generator(device="cuda").manual_seed(5)
    kv = torch.randn((T, H, D), generator=g, device="cuda").to(torch.bfloat16)
    slot = torch.arange(T - 1, -1, -1, dtype=torch.int32, device="cuda")
    cache = torch.empty((T, H, D), dtype=torch.uint8, device="cuda")
    scale = torch.empty((T, H), dtype=torch.float32, device="cuda")
    say("kv_cache_store 75600x40x128")
    tfq.tfq_kv_cache_store(kv, slot, cache, scale)
    perm = torch.randperm(T, generator=g, device="cuda").to(torch.int32)
    y = tfq.tfq_kv_cache_load(cache, scale, perm)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    pick = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, 40)]))
    x_s = host_bits(kv[pick])
    cache_e = np.zeros((T, H, D), np.uint8)
    scale_e = np.zeros((T, H), np.float32)
    orc.kv_store(x_s, (T - 1) - pick, cache_e, scale_e)
    rows = (T - 1) - pick
    assert np.array_equal(host_bits(cache)[rows], cache_e[rows])
    assert np.array_equal(host_bits(scale)[rows], scale_e[rows])
    perm_h = perm.cpu().numpy()
    at = np.nonzero(np.isin(perm_h, rows))[0][:40]
    want = orc.kv_load(cache_e, scale_e, perm_h[at], "bf16")
    assert np.array_equal(host_bits(y)[at], want)
