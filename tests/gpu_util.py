"""Helpers for the GPU parity tests: host <-> device transfers and the FP8
output tolerance stated for the scaled GEMM."""
import sys

import numpy as np
import pytest
import torch

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")


def say(msg: str) -> None:
    """Name the case (shape, seed, entry point) before a GPU step, flushed."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """BF16 bit array (uint16) -> device bfloat16 tensor."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_u8(a: np.ndarray, dtype=torch.uint8) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.uint8)).cuda()
    return t if dtype == torch.uint8 else t.view(dtype)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy raw bits (uint8 for codes, uint16 for bf16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.uint8, torch.int8):
        return t.view(torch.uint8).numpy()
    return t.numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(
        np.float32).astype(np.float64)


def assert_fp8_tolerance(y_bits: np.ndarray, y_ref: np.ndarray, what: str = "") -> float:
    """max|y - y_ref| <= 2^-7 |y_ref| + 1e-3 max_row|y_ref|, element by
    element; returns the largest ratio of error to allowance."""
    y = bf16_to_f64(y_bits)
    assert y.shape == y_ref.shape
    rowmax = np.abs(y_ref).max(axis=1, keepdims=True)
    allow = 2.0 ** -7 * np.abs(y_ref) + 1e-3 * rowmax
    err = np.abs(y - y_ref)
    assert np.all(np.isfinite(y)), what
    bad = err > allow
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} outputs out of tolerance, first at {tuple(i)}: "
                             f"y={y[tuple(i)]!r} ref={y_ref[tuple(i)]!r} allow={allow[tuple(i)]!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(allow > 0, err / allow, 0.0)
    return float(ratio.max())


# MX scale layout of the library: [cols/128, rows, 4], the four block scales
# of a 128-element K group together in the byte order 0, 2, 1, 3
MX_ORDER = [0, 2, 1, 3]


def mx_grouped(s):
    """Oracle scales [rows, cols/32] -> library layout [cols/128, rows, 4]."""
    r, nb = s.shape
    return np.ascontiguousarray(s.reshape(r, nb // 4, 4)[:, :, MX_ORDER].transpose(1, 0, 2))


def mx6_grouped(q):
    """MXFP6 codes [rows, 3 cols / 4] (a 6-bit stream per row, as the oracle
    writes them) -> library layout [cols/128, rows, 96] (96 bytes per
    128-element group, group-major)."""
    r, nb = q.shape
    return np.ascontiguousarray(q.reshape(r, nb // 96, 96).transpose(1, 0, 2))


def mx6_ungrouped(q):
    """Library layout [cols/128, rows, 96] -> MXFP6 codes [rows, 3 cols / 4]."""
    g, r, _ = q.shape
    return np.ascontiguousarray(q.transpose(1, 0, 2).reshape(r, 96 * g))


def mx_ungrouped(s):
    """Library layout [cols/128, rows, 4] -> oracle scales [rows, cols/32]."""
    g, r, _ = s.shape
    return np.ascontiguousarray(s[:, :, MX_ORDER].transpose(1, 0, 2).reshape(r, 4 * g))


def every_bf16_blocks(kemax: int, shared_list, cols: int = 4096) -> np.ndarray:
    """BF16 rows that put every finite BF16 value through an MX quantiser
    under each shared exponent in shared_list.  For shared exponent S the
    block amax is the largest BF16 value of exponent field S + 127 + kemax
    (kemax: exponent of the element type's largest normal), so the block's
    E8M0 byte is S + 127; each 32-element block is that amax (alternating
    sign) followed by 31 values of magnitude at most it, every such BF16
    value of both signs once.  For S = -127 the amax is the largest value
    with exponent field kemax (every smaller amax also gives the byte 0).
    Rows of `cols` elements; the tail is padded with zeros."""
    blocks = []
    mag = np.arange(0x7F80, dtype=np.uint32)  # finite magnitudes (bits)
    for S in shared_list:
        e = S + 127 + kemax if S > -127 else kemax
        assert 1 <= e <= 254, S
        amax = np.uint32((e << 7) | 0x7F)
        vals = mag[mag <= amax]
        vals = np.concatenate([vals, vals | 0x8000]).astype(np.uint16)
        nb = (vals.size + 30) // 31
        body = np.zeros(nb * 31, dtype=np.uint16)
        body[:vals.size] = vals
        head = np.where(np.arange(nb) % 2 == 0, amax, amax | 0x8000).astype(np.uint16)
        blocks.append(np.concatenate([head[:, None], body.reshape(nb, 31)], axis=1))
    b = np.concatenate(blocks, axis=0).reshape(-1)
    rows = (b.size + cols - 1) // cols
    out = np.zeros(rows * cols, dtype=np.uint16)
    out[:b.size] = b
    return out.reshape(rows, cols)
