"""Seeded synthetic inputs for the W8A8 Linear workloads.

This module only draws random numbers and rounds them to BF16; it holds none
of the quantisation or GEMM arithmetic, so the oracle, the tests and the
benchmark can all use it without sharing method code.

Recipe (one ``numpy.random.default_rng(seed)`` per workload, seed 0 unless
stated; draws happen in the order listed; float32 draws are rounded to BF16
with round-to-nearest-even by torch's CPU cast):

  * ``normal(std)``            -- ``standard_normal`` (float32) times std;
  * ``student_t4(scale)``      -- Student-t with 4 degrees of freedom built
    from its definition: Z / sqrt(V / 4) with Z ~ N(0, 1) and
    V ~ chi-square(4) = 2 (E1 + E2), E1, E2 ~ Exp(1); drawn as the arrays Z,
    E1, E2 in that order, then multiplied by ``scale``;
  * outliers ``(p, c)``        -- after X: a ``random`` float32 array of
    X's shape; entries whose draw is < p are multiplied by c.

Workloads (the activation X, then the outlier mask, then W, then W_down):

  c1_tiny_fp8     X [128, 256] N(0,1), 1% x20;    W [512, 256] N(0, 0.02)
  c2_int8         X [4096, 3072] N(0,1), 0.5% x30; W [3072, 3072] N(0, 0.02)
  c3_image_dit    X [7145, 3072] 0.5 * t4;         W [12288, 3072] N(0, 0.02)
  c4_video_dit    X [75600, 5120] t4;  W_up [13824, 5120] N(0, 0.015),
                  W_down [5120, 13824] N(0, 0.015)
  c5_block_fp8    X [8192, 5120] N(0,1), 1% x20;   W [5120, 5120] N(0, 0.02)

The C3 token count is 83 x 83 image tokens of a 1328 x 1328 image with a
16-pixel latent patch plus 256 text tokens; C4's is a 21 x 45 x 80 video
latent.  ``make(name, M=..., ...)`` overrides shapes for small parity cases
with the same distributions.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    qtype: str                      # "fp8" | "int8"
    x_dist: tuple                   # ("normal", std) | ("t4", scale)
    outliers: tuple | None          # (p, multiplier) or None
    w_std: float
    n_down: int = 0                 # > 0: FFN pair, W_down [n_down, N]
    w_down_std: float = 0.0
    act_qmax: tuple = (448.0,)      # activation qmax values
    w_qmax: float = 448.0
    scale_block: int = 0            # 0 = per-token / per-channel, 128 = block
    gelu: bool = False              # GELU-tanh on the (up) projection
    seed: int = 0
    note: str = ""


WORKLOADS = {
    "c1_tiny_fp8": Workload("c1_tiny_fp8", 128, 256, 512, "fp8", ("normal", 1.0), (0.01, 20.0),
                            0.02, note="tiny FP8 W8A8 Linear"),
    "c2_int8": Workload("c2_int8", 4096, 3072, 3072, "int8", ("normal", 1.0), (0.005, 30.0), 0.02,
                        act_qmax=(127.0,), w_qmax=127.0, note="INT8 W8A8 Linear"),
    "c3_image_dit": Workload("c3_image_dit", 7145, 3072, 12288, "fp8", ("t4", 0.5), None, 0.02,
                             note="image-DiT FFN-up, 1328x1328 (6889 image + 256 text tokens)"),
    "c4_video_dit": Workload("c4_video_dit", 75600, 5120, 13824, "fp8", ("t4", 1.0), None, 0.015,
                             n_down=5120, w_down_std=0.015, act_qmax=(448.0, 14.0, 7.0),
                             gelu=True, note="video-DiT FFN pair, 21x45x80 latent tokens"),
    "c5_block_fp8": Workload("c5_block_fp8", 8192, 5120, 5120, "fp8", ("normal", 1.0),
                             (0.01, 20.0), 0.02, scale_block=128,
                             note="block-scaled FP8 (128x128 W blocks, 1x128 X groups)"),
}


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> BF16 bit pattern (uint16), round-to-nearest-even."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _draw_x(rng: np.random.Generator, shape, dist) -> np.ndarray:
    kind, p = dist
    if kind == "normal":
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if p != 1.0:
            x *= np.float32(p)
        return x
    if kind == "t4":
        z = rng.standard_normal(size=shape, dtype=np.float32)
        e1 = rng.standard_exponential(size=shape, dtype=np.float32)
        e2 = rng.standard_exponential(size=shape, dtype=np.float32)
        e1 += e2
        del e2
        e1 *= np.float32(0.5)
        np.sqrt(e1, out=e1)
        z /= e1
        del e1
        if p != 1.0:
            z *= np.float32(p)
        return z
    raise ValueError(kind)


def make(name: str, *, M: int | None = None, K: int | None = None, N: int | None = None,
         n_down: int | None = None, seed: int | None = None, with_weights: bool = True) -> dict:
    """Draw one workload's inputs.  Returns a dict with the Workload under
    "spec" and BF16 bit arrays (uint16) "x" [M,K], "w" [N,K] and, for the
    FFN pair, "w_down" [n_down, N]."""
    wl = WORKLOADS[name]
    over = {}
    if M is not None:
        over["M"] = M
    if K is not None:
        over["K"] = K
    if N is not None:
        over["N"] = N
    if n_down is not None:
        over["n_down"] = n_down
    if seed is not None:
        over["seed"] = seed
    wl = replace(wl, **over)
    rng = np.random.default_rng(wl.seed)
    x = _draw_x(rng, (wl.M, wl.K), wl.x_dist)
    if wl.outliers is not None:
        p, c = wl.outliers
        mask = rng.random(size=(wl.M, wl.K), dtype=np.float32) < np.float32(p)
        x[mask] *= np.float32(c)
        del mask
    out = {"spec": wl, "x": to_bf16_bits(x)}
    del x
    if with_weights:
        w = rng.standard_normal(size=(wl.N, wl.K), dtype=np.float32)
        w *= np.float32(wl.w_std)
        out["w"] = to_bf16_bits(w)
        del w
        if wl.n_down > 0:
            wd = rng.standard_normal(size=(wl.n_down, wl.N), dtype=np.float32)
            wd *= np.float32(wl.w_down_std)
            out["w_down"] = to_bf16_bits(wd)
    return out


def bf16_rows(rng_seed: int, rows: int, cols: int, std: float = 1.0) -> np.ndarray:
    """Plain N(0, std) BF16 bits, for small property tests."""
    rng = np.random.default_rng(rng_seed)
    return to_bf16_bits(rng.standard_normal(size=(rows, cols), dtype=np.float32) * np.float32(std))
