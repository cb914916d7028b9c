"""Pins for the oracle's MoE routed W8A8 functions (CPU only).

TeleFuser "Quantization", "Other quantized data paths" (LingBot-Video MoE
FP8): expert weights per output channel, routed activations per row, one
scaled matmul per expert.  The pins check the row gather against plain
row quantisation of the same rows, and the grouped Linear against a
computation that shares nothing with the oracle's C code (torch's float8
decode, numpy binary64 sums, exact for these sizes), plus invariants: one
group is the plain Linear, permuting experts or adding empty ones changes
nothing, sampled rows equal the full result.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import synth

pytestmark = pytest.mark.filterwarnings("ignore")


def _x(rng, rows, cols):
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[rng.random((rows, cols)) < 0.02] *= 30
    return synth.to_bf16_bits(x)


def _decode(q):
    """E4M3FN codes -> float64 through torch's own float8 type."""
    t = torch.from_numpy(np.ascontiguousarray(q, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


@pytest.mark.parametrize("qtype,qmax,group", [("fp8", 448.0, 0), ("fp8", 14.0, 0),
                                              ("int8", 127.0, 0), ("fp8", 448.0, 128)])
def test_gather_quantize_equals_rowwise_quantize(qtype, qmax, group):
    rng = np.random.default_rng(1)
    x = _x(rng, 40, 256)
    q_all, s_all = orc.quantize_rows(x, qtype, qmax, group)
    # identity, reversal and a routed order with repeats (top-2 routing sends a
    # token to two experts)
    for idx in (np.arange(40), np.arange(39, -1, -1), rng.integers(0, 40, 70)):
        q, s = orc.quantize_rows_gather(x, idx, qtype, qmax, group)
        assert np.array_equal(q, q_all[idx]) and np.array_equal(s, s_all[idx])
    # each gathered row on its own, as a one-row matrix
    idx = rng.integers(0, 40, 6)
    q, s = orc.quantize_rows_gather(x, idx, qtype, qmax, group)
    for r, i in enumerate(idx):
        q1, s1 = orc.quantize_rows(x[i:i + 1], qtype, qmax, group)
        assert np.array_equal(q[r], q1[0]) and np.array_equal(s[r], s1[0])


def test_gather_out_of_range_rows_are_zero_rows():
    rng = np.random.default_rng(2)
    x = _x(rng, 8, 128)
    idx = np.array([3, -1, 8, 2**31 - 1, -2**31, 0])
    q, s = orc.quantize_rows_gather(x, idx, "fp8", 448.0)
    for r in (1, 2, 3, 4):
        assert s[r] == 0.0 and not q[r].any()
    q_ok, s_ok = orc.quantize_rows(x, "fp8", 448.0)
    assert np.array_equal(q[0], q_ok[3]) and np.array_equal(q[5], q_ok[0])


def _grouped_operands(seed, M, N, K, E):
    rng = np.random.default_rng(seed)
    qa, sa = orc.quantize_rows(_x(rng, M, K), "fp8", 448.0)
    w = (rng.standard_normal((E * N, K)) * 0.02).astype(np.float32)
    qb, sb = orc.quantize_rows(synth.to_bf16_bits(w), "fp8", 448.0)
    bias = synth.to_bf16_bits(rng.standard_normal((E, N)).astype(np.float32))
    return qa, sa, qb.reshape(E, N, K), sb.reshape(E, N), bias


def test_grouped_against_independent_binary64():
    """Ragged groups (one empty) against torch-decoded operands summed with
    numpy in binary64 (exact: every product is a multiple of 2^-18 below
    448^2, and K is small), scales applied in binary64, bias added."""
    M, N, K, E = 23, 16, 64, 4
    qa, sa, qb, sb, bias = _grouped_operands(3, M, N, K, E)
    off = np.array([0, 7, 7, 20, 23])
    y = orc.grouped_linear_ref(qa, sa, qb, sb, off, bias=bias)
    A = _decode(qa)
    bb = (bias.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for e in range(E):
        r = slice(off[e], off[e + 1])
        want = (A[r] @ _decode(qb[e]).T) * sa[r, None].astype(np.float64) \
            * sb[e][None, :].astype(np.float64) + bb[e][None, :]
        assert np.array_equal(y[r], want)


def test_single_group_is_the_plain_linear():
    M, N, K = 37, 24, 96
    qa, sa, qb, sb, bias = _grouped_operands(4, M, N, K, 1)
    y = orc.grouped_linear_ref(qa, sa, qb, sb, [0, M], bias=bias, gelu=True)
    assert np.array_equal(y, orc.linear_ref(qa, sa, qb[0], sb[0], "fp8", bias=bias[0], gelu=True))


def test_expert_permutation_and_empty_groups_change_nothing():
    M, N, K, E = 30, 8, 32, 3
    qa, sa, qb, sb, _ = _grouped_operands(5, M, N, K, E)
    off = np.array([0, 10, 18, 30])
    y = orc.grouped_linear_ref(qa, sa, qb, sb, off)
    # experts in the order 2, 0, 1 with their row blocks moved along
    perm = [2, 0, 1]
    rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in perm])
    sizes = [off[e + 1] - off[e] for e in perm]
    off_p = np.concatenate([[0], np.cumsum(sizes)])
    y_p = orc.grouped_linear_ref(qa[rows], sa[rows], qb[perm], sb[perm], off_p)
    assert np.array_equal(y_p, y[rows])
    # empty experts inserted at the front, middle and end
    qb_e = np.concatenate([qb[:1] * 0, qb[:1], qb[1:2] * 0, qb[1:], qb[:1] * 0])
    sb_e = np.concatenate([sb[:1], sb[:1], sb[:1], sb[1:], sb[:1]])
    off_e = np.array([0, 0, 10, 10, 18, 30, 30])
    assert np.array_equal(orc.grouped_linear_ref(qa, sa, qb_e, sb_e, off_e), y)


def test_rows_outside_every_group_and_sampled_rows():
    M, N, K, E = 40, 8, 64, 2
    qa, sa, qb, sb, _ = _grouped_operands(6, M, N, K, E)
    off = np.array([5, 20, 33])
    y = orc.grouped_linear_ref(qa, sa, qb, sb, off)
    assert np.isnan(y[:5]).all() and np.isnan(y[33:]).all() and not np.isnan(y[5:33]).any()
    rows = np.array([0, 5, 19, 20, 32, 33, 39])
    ys = orc.grouped_linear_ref(qa, sa, qb, sb, off, rows=rows)
    assert np.array_equal(ys, y[rows], equal_nan=True)
