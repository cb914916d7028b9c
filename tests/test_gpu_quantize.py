"""GPU parity of the quantisers against the oracle: codes and FP32 scales must
match bit for bit (TeleFuser "Quantization", "Scaled FP8 checkpoints: W8A8"
and "Core ideas"; LightX2V "模型量化技术", "MiniMax-H3 FP8 FP16 累加" and
table "量化模式")."""
import numpy as np
import pytest
import torch

import oracle as orc
import synth
from gpu_util import dev_bf16, dev_f32, host_bits, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module")
def tfq():
    import int8_w8a8_quantized_amd as m

    return m


def _rows(seed, rows, cols, spread=20):
    """BF16 rows with per-row magnitudes spread over 2^-spread .. 2^spread,
    1% outliers x30, plus special rows when there is room."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-spread, spread, (rows, 1))).astype(np.float32)
    x[rng.random((rows, cols)) < 0.01] *= 30
    b = synth.to_bf16_bits(x)
    if rows >= 6:
        b[0] = 0                                   # all-zero row: s = 0
        b[1] = 0x8000                              # all -0
        b[2] = (np.arange(cols) % 7).astype(np.uint16)           # subnormal amax
        b[2, ::3] |= 0x8000
        b[3, :] = 0x7F7F                           # max finite BF16 everywhere
        b[3, 1::2] = 0xFF7F
        b[4, 5 % cols] = 0x0001                    # tiny elements in a normal row
        b[4, 7 % cols] = 0x8001
    return b


def _check(tfq, xbits, qtype, qmax, group=0, ld=None):
    rows, cols = xbits.shape
    say(f"quantize_rows qtype={qtype} qmax={qmax} rows={rows} cols={cols} group={group} ld={ld}")
    if ld is None:
        xd = dev_bf16(xbits)
    else:
        pad = np.zeros((rows, ld), dtype=np.uint16)
        pad[:, :cols] = xbits
        pad[:, cols:] = 0x7F7F  # must be ignored
        xd = dev_bf16(pad)[:, :cols]
    q, s = tfq.tfq_quantize_rows(xd, qtype, qmax, group)
    torch.cuda.synchronize()
    qe, se = orc.quantize_rows(xbits, qtype, qmax, group)
    qg, sg = host_bits(q), host_bits(s)
    assert np.array_equal(sg.view(np.uint32), se.view(np.uint32)), "scales differ"
    if not np.array_equal(qg, qe):
        r, c = np.argwhere(qg != qe)[0]
        raise AssertionError(f"codes differ at ({r},{c}): gpu {qg[r, c]:#x} oracle {qe[r, c]:#x} "
                             f"x={xbits[r, c]:#06x} s={se.ravel()[r] if group == 0 else se[r]}")


SHAPES = [(7, 16), (33, 256), (65, 528), (17, 3072), (9, 5120), (5, 13824), (3, 16400),
          (4, 32768)]


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_fp8_rows(tfq, rows, cols):
    _check(tfq, _rows(rows * 1000 + cols, max(rows, 6), cols), "fp8", 448.0)


@pytest.mark.parametrize("qmax", [14.0, 12.0, 7.0, 0.5, 240.0])
def test_fp8_reduced_qmax(tfq, qmax):
    _check(tfq, _rows(int(qmax * 10), 33, 5120), "fp8", qmax)


@pytest.mark.parametrize("rows,cols", SHAPES[:6])
def test_int8_rows(tfq, rows, cols):
    _check(tfq, _rows(rows * 7 + cols, max(rows, 6), cols), "int8", 127.0)
    _check(tfq, _rows(rows * 7 + cols + 1, max(rows, 6), cols), "int8", 100.0)


def test_leading_dimension(tfq):
    _check(tfq, _rows(5, 10, 512), "fp8", 448.0, ld=520)
    _check(tfq, _rows(6, 10, 512), "int8", 127.0, ld=1024)


def test_division_sensitive_rows(tfq):
    """Rows in which multiplying by RN(1/s) would change codes: the kernel must
    produce the correctly rounded quotient's codes."""
    from test_oracle_quantize import _rows_where_reciprocal_differs

    for qtype, qmax in [("fp8", 448.0), ("fp8", 7.0), ("int8", 127.0)]:
        x = _rows_where_reciprocal_differs(qmax, qtype, nrows=64, cols=256, seed=21)
        _check(tfq, x, qtype, qmax)


@pytest.mark.parametrize("rows,cols", [(9, 128), (33, 640), (17, 5120), (5, 16512)])
def test_groups_128(tfq, rows, cols):
    _check(tfq, _rows(rows + cols, max(rows, 6), cols), "fp8", 448.0, group=128)
    _check(tfq, _rows(rows + cols + 3, max(rows, 6), cols), "int8", 127.0, group=128)


def test_groups_of_every_kind_in_one_wave(tfq):
    """The 1x128-group kernel quantises 4 groups of a row per 64-lane chunk,
    each with its own scale: all-zero groups (s = 0, with -0 elements),
    subnormal absmax (s below the division shortcut's window), BF16-max
    groups (s overflows to inf at qmax 0.5) and normal groups side by side."""
    rng = np.random.default_rng(77)
    rows, cols = 8, 1024
    x = synth.to_bf16_bits(rng.standard_normal((rows, cols)).astype(np.float32))
    for r in range(rows):
        g = np.roll(np.arange(8), r) * 128
        x[r, g[0]:g[0] + 128] = 0
        x[r, g[0]:g[0] + 128:3] = 0x8000
        x[r, g[1]:g[1] + 128] = (np.arange(128) % 5).astype(np.uint16)
        x[r, g[1]:g[1] + 128:2] |= 0x8000
        x[r, g[2]:g[2] + 128] = 0x7F7F
        x[r, g[2] + 1:g[2] + 128:2] = 0xFF7F
    for qtype, qmax in [("fp8", 448.0), ("fp8", 0.5), ("fp8", 14.0), ("int8", 127.0)]:
        _check(tfq, x, qtype, qmax, group=128)


def test_weight_per_channel_and_blocks(tfq):
    d = synth.make("c5_block_fp8", M=8, K=640, N=384)
    w = d["w"]
    say("quantize_weight_per_channel fp8 384x640 block 0/128")
    wd = dev_bf16(w)
    q, s = tfq.tfq_quantize_weight_per_channel(wd, "fp8", 448.0, 0)
    qe, se = orc.quantize_rows(w, "fp8", 448.0)
    assert np.array_equal(host_bits(q), qe) and np.array_equal(host_bits(s), se)
    q, s = tfq.tfq_quantize_weight_per_channel(wd, "fp8", 448.0, 128)
    qe, se = orc.quantize_blocks(w, "fp8", 448.0, 128)
    assert np.array_equal(host_bits(q), qe) and np.array_equal(host_bits(s), se)
    q, s = tfq.tfq_quantize_weight_per_channel(wd, "int8", 127.0, 128)
    qe, se = orc.quantize_blocks(w, "int8", 127.0, 128)
    assert np.array_equal(host_bits(q), qe) and np.array_equal(host_bits(s), se)


def test_device_e4m3fn_encoder_every_binary32(tfq):
    """The conversion the FP8 quantiser uses, over every finite binary32 value
    of both signs, against the oracle's encoder."""
    chunk = 1 << 27
    top = 0x7F800000  # exclusive: all finite positive patterns
    lib = orc.lib()
    for start in range(0, top, chunk):
        n = min(chunk, top - start)
        say(f"e4m3fn_encode patterns [{start:#x}, {start + n:#x})")
        pos = torch.arange(start, start + n, dtype=torch.int32, device="cuda")
        for sign in (0, 1):
            bits = pos if sign == 0 else (pos | torch.tensor(-2 ** 31, dtype=torch.int32,
                                                               device="cuda"))
            q = tfq.tfq_e4m3fn_encode_f32(bits.view(torch.float32))
            hb = np.arange(start, start + n, dtype=np.uint32)
            if sign:
                hb |= np.uint32(0x80000000)
            ref = orc.e4m3fn_encode_array(hb.view(np.float32))
            got = host_bits(q)
            if not np.array_equal(got, ref):
                i = np.flatnonzero(got != ref)[0]
                raise AssertionError(f"pattern {hb[i]:#010x}: gpu {got[i]:#x} oracle {ref[i]:#x}")
        del pos
    _ = lib


@pytest.mark.parametrize("qtype,qmax", [("fp8", 448.0), ("int8", 127.0)])
def test_every_bf16_pair_division(tfq, qtype, qmax):
    """Every positive finite BF16 amax with every BF16 x, |x| <= amax: row j
    holds amax_j and all BF16 magnitudes up to it (signs alternating), so the
    kernel's division x / s runs on every (amax, x) pair; codes and scales
    must equal the oracle's (true binary32 division) bit for bit."""
    top = 0x7F7F  # largest finite BF16 magnitude
    per = 1024
    for lo in range(1, top + 1, per):
        ab = np.arange(lo, min(lo + per, top + 1), dtype=np.int64)
        width = int(-(-(int(ab[-1]) + 1) // 16) * 16)
        col = np.arange(width, dtype=np.int64)
        inside = col[None, :] <= ab[:, None]
        sign = ((col[None, :] + ab[:, None]) & 1) << 15
        x = np.where(inside, col[None, :] | sign, 0).astype(np.uint16)
        say(f"every-pair division {qtype} qmax={qmax} amax bits [{lo:#06x}, {int(ab[-1]):#06x}] "
            f"cols={width}")
        xd = dev_bf16(x)
        q, s = tfq.tfq_quantize_rows(xd, qtype, qmax)
        torch.cuda.synchronize()
        qe, se = orc.quantize_rows(x, qtype, qmax)
        qg, sg = host_bits(q), host_bits(s)
        assert np.array_equal(sg.view(np.uint32), se.view(np.uint32)), f"scales differ from {lo:#x}"
        if not np.array_equal(qg, qe):
            r, c = np.argwhere(qg != qe)[0]
            raise AssertionError(f"codes differ: amax {int(ab[r]):#06x} x {x[r, c]:#06x}: "
                                 f"gpu {qg[r, c]:#x} oracle {qe[r, c]:#x}")
        del xd, q, s
