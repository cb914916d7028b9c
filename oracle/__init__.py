"""CPU oracle for the W8A8 scaled-quantized Linear -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library
(``int8_w8a8_quantized_amd``) never imports it, and it imports nothing from
the product: the two share no code.

The arithmetic lives in ``tfq_oracle.c`` (plain C, binary32 quantisation with
strict IEEE semantics, exact binary64 GEMM sums); this module only compiles it
with gcc and marshals numpy arrays through ctypes.  Every function cites the
page passage it follows in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tfq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libtfq_oracle.so")

QTYPE_E4M3FN = 0
QTYPE_INT8 = 1

_CFLAGS = [
    "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
    "-fexcess-precision=standard", "-fopenmp", "-shared", "-fPIC",
]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libtfq_oracle.so``."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.tfq_oracle_bf16_to_f32.restype = ctypes.c_float
        L.tfq_oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.tfq_oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.tfq_oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.tfq_oracle_e4m3fn_value.restype = ctypes.c_double
        L.tfq_oracle_e4m3fn_value.argtypes = [ctypes.c_uint8]
        L.tfq_oracle_e4m3fn_encode.restype = ctypes.c_uint8
        L.tfq_oracle_e4m3fn_encode.argtypes = [ctypes.c_float]
        L.tfq_oracle_e4m3fn_encode_search.restype = ctypes.c_uint8
        L.tfq_oracle_e4m3fn_encode_search.argtypes = [ctypes.c_float]
        L.tfq_oracle_e4m3fn_encode_array.restype = None
        L.tfq_oracle_e4m3fn_encode_array.argtypes = [P, P, i64]
        L.tfq_oracle_encoder_mismatches.restype = i64
        L.tfq_oracle_encoder_mismatches.argtypes = [ctypes.c_uint32, ctypes.c_uint32, P]
        L.tfq_oracle_quantize_rows.restype = None
        L.tfq_oracle_quantize_rows.argtypes = [P, i64, i64, i64, ctypes.c_int, ctypes.c_float, i64, P, P]
        L.tfq_oracle_quantize_blocks.restype = None
        L.tfq_oracle_quantize_blocks.argtypes = [P, i64, i64, ctypes.c_int, ctypes.c_float, i64, P, P]
        L.tfq_oracle_gelu_tanh.restype = ctypes.c_double
        L.tfq_oracle_gelu_tanh.argtypes = [ctypes.c_double]
        L.tfq_oracle_dot.restype = None
        L.tfq_oracle_dot.argtypes = [P, P, ctypes.c_int, i64, i64, i64, P, i64, P]
        L.tfq_oracle_linear_ref.restype = None
        L.tfq_oracle_linear_ref.argtypes = [P, P, P, P, ctypes.c_int, i64, i64, i64, i64, P,
                                            ctypes.c_int, P, i64, P]
        L.tfq_oracle_mx_scale_code.restype = ctypes.c_uint8
        L.tfq_oracle_mx_scale_code.argtypes = [ctypes.c_float]
        L.tfq_oracle_quantize_mx.restype = None
        L.tfq_oracle_quantize_mx.argtypes = [P, i64, i64, i64, P, P]
        L.tfq_oracle_linear_mx_ref.restype = None
        L.tfq_oracle_linear_mx_ref.argtypes = [P, P, P, P, i64, i64, i64, P, ctypes.c_int, P, i64, P]
        L.tfq_oracle_fp6_value.restype = ctypes.c_double
        L.tfq_oracle_fp6_value.argtypes = [ctypes.c_int, ctypes.c_uint8]
        L.tfq_oracle_fp6_encode.restype = ctypes.c_uint8
        L.tfq_oracle_fp6_encode.argtypes = [ctypes.c_int, ctypes.c_float]
        L.tfq_oracle_mx6_scale_code.restype = ctypes.c_uint8
        L.tfq_oracle_mx6_scale_code.argtypes = [ctypes.c_int, ctypes.c_float]
        L.tfq_oracle_quantize_mx6.restype = None
        L.tfq_oracle_quantize_mx6.argtypes = [ctypes.c_int, P, i64, i64, i64, P, P]
        L.tfq_oracle_linear_mx6_ref.restype = None
        L.tfq_oracle_linear_mx6_ref.argtypes = [ctypes.c_int, P, P, P, P, i64, i64, i64, P,
                                                ctypes.c_int, P, i64, P]
        L.tfq_oracle_e2m1_value.restype = ctypes.c_double
        L.tfq_oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        L.tfq_oracle_e2m1_encode.restype = ctypes.c_uint8
        L.tfq_oracle_e2m1_encode.argtypes = [ctypes.c_float]
        L.tfq_oracle_mx4_scale_code.restype = ctypes.c_uint8
        L.tfq_oracle_mx4_scale_code.argtypes = [ctypes.c_float]
        L.tfq_oracle_quantize_mx4.restype = None
        L.tfq_oracle_quantize_mx4.argtypes = [P, i64, i64, i64, P, P]
        L.tfq_oracle_linear_mx4_ref.restype = None
        L.tfq_oracle_linear_mx4_ref.argtypes = [P, P, P, P, i64, i64, i64, P, ctypes.c_int, P, i64, P]
        L.tfq_oracle_gelu_tanh_array.restype = None
        L.tfq_oracle_gelu_tanh_array.argtypes = [P, i64]
        L.tfq_oracle_int8_epilogue.restype = None
        L.tfq_oracle_int8_epilogue.argtypes = [P, P, P, i64, i64, P, P, P]
        L.tfq_oracle_int8_linear.restype = None
        L.tfq_oracle_int8_linear.argtypes = [P, P, P, P, i64, i64, i64, P, P, i64, P, P]
        L.tfq_oracle_error_measures.restype = None
        L.tfq_oracle_error_measures.argtypes = [P, P, i64, P, P]
        L.tfq_oracle_num_threads.restype = ctypes.c_int
        L.tfq_oracle_num_threads.argtypes = []
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _qtype(q) -> int:
    if q in ("fp8", "e4m3fn", QTYPE_E4M3FN):
        return QTYPE_E4M3FN
    if q in ("int8", QTYPE_INT8):
        return QTYPE_INT8
    raise ValueError(f"unknown qtype {q!r}")


def num_threads() -> int:
    return lib().tfq_oracle_num_threads()


# --------------------------------------------------------------------------
# scalar helpers
# --------------------------------------------------------------------------
def bf16_to_f32(h: int) -> float:
    return lib().tfq_oracle_bf16_to_f32(h)


def f32_to_bf16(v: float) -> int:
    return lib().tfq_oracle_f32_to_bf16(v)


def e4m3fn_value(code: int) -> float:
    """Closed-form E4M3FN decode of one code (OCP OFP8)."""
    return lib().tfq_oracle_e4m3fn_value(code)


def e4m3fn_encode(v: float) -> int:
    """E4M3FN encoder 1 (field arithmetic, RNE, saturating)."""
    return lib().tfq_oracle_e4m3fn_encode(v)


def e4m3fn_encode_search(v: float) -> int:
    """E4M3FN encoder 2 (nearest-value search, ties to even code)."""
    return lib().tfq_oracle_e4m3fn_encode_search(v)


def e4m3fn_encode_array(v: np.ndarray) -> np.ndarray:
    """Encoder 1 applied elementwise to a float32 array."""
    a = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint8)
    lib().tfq_oracle_e4m3fn_encode_array(_ptr(a), _ptr(out), a.size)
    return out


def encoder_mismatches(first_bits: int, last_bits: int) -> tuple[int, int]:
    """Count binary32 patterns in [first, last] (both signs) where the two
    encoders disagree; returns (count, first bad pattern or 0xFFFFFFFF)."""
    fb = ctypes.c_uint32(0)
    n = lib().tfq_oracle_encoder_mismatches(first_bits, last_bits, ctypes.byref(fb))
    return int(n), int(fb.value)


def gelu_tanh(h: float) -> float:
    return lib().tfq_oracle_gelu_tanh(h)


def e4m3fn_table() -> np.ndarray:
    """Values of all 256 codes (NaN for 0x7F and 0xFF)."""
    return np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


# --------------------------------------------------------------------------
# array functions
# --------------------------------------------------------------------------
def quantize_rows(x_bf16: np.ndarray, qtype, qmax: float, group: int = 0):
    """Per-row (group=0) or per-1xgroup dynamic absmax quantisation.

    x_bf16: uint16 [rows, cols] (BF16 bits). Returns (codes uint8 [rows, cols],
    scales float32 [rows] or [rows, ceil(cols/group)])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    ng = 1 if group <= 0 else (cols + group - 1) // group
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty((rows, ng), dtype=np.float32)
    lib().tfq_oracle_quantize_rows(_ptr(x), rows, cols, cols, _qtype(qtype), float(qmax),
                                   int(group), _ptr(q), _ptr(s))
    return q, (s[:, 0].copy() if group <= 0 else s)


def quantize_blocks(w_bf16: np.ndarray, qtype, qmax: float, block: int = 128):
    """One scale per block x block tile of W [n, k]."""
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    n, k = w.shape
    nb, kb = (n + block - 1) // block, (k + block - 1) // block
    q = np.empty((n, k), dtype=np.uint8)
    s = np.empty((nb, kb), dtype=np.float32)
    lib().tfq_oracle_quantize_blocks(_ptr(w), n, k, _qtype(qtype), float(qmax), int(block),
                                     _ptr(q), _ptr(s))
    return q, s


def _rows_arg(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, int(r.shape[0])


def dot(a_q: np.ndarray, b_q: np.ndarray, qtype, rows=None) -> np.ndarray:
    """Exact sum_k a[m,k] b[n,k] of decoded codes, binary64, for selected rows."""
    a = np.ascontiguousarray(a_q).view(np.uint8)
    b = np.ascontiguousarray(b_q).view(np.uint8)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape[1] == K
    r, nr = _rows_arg(rows)
    R = M if r is None else nr
    out = np.empty((R, N), dtype=np.float64)
    lib().tfq_oracle_dot(_ptr(a), _ptr(b), _qtype(qtype), M, N, K, _ptr(r), nr, _ptr(out))
    return out


def linear_ref(a_q, a_scale, b_q, b_scale, qtype, scale_block: int = 0, bias=None,
               gelu: bool = False, rows=None) -> np.ndarray:
    """Scaled Linear reference y [R, N] in binary64 (see tfq_oracle_linear_ref)."""
    a = np.ascontiguousarray(a_q).view(np.uint8)
    b = np.ascontiguousarray(b_q).view(np.uint8)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape[1] == K
    sa = np.ascontiguousarray(a_scale, dtype=np.float32)
    sb = np.ascontiguousarray(b_scale, dtype=np.float32)
    bi = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16)
    r, nr = _rows_arg(rows)
    R = M if r is None else nr
    out = np.empty((R, N), dtype=np.float64)
    lib().tfq_oracle_linear_ref(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _qtype(qtype), M, N, K,
                                int(scale_block), _ptr(bi), 1 if gelu else 0, _ptr(r), nr,
                                _ptr(out))
    return out


def _code_values64(codes: np.ndarray, qtype) -> np.ndarray:
    """Exact binary64 values of FP8 (E4M3FN) or INT8 codes."""
    c = np.ascontiguousarray(codes).view(np.uint8)
    if _qtype(qtype) == QTYPE_E4M3FN:
        return e4m3fn_table()[c]
    return c.view(np.int8).astype(np.float64)


def linear_ref_fast(a_q, a_scale, b_q, b_scale, qtype, scale_block: int = 0, bias=None,
                    gelu: bool = False, rows=None) -> np.ndarray:
    """linear_ref with the dots formed by numpy's binary64 matmul (BLAS).

    The exact-dot property makes this the same reference, bit for bit: every
    E4M3FN or INT8 code value is an integer multiple of 2^-9 of magnitude at
    most 448, so each product is a multiple of 2^-18 below 2^17.7 and any
    partial sum of K <= 2^17 of them is exactly representable in binary64 --
    in whatever order or blocking the library sums.  The scaling then follows
    tfq_oracle_linear_ref's binary64 steps in its order: (dot * s_row) * s_col,
    or sum over K blocks of (s_row[m,kb] * s_col[n/blk,kb]) * dot_kb in block
    order; + bias; GELU-tanh by the C function.  Pinned bit-equal to
    linear_ref in tests/test_oracle_gemm.py."""
    a = np.ascontiguousarray(a_q).view(np.uint8)
    M, K = a.shape
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    ar = _code_values64(a if r is None else a[r], qtype)
    b64 = _code_values64(b_q, qtype)
    N = b64.shape[0]
    assert b64.shape[1] == K and K <= (1 << 17)
    sa = np.ascontiguousarray(a_scale, dtype=np.float32).astype(np.float64)
    sb = np.ascontiguousarray(b_scale, dtype=np.float32).astype(np.float64)
    if scale_block <= 0:
        s_row = sa if r is None else sa[r]
        y = ((ar @ b64.T) * s_row[:, None]) * sb[None, :]
    else:
        blk = int(scale_block)
        nkb = (K + blk - 1) // blk
        sa2 = sa.reshape(M, nkb)
        sb2 = sb.reshape(-1, nkb)
        s_rows = sa2 if r is None else sa2[r]
        y = np.zeros((ar.shape[0], N), dtype=np.float64)
        nb_of = np.arange(N) // blk
        for kb in range(nkb):
            k0, k1 = kb * blk, min(K, (kb + 1) * blk)
            d = ar[:, k0:k1] @ b64[:, k0:k1].T
            y = y + (s_rows[:, kb][:, None] * sb2[nb_of, kb][None, :]) * d
    if bias is not None:
        bv = (np.ascontiguousarray(bias, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
        y = y + bv.astype(np.float64)[None, :]
    y = np.ascontiguousarray(y)
    if gelu:
        lib().tfq_oracle_gelu_tanh_array(_ptr(y), y.size)
    return y


def int8_linear_fast(a_q, a_scale, b_q, b_scale, bias=None, rows=None):
    """int8_linear with the integer sums formed by a binary64 matmul (exact:
    |q| <= 128 so |sum| < 2^31 << 2^53 for K <= 131071) and the BF16
    epilogue by the C function.  Returns (acc int64 [R,N], y bf16 bits [R,N]).
    Pinned equal to int8_linear in tests/test_oracle_gemm.py."""
    a = np.ascontiguousarray(a_q).view(np.uint8)
    M, K = a.shape
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    ar = _code_values64(a if r is None else a[r], QTYPE_INT8)
    b64 = _code_values64(b_q, QTYPE_INT8)
    N = b64.shape[0]
    assert b64.shape[1] == K and K <= 131071
    acc = np.ascontiguousarray((ar @ b64.T).astype(np.int64))
    sa = np.ascontiguousarray(a_scale, dtype=np.float32)
    sb = np.ascontiguousarray(b_scale, dtype=np.float32)
    bi = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16)
    y = np.empty(acc.shape, dtype=np.uint16)
    lib().tfq_oracle_int8_epilogue(_ptr(acc), _ptr(sa), _ptr(sb), acc.shape[0], N, _ptr(bi),
                                   _ptr(r), _ptr(y))
    return acc, y


def mx_scale_code(amax: float) -> int:
    """E8M0 byte of a 32-element block with largest magnitude amax (OCP MX v1.0 rule)."""
    return int(lib().tfq_oracle_mx_scale_code(float(amax)))


def quantize_mx(x_bf16: np.ndarray):
    """MXFP8 quantisation of BF16 rows: (codes uint8 [R, C], E8M0 scales uint8 [R, C/32])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    R, C = x.shape
    assert C % 32 == 0
    q = np.empty((R, C), dtype=np.uint8)
    s = np.empty((R, C // 32), dtype=np.uint8)
    lib().tfq_oracle_quantize_mx(_ptr(x), R, C, C, _ptr(q), _ptr(s))
    return q, s


def linear_mx_ref(a_q, a_scale, b_q, b_scale, bias=None, gelu: bool = False, rows=None) -> np.ndarray:
    """MXFP8 Linear reference y [R, N] in binary64 (see tfq_oracle_linear_mx_ref)."""
    a = np.ascontiguousarray(a_q).view(np.uint8)
    b = np.ascontiguousarray(b_q).view(np.uint8)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape[1] == K and K % 32 == 0
    sa = np.ascontiguousarray(a_scale, dtype=np.uint8)
    sb = np.ascontiguousarray(b_scale, dtype=np.uint8)
    assert sa.shape == (M, K // 32) and sb.shape == (N, K // 32)
    bi = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16)
    r, nr = _rows_arg(rows)
    R = M if r is None else nr
    out = np.empty((R, N), dtype=np.float64)
    lib().tfq_oracle_linear_mx_ref(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), M, N, K, _ptr(bi),
                                   1 if gelu else 0, _ptr(r), nr, _ptr(out))
    return out


# --------------------------------------------------------------------------
# MoE routed W8A8 -- TeleFuser "Quantization", "Other quantized data paths"
# (LingBot-Video MoE FP8): expert weights quantised per output channel,
# the routed activations quantised per row, then one scaled matmul per
# expert.  Reading: the routed rows of an expert are contiguous (rows
# offsets[e] .. offsets[e+1]); which token goes to which row is the router's
# choice, given here as a row index.
# --------------------------------------------------------------------------
def gather_rows(x_bf16: np.ndarray, index) -> np.ndarray:
    """Rows index[r] of x (BF16 bits); an index outside [0, rows) gives a zero row."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    idx = np.asarray(index, dtype=np.int64)
    out = np.zeros((idx.shape[0], x.shape[1]), dtype=np.uint16)
    ok = (idx >= 0) & (idx < x.shape[0])
    out[ok] = x[idx[ok]]
    return out


def quantize_rows_gather(x_bf16: np.ndarray, index, qtype, qmax: float, group: int = 0):
    """Per-row (or 1x128-group) quantisation of the gathered rows x[index[r]]."""
    return quantize_rows(gather_rows(x_bf16, index), qtype, qmax, group)


def grouped_linear_ref(a_q, a_scale, b_q, b_scale, offsets, qtype="fp8", bias=None,
                       gelu: bool = False, rows=None) -> np.ndarray:
    """Routed Linear y [R, N] in binary64: row m of group e (offsets[e] <= m <
    offsets[e+1]) is the scaled Linear of a[m] against expert e's weights
    b_q[e] [N, K], b_scale[e] [N] (and bias[e]); rows in no group are NaN.
    offsets: non-decreasing, offsets[0] >= 0, offsets[-1] <= M."""
    a = np.ascontiguousarray(a_q).view(np.uint8)
    b = np.ascontiguousarray(b_q).view(np.uint8)
    M, K = a.shape
    E, N, Kb = b.shape
    assert Kb == K
    off = np.asarray(offsets, dtype=np.int64)
    assert off.shape == (E + 1,) and off[0] >= 0 and off[-1] <= M and np.all(np.diff(off) >= 0)
    sel = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.full((sel.shape[0], N), np.nan)
    group_of = np.searchsorted(off, sel, side="right") - 1
    for e in range(E):
        pick = np.nonzero((group_of == e) & (sel < off[e + 1]))[0]
        if pick.size == 0:
            continue
        out[pick] = linear_ref(a, a_scale, b[e], np.asarray(b_scale)[e], qtype,
                               bias=None if bias is None else np.asarray(bias)[e], gelu=gelu,
                               rows=sel[pick])
    return out


# --------------------------------------------------------------------------
# FP8 KV cache -- TeleFuser "Quantization", "Other quantized data paths"
# (LiveAct FP8 KV cache): K and V stored as E4M3FN with one FP32 scale per
# last-dimension vector, dequantised to the attention's dtype on load.
# Readings: a vector is quantised exactly as a row of the FP8 activation
# path (absmax / qmax, qmax = 448 by default); dequantisation is the binary32
# product scale * value, then one conversion (RNE) to the requested type;
# tokens are written to / read from cache slots named by an index, and an
# index outside the cache is skipped (store) or reads as zeros (load).
# --------------------------------------------------------------------------
KV_DTYPES = {"bf16": 0, "fp16": 1, "fp32": 2}


def kv_store(kv_bf16: np.ndarray, slot, cache: np.ndarray, scale: np.ndarray,
             qmax: float = 448.0) -> None:
    """Quantise kv [tokens, heads, head_dim] (BF16 bits) per (token, head)
    vector into cache [slots, heads, head_dim] (uint8) and scale [slots, heads]
    (float32) at rows slot[token], in place; out-of-range slots are skipped.
    Slots must be distinct."""
    kv = np.ascontiguousarray(kv_bf16, dtype=np.uint16)
    T, H, D = kv.shape
    sl = np.asarray(slot, dtype=np.int64)
    ok = (sl >= 0) & (sl < cache.shape[0])
    assert np.unique(sl[ok]).size == int(ok.sum()), "distinct slots"
    if not ok.any():
        return
    q, s = quantize_rows(kv[ok].reshape(-1, D), "fp8", qmax)
    cache[sl[ok]] = q.reshape(-1, H, D)
    scale[sl[ok]] = s.reshape(-1, H)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """binary32 -> BF16 bits, round to nearest even (finite values)."""
    b = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def kv_load(cache: np.ndarray, scale: np.ndarray, index, out_dtype: str = "bf16") -> np.ndarray:
    """Dequantised rows index[i] of the cache: [n, heads, head_dim] as BF16
    bits (uint16), FP16 bits (uint16) or float32; out-of-range rows are zero."""
    idx = np.asarray(index, dtype=np.int64)
    S, H, D = cache.shape
    ok = (idx >= 0) & (idx < S)
    vals = e4m3fn_table().astype(np.float32)
    prod = np.zeros((idx.shape[0], H, D), dtype=np.float32)
    prod[ok] = np.asarray(scale, dtype=np.float32)[idx[ok]][:, :, None] * vals[cache[idx[ok]]]
    if out_dtype == "fp32":
        return prod
    if out_dtype == "bf16":
        return f32_to_bf16_bits(prod)
    if out_dtype == "fp16":
        with np.errstate(over="ignore"):  # beyond FP16's range: infinity
            return prod.astype(np.float16).view(np.uint16)
    raise ValueError(out_dtype)


def e2m1_value(code: int) -> float:
    """E2M1 (FP4) value of the low 4 bits of code."""
    return lib().tfq_oracle_e2m1_value(code)


def e2m1_encode(v: float) -> int:
    return int(lib().tfq_oracle_e2m1_encode(v))


def mx4_scale_code(amax: float) -> int:
    """E8M0 byte of an MXFP4 block with largest magnitude amax (OCP MX v1.0 rule)."""
    return int(lib().tfq_oracle_mx4_scale_code(float(amax)))


def quantize_mx4(x_bf16: np.ndarray):
    """MXFP4 quantisation of BF16 rows: (codes uint8 [R, C/2], two per byte,
    lower index in the low nibble; E8M0 scales uint8 [R, C/32])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    R, C = x.shape
    assert C % 32 == 0
    q = np.empty((R, C // 2), dtype=np.uint8)
    s = np.empty((R, C // 32), dtype=np.uint8)
    lib().tfq_oracle_quantize_mx4(_ptr(x), R, C, C, _ptr(q), _ptr(s))
    return q, s


def linear_mx4_ref(a_q, a_scale, b_q, b_scale, bias=None, gelu: bool = False,
                   rows=None) -> np.ndarray:
    """MXFP4 Linear reference y [R, N] in binary64 (see tfq_oracle_linear_mx4_ref)."""
    a = np.ascontiguousarray(a_q, dtype=np.uint8)
    b = np.ascontiguousarray(b_q, dtype=np.uint8)
    M, K2 = a.shape
    N = b.shape[0]
    K = 2 * K2
    assert b.shape[1] == K2 and K % 32 == 0
    sa = np.ascontiguousarray(a_scale, dtype=np.uint8)
    sb = np.ascontiguousarray(b_scale, dtype=np.uint8)
    assert sa.shape == (M, K // 32) and sb.shape == (N, K // 32)
    bi = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16)
    r, nr = _rows_arg(rows)
    R = M if r is None else nr
    out = np.empty((R, N), dtype=np.float64)
    lib().tfq_oracle_linear_mx4_ref(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), M, N, K, _ptr(bi),
                                    1 if gelu else 0, _ptr(r), nr, _ptr(out))
    return out


FP6_FORMATS = {"e2m3": 0, "e3m2": 1}


def _fp6(fmt) -> int:
    return FP6_FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def fp6_value(fmt, code: int) -> float:
    """Value of a 6-bit E2M3 / E3M2 code (sign in bit 5)."""
    return lib().tfq_oracle_fp6_value(_fp6(fmt), code)


def fp6_encode(fmt, v: float) -> int:
    return int(lib().tfq_oracle_fp6_encode(_fp6(fmt), v))


def mx6_scale_code(fmt, amax: float) -> int:
    return int(lib().tfq_oracle_mx6_scale_code(_fp6(fmt), float(amax)))


def quantize_mx6(x_bf16: np.ndarray, fmt):
    """MXFP6 quantisation of BF16 rows: (codes uint8 [R, 3C/4], a little-endian
    6-bit stream per row; E8M0 scales uint8 [R, C/32])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    R, C = x.shape
    assert C % 32 == 0
    q = np.empty((R, C * 3 // 4), dtype=np.uint8)
    s = np.empty((R, C // 32), dtype=np.uint8)
    lib().tfq_oracle_quantize_mx6(_fp6(fmt), _ptr(x), R, C, C, _ptr(q), _ptr(s))
    return q, s


def linear_mx6_ref(a_q, a_scale, b_q, b_scale, fmt, bias=None, gelu: bool = False,
                   rows=None) -> np.ndarray:
    """MXFP6 Linear reference y [R, N] in binary64."""
    a = np.ascontiguousarray(a_q, dtype=np.uint8)
    b = np.ascontiguousarray(b_q, dtype=np.uint8)
    M, KB = a.shape
    N = b.shape[0]
    K = KB * 4 // 3
    assert b.shape[1] == KB and K % 32 == 0
    sa = np.ascontiguousarray(a_scale, dtype=np.uint8)
    sb = np.ascontiguousarray(b_scale, dtype=np.uint8)
    assert sa.shape == (M, K // 32) and sb.shape == (N, K // 32)
    bi = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16)
    r, nr = _rows_arg(rows)
    R = M if r is None else nr
    out = np.empty((R, N), dtype=np.float64)
    lib().tfq_oracle_linear_mx6_ref(_fp6(fmt), _ptr(a), _ptr(sa), _ptr(b), _ptr(sb), M, N, K,
                                    _ptr(bi), 1 if gelu else 0, _ptr(r), nr, _ptr(out))
    return out


def int8_linear(a_q, a_scale, b_q, b_scale, bias=None, rows=None, want_acc=True,
                want_bf16=True):
    """INT8 W8A8: (acc int64 [R,N] or None, y bf16 bits uint16 [R,N] or None)."""
    a = np.ascontiguousarray(a_q).view(np.int8)
    b = np.ascontiguousarray(b_q).view(np.int8)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape[1] == K
    sa = np.ascontiguousarray(a_scale, dtype=np.float32)
    sb = np.ascontiguousarray(b_scale, dtype=np.float32)
    bi = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16)
    r, nr = _rows_arg(rows)
    R = M if r is None else nr
    acc = np.empty((R, N), dtype=np.int64) if want_acc else None
    y = np.empty((R, N), dtype=np.uint16) if want_bf16 else None
    lib().tfq_oracle_int8_linear(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), M, N, K, _ptr(bi),
                                 _ptr(r), nr, _ptr(acc), _ptr(y))
    return acc, y


def error_measures(yq: np.ndarray, y: np.ndarray) -> tuple[float, float]:
    """(E_max, E_rel) of the pages' operator comparison."""
    a = np.ascontiguousarray(yq, dtype=np.float64).ravel()
    b = np.ascontiguousarray(y, dtype=np.float64).ravel()
    emax = ctypes.c_double(0)
    erel = ctypes.c_double(0)
    lib().tfq_oracle_error_measures(_ptr(a), _ptr(b), a.shape[0], ctypes.byref(emax),
                                    ctypes.byref(erel))
    return emax.value, erel.value


def bf16_bits_to_f64(h: np.ndarray) -> np.ndarray:
    """Exact decode of BF16 bit arrays (upper half of binary32)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
