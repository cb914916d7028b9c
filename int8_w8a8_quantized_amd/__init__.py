"""MI355X (gfx950) W8A8 scaled-quantized Linear.

Thin Python binding over the C ABI of ``include/tfq.h`` (``libtfq.so``): every
function below has the name of the C entry point it calls and only marshals
arguments -- torch tensors supply device memory and the current HIP stream;
all quantisation and GEMM work runs in the library's HIP kernels.  There is
no CPU or PyTorch fallback: a missing library or a failing call raises.

Method (web pages, cited by title and section): TeleFuser "Quantization",
"tf-kernel FP8: online W8A8" (per-token activation quantisation at each
forward, per-output-channel weights quantised and cached on first use, BF16
output) and "Core ideas" (symmetric INT8); LightX2V "模型量化技术", table
"量化模式" (fp8-b128-deepgemm block scaling) and "MiniMax-H3 FP8 FP16 累加"
(reduced activation qmax).
"""
from __future__ import annotations

import torch

from ._lib import TfqError, check, lib

__all__ = [
    "TfqError", "QTYPE", "EPI", "tfq_quantize_rows", "tfq_quantize_weight_per_channel",
    "tfq_scaled_mm_fp8", "tfq_scaled_mm_int8", "tfq_quant_linear_workspace_bytes",
    "tfq_quant_linear_fused", "tfq_quant_linear_fused_noalloc", "NOALLOC_WORKSPACE_BYTES",
    "tfq_quantize_mx", "tfq_scaled_mm_mxfp8", "tfq_e4m3fn_encode_f32",
    "tfq_quantize_rows_gather", "tfq_grouped_scaled_mm_fp8", "tfq_kv_cache_store",
    "tfq_kv_cache_load", "KV_DTYPE", "tfq_set_autotune", "tfq_autotune_lookup",
    "tfq_autotune_clear", "tfq_autotune_set", "tfq_quantize_mxfp4", "tfq_scaled_mm_mxfp4", "tfq_quantize_mxfp6",
    "tfq_scaled_mm_mxfp6", "FP6",
    "tfq_abi_version", "QuantLinear",
]

QTYPE = {"fp8": 0, "e4m3fn": 0, "int8": 1}
EPI = {None: 0, "none": 0, "gelu_tanh": 1, "gelu": 1}
KV_DTYPE = {torch.bfloat16: 0, torch.float16: 1, torch.float32: 2}


def _qt(qtype) -> int:
    return QTYPE[qtype] if isinstance(qtype, str) else int(qtype)


def _epi(epi) -> int:
    return EPI[epi] if (epi is None or isinstance(epi, str)) else int(epi)


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _torch_stream(stream):
    """`stream` (a torch stream or a raw hipStream_t handle) as a torch stream."""
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _on_stream(fn):
    """Run a wrapper with the caller's `stream` (when one is given) as torch's
    current stream, so that every tensor the wrapper allocates -- outputs,
    the fused call's workspace -- belongs to that stream in torch's caching
    allocator: a block freed there is handed out again only to later work on
    the same stream, never to another stream while the kernels still use it.
    The kernels run on that stream either way."""
    import functools
    import inspect

    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        bound = sig.bind_partial(*args, **kwargs)
        st = bound.arguments.get("stream")
        if st is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(_torch_stream(st)):
            return fn(*args, **kwargs)

    return wrapper


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _code_dtype(qt: int):
    return torch.uint8 if qt == 0 else torch.int8


# accepted element types: one-byte codes, FP32 scales, BF16 data, int32
# indices, and MX scale words (viewed as bytes or 32-bit words)
_CODES = (torch.uint8, torch.int8, torch.float8_e4m3fn)
_F32 = (torch.float32,)
_BF16 = (torch.bfloat16,)
_I32 = (torch.int32,)
_MXS = (torch.uint8, torch.int32)


def _arg(t, name, dtypes, shape=None, numel=None, rows=False):
    """Check a tensor argument before its pointer reaches the library: a
    tensor of one of `dtypes`, of `shape` (None entries match any size) or
    `numel` elements; `rows`: a 2-D tensor whose rows are contiguous (any row
    stride), else contiguous as a whole.  Raises TypeError / ValueError naming
    the argument.  (Device memory is checked by _gpu, once every argument's
    type and shape have been.)"""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if shape is not None and (t.dim() != len(shape) or
                              any(w is not None and g != w for g, w in zip(t.shape, shape))):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {shape}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    if rows:
        if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1) or t.stride(0) < t.shape[1]:
            raise ValueError(f"{name}: expected a 2-D tensor with contiguous rows")
    elif not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


def _gpu(**named):
    """Every tensor given (None skipped) must be in GPU memory: the kernels
    take its pointer as a device address."""
    for name, t in named.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name}: must be in GPU memory, got device {t.device}")


def _opt(t, name, dtypes, **kw):
    return None if t is None else _arg(t, name, dtypes, **kw)


def _mx_scales(t, name, rows, k):
    """MX scale words [k/128, rows] (as bytes [k/128, rows, 4] or int32)."""
    return _arg(t, name, _MXS, numel=(k // 128) * rows * (4 if t.dtype == torch.uint8 else 1))


def tfq_abi_version() -> int:
    return lib().tfq_abi_version()


@_on_stream
def tfq_quantize_rows(x: torch.Tensor, qtype="fp8", qmax: float = 448.0, group_cols: int = 0,
                      q_out: torch.Tensor | None = None, scale_out: torch.Tensor | None = None,
                      stream=None):
    """Per-token absmax quantisation of BF16 rows x [rows, cols] (row stride
    x.stride(0)).  Returns (codes [rows, cols], scales [rows] or
    [rows, cols/128])."""
    qt = _qt(qtype)
    _arg(x, "x", _BF16, rows=True)
    rows, cols = x.shape
    if q_out is None:
        q_out = torch.empty((rows, cols), dtype=_code_dtype(qt), device=x.device)
    if scale_out is None:
        shape = (rows,) if group_cols == 0 else (rows, cols // max(group_cols, 1))
        scale_out = torch.empty(shape, dtype=torch.float32, device=x.device)
    _arg(q_out, "q_out", _CODES, shape=(rows, cols))
    _arg(scale_out, "scale_out", _F32, numel=rows if group_cols == 0 else rows * (cols // max(group_cols, 1)))
    _gpu(x=x, q_out=q_out, scale_out=scale_out)
    check(lib().tfq_quantize_rows(_ptr(x), rows, cols, x.stride(0), qt, float(qmax),
                                  int(group_cols), _ptr(q_out), _ptr(scale_out), _stream(stream)),
          "tfq_quantize_rows")
    return q_out, scale_out


@_on_stream
def tfq_quantize_rows_gather(x: torch.Tensor, row_index: torch.Tensor, qtype="fp8",
                             qmax: float = 448.0, group_cols: int = 0, q_out=None, scale_out=None,
                             stream=None):
    """Routed per-token quantisation: output row r quantises x[row_index[r]]
    (row_index int32 on the device; an index outside x's rows gives a zero
    row).  Returns (codes [rows, cols], scales [rows] or [rows, cols/128])."""
    qt = _qt(qtype)
    _arg(x, "x", _BF16, rows=True)
    _arg(row_index, "row_index", _I32, shape=(None,))
    src_rows, cols = x.shape
    rows = row_index.shape[0]
    if q_out is None:
        q_out = torch.empty((rows, cols), dtype=_code_dtype(qt), device=x.device)
    if scale_out is None:
        shape = (rows,) if group_cols == 0 else (rows, cols // max(group_cols, 1))
        scale_out = torch.empty(shape, dtype=torch.float32, device=x.device)
    _arg(q_out, "q_out", _CODES, shape=(rows, cols))
    _arg(scale_out, "scale_out", _F32, numel=rows if group_cols == 0 else rows * (cols // max(group_cols, 1)))
    _gpu(x=x, row_index=row_index, q_out=q_out, scale_out=scale_out)
    check(lib().tfq_quantize_rows_gather(_ptr(x), src_rows, cols, x.stride(0), _ptr(row_index),
                                         rows, qt, float(qmax), int(group_cols), _ptr(q_out),
                                         _ptr(scale_out), _stream(stream)),
          "tfq_quantize_rows_gather")
    return q_out, scale_out


@_on_stream
def tfq_quantize_weight_per_channel(w: torch.Tensor, qtype="fp8", qmax: float = 448.0,
                                    block: int = 0, q_out=None, scale_out=None, stream=None):
    """Weights W [n, k] BF16 -> (codes [n, k], scales [n] or [n/128, k/128])."""
    qt = _qt(qtype)
    _arg(w, "w", _BF16, shape=(None, None))
    n, k = w.shape
    if q_out is None:
        q_out = torch.empty((n, k), dtype=_code_dtype(qt), device=w.device)
    if scale_out is None:
        shape = (n,) if block == 0 else (n // block, k // block)
        scale_out = torch.empty(shape, dtype=torch.float32, device=w.device)
    _arg(q_out, "q_out", _CODES, shape=(n, k))
    _arg(scale_out, "scale_out", _F32, numel=n if block == 0 else (n // block) * (k // block))
    _gpu(w=w, q_out=q_out, scale_out=scale_out)
    check(lib().tfq_quantize_weight_per_channel(_ptr(w), n, k, qt, float(qmax), int(block),
                                                _ptr(q_out), _ptr(scale_out), _stream(stream)),
          "tfq_quantize_weight_per_channel")
    return q_out, scale_out


@_on_stream
def tfq_scaled_mm_fp8(a_q, a_scale, b_q, b_scale, scale_block: int = 0, bias=None, epi=None,
                      y=None, stream=None):
    """y [m, n] BF16 = (a_q [m,k] . b_q [n,k]^T) scaled per row / column (or per block)."""
    m, k = _arg(a_q, "a_q", _CODES, shape=(None, None)).shape
    n = _arg(b_q, "b_q", _CODES, shape=(None, k)).shape[0]
    blk = int(scale_block)
    _arg(a_scale, "a_scale", _F32, numel=m if blk == 0 else m * (-(-k // 128)))
    _arg(b_scale, "b_scale", _F32, numel=n if blk == 0 else (-(-n // 128)) * (-(-k // 128)))
    _opt(bias, "bias", _BF16, numel=n)
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=a_q.device)
    _arg(y, "y", _BF16, shape=(m, n))
    _gpu(a_q=a_q, a_scale=a_scale, b_q=b_q, b_scale=b_scale, bias=bias, y=y)
    check(lib().tfq_scaled_mm_fp8(_ptr(a_q), _ptr(a_scale), _ptr(b_q), _ptr(b_scale), m, n, k,
                                  int(scale_block), _ptr(bias), _epi(epi), _ptr(y),
                                  _stream(stream)), "tfq_scaled_mm_fp8")
    return y


@_on_stream
def tfq_scaled_mm_int8(a_q, a_scale, b_q, b_scale, bias=None, epi=None, want_y: bool = True,
                       want_acc: bool = False, y=None, acc=None, stream=None):
    """INT8 scaled GEMM; returns (y BF16 or None, acc INT32 or None)."""
    m, k = _arg(a_q, "a_q", _CODES, shape=(None, None)).shape
    n = _arg(b_q, "b_q", _CODES, shape=(None, k)).shape[0]
    _arg(a_scale, "a_scale", _F32, numel=m)
    _arg(b_scale, "b_scale", _F32, numel=n)
    _opt(bias, "bias", _BF16, numel=n)
    if want_y and y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=a_q.device)
    if want_acc and acc is None:
        acc = torch.empty((m, n), dtype=torch.int32, device=a_q.device)
    _opt(y, "y", _BF16, shape=(m, n))
    _opt(acc, "acc", _I32, shape=(m, n))
    _gpu(a_q=a_q, a_scale=a_scale, b_q=b_q, b_scale=b_scale, bias=bias, y=y, acc=acc)
    check(lib().tfq_scaled_mm_int8(_ptr(a_q), _ptr(a_scale), _ptr(b_q), _ptr(b_scale), m, n, k,
                                   _ptr(bias), _epi(epi), _ptr(y), _ptr(acc), _stream(stream)),
          "tfq_scaled_mm_int8")
    return y, acc


@_on_stream
def tfq_grouped_scaled_mm_fp8(a_q, a_scale, b_q, b_scale, group_offsets, bias=None, epi=None,
                              y=None, stream=None):
    """Grouped (MoE) FP8 GEMM: rows group_offsets[g]..group_offsets[g+1] of
    a_q [m, k] against expert g's b_q[g] [n, k]; group_offsets int32 on the
    device.  Returns y [m, n] BF16 (rows in no group are left as allocated)."""
    m, k = _arg(a_q, "a_q", _CODES, shape=(None, None)).shape
    groups, n, _ = _arg(b_q, "b_q", _CODES, shape=(None, None, k)).shape
    _arg(a_scale, "a_scale", _F32, numel=m)
    _arg(b_scale, "b_scale", _F32, numel=groups * n)
    _arg(group_offsets, "group_offsets", _I32, numel=groups + 1)
    _opt(bias, "bias", _BF16, numel=groups * n)
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=a_q.device)
    _arg(y, "y", _BF16, shape=(m, n))
    _gpu(a_q=a_q, a_scale=a_scale, b_q=b_q, b_scale=b_scale, group_offsets=group_offsets, bias=bias, y=y)
    check(lib().tfq_grouped_scaled_mm_fp8(_ptr(a_q), _ptr(a_scale), _ptr(b_q), _ptr(b_scale),
                                          _ptr(group_offsets), groups, m, n, k, _ptr(bias),
                                          _epi(epi), _ptr(y), _stream(stream)),
          "tfq_grouped_scaled_mm_fp8")
    return y


def tfq_quant_linear_workspace_bytes(m: int, k: int, qtype="fp8", scale_block: int = 0) -> int:
    return int(lib().tfq_quant_linear_workspace_bytes(m, k, _qt(qtype), int(scale_block)))


@_on_stream
def tfq_quant_linear_fused(x, w_q, w_scale, qtype="fp8", act_qmax: float = 448.0,
                           scale_block: int = 0, bias=None, epi=None, y=None, workspace=None,
                           stream=None):
    """The W8A8 Linear forward: quantise x [m, k] per token, then the scaled
    GEMM against pre-quantised weights; returns y [m, n] BF16."""
    qt = _qt(qtype)
    m, k = _arg(x, "x", _BF16, rows=True).shape
    n = _arg(w_q, "w_q", _CODES, shape=(None, k)).shape[0]
    blk = int(scale_block)
    _arg(w_scale, "w_scale", _F32, numel=n if blk == 0 else (-(-n // 128)) * (-(-k // 128)))
    _opt(bias, "bias", _BF16, numel=n)
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    _arg(y, "y", _BF16, shape=(m, n))
    need = tfq_quant_linear_workspace_bytes(m, k, qt, scale_block)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _arg(workspace, "workspace", (torch.uint8,), shape=(None,))
    _gpu(x=x, w_q=w_q, w_scale=w_scale, bias=bias, y=y, workspace=workspace)
    check(lib().tfq_quant_linear_fused(_ptr(x), m, k, x.stride(0), _ptr(w_q), _ptr(w_scale), n, qt,
                                       float(act_qmax), int(scale_block), _ptr(bias), _epi(epi),
                                       _ptr(y), _ptr(workspace), workspace.numel(),
                                       _stream(stream)), "tfq_quant_linear_fused")
    return y


NOALLOC_WORKSPACE_BYTES = 64 << 20  # TFQ_NOALLOC_WORKSPACE_BYTES of include/tfq.h


def tfq_quant_linear_fused_noalloc(x, w_q, w_scale, y, qtype="fp8", act_qmax: float = 448.0,
                                   scale_block: int = 0, bias=None, epi=None, stream=None):
    """tfq_quant_linear_fused with the activation codes in the library's own
    per-GPU device scratch: the C call allocates nothing (the caller passes
    the output y [m, n] BF16).  Calls that overlap in time on one GPU race."""
    qt = _qt(qtype)
    m, k = _arg(x, "x", _BF16, rows=True).shape
    n = _arg(w_q, "w_q", _CODES, shape=(None, k)).shape[0]
    blk = int(scale_block)
    _arg(w_scale, "w_scale", _F32, numel=n if blk == 0 else (-(-n // 128)) * (-(-k // 128)))
    _opt(bias, "bias", _BF16, numel=n)
    _arg(y, "y", _BF16, shape=(m, n))
    _gpu(x=x, w_q=w_q, w_scale=w_scale, bias=bias, y=y)
    check(lib().tfq_quant_linear_fused_noalloc(_ptr(x), m, k, x.stride(0), _ptr(w_q), _ptr(w_scale),
                                               n, qt, float(act_qmax), blk, _ptr(bias), _epi(epi),
                                               _ptr(y), _stream(stream)),
          "tfq_quant_linear_fused_noalloc")
    return y


@_on_stream
def tfq_quantize_mx(x: torch.Tensor, q_out=None, scale_out=None, stream=None):
    """MXFP8 quantisation of BF16 rows x [rows, cols] (row stride x.stride(0)):
    returns (E4M3FN codes [rows, cols], E8M0 scales as uint8
    [cols/128, rows, 4]: entries (g, r, 0..3) are the scales of blocks
    4 g, 4 g + 2, 4 g + 1, 4 g + 3 of row r)."""
    rows, cols = _arg(x, "x", _BF16, rows=True).shape
    if q_out is None:
        q_out = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scale_out is None:
        scale_out = torch.empty((cols // 128, rows, 4), dtype=torch.uint8, device=x.device)
    _arg(q_out, "q_out", _CODES, shape=(rows, cols))
    _mx_scales(scale_out, "scale_out", rows, cols)
    _gpu(x=x, q_out=q_out, scale_out=scale_out)
    check(lib().tfq_quantize_mx(_ptr(x), rows, cols, x.stride(0), _ptr(q_out), _ptr(scale_out),
                                _stream(stream)), "tfq_quantize_mx")
    return q_out, scale_out


@_on_stream
def tfq_scaled_mm_mxfp8(a_q, a_scale, b_q, b_scale, bias=None, epi=None, y=None, stream=None):
    """y [m, n] BF16 from MXFP8 operands a_q [m, k], b_q [n, k] with E8M0
    block scales in the layout tfq_quantize_mx returns ([k/128, m, 4] and
    [k/128, n, 4])."""
    m, k = _arg(a_q, "a_q", _CODES, shape=(None, None)).shape
    n = _arg(b_q, "b_q", _CODES, shape=(None, k)).shape[0]
    _mx_scales(a_scale, "a_scale", m, k)
    _mx_scales(b_scale, "b_scale", n, k)
    _opt(bias, "bias", _BF16, numel=n)
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=a_q.device)
    _arg(y, "y", _BF16, shape=(m, n))
    _gpu(a_q=a_q, a_scale=a_scale, b_q=b_q, b_scale=b_scale, bias=bias, y=y)
    check(lib().tfq_scaled_mm_mxfp8(_ptr(a_q), _ptr(a_scale), _ptr(b_q), _ptr(b_scale), m, n, k,
                                    _ptr(bias), _epi(epi), _ptr(y), _stream(stream)),
          "tfq_scaled_mm_mxfp8")
    return y


@_on_stream
def tfq_kv_cache_store(kv: torch.Tensor, slot_index: torch.Tensor, cache: torch.Tensor,
                       cache_scale: torch.Tensor, qmax: float = 448.0, stream=None):
    """Quantise kv [tokens, heads, head_dim] BF16 (heads and head_dim
    contiguous) per vector into cache [slots, heads, head_dim] uint8 and
    cache_scale [slots, heads] FP32 at rows slot_index[t] (int32, device)."""
    if not isinstance(kv, torch.Tensor) or kv.dtype != torch.bfloat16 or kv.dim() != 3:
        raise TypeError("kv: expected a 3-D bfloat16 tensor [tokens, heads, head_dim]")
    tokens, heads, hd = kv.shape
    if kv.stride(2) != 1 or kv.stride(1) != hd or kv.stride(0) < heads * hd:
        raise ValueError("kv: heads and head_dim must be contiguous")
    _arg(slot_index, "slot_index", _I32, numel=tokens)
    slots = _arg(cache, "cache", (torch.uint8,), shape=(None, heads, hd)).shape[0]
    _arg(cache_scale, "cache_scale", _F32, shape=(slots, heads))
    _gpu(kv=kv, slot_index=slot_index, cache=cache, cache_scale=cache_scale)
    check(lib().tfq_kv_cache_store(_ptr(kv), tokens, heads, hd, kv.stride(0), _ptr(slot_index),
                                   cache.shape[0], float(qmax), _ptr(cache), _ptr(cache_scale),
                                   _stream(stream)), "tfq_kv_cache_store")


@_on_stream
def tfq_kv_cache_load(cache: torch.Tensor, cache_scale: torch.Tensor, slot_index: torch.Tensor,
                      dtype=torch.bfloat16, out=None, stream=None):
    """Dequantised cache rows slot_index[i]: [n, heads, head_dim] in dtype
    (bfloat16, float16 or float32)."""
    slots, heads, hd = _arg(cache, "cache", (torch.uint8,), shape=(None, None, None)).shape
    _arg(cache_scale, "cache_scale", _F32, shape=(slots, heads))
    n = _arg(slot_index, "slot_index", _I32, shape=(None,)).shape[0]
    if out is None:
        out = torch.empty((n, heads, hd), dtype=dtype, device=cache.device)
    _arg(out, "out", tuple(KV_DTYPE), shape=(n, heads, hd))
    _gpu(cache=cache, cache_scale=cache_scale, slot_index=slot_index, out=out)
    check(lib().tfq_kv_cache_load(_ptr(cache), _ptr(cache_scale), slots, heads, hd,
                                  _ptr(slot_index), n, KV_DTYPE[out.dtype], _ptr(out),
                                  _stream(stream)), "tfq_kv_cache_load")
    return out


def tfq_set_autotune(mode: int) -> None:
    """0: fixed heuristic GEMM configurations (default); 1: tune each GEMM
    shape on its first call and cache the winner in this process."""
    check(lib().tfq_set_autotune(int(mode)), "tfq_set_autotune")


AUTOTUNE_KIND = {"fp8": 0, "int8": 1, "fp8_block": 2, "mxfp8": 3, "grouped_fp8": 4, "mxfp4": 5,
                 "mxfp6_e2m3": 6, "mxfp6_e3m2": 7}
FP6 = {"e2m3": 0, "e3m2": 1}


def tfq_autotune_lookup(kind, m: int, n: int, k: int, epi=None, groups: int = 0):
    """(kernel, band) cached for a GEMM shape on the current device, or None."""
    import ctypes

    kern, band = ctypes.c_int32(0), ctypes.c_int32(0)
    kd = AUTOTUNE_KIND[kind] if isinstance(kind, str) else int(kind)
    found = lib().tfq_autotune_lookup(kd, m, n, k, _epi(epi), int(groups), ctypes.byref(kern),
                                      ctypes.byref(band))
    return (kern.value, band.value) if found else None


def tfq_autotune_clear() -> None:
    lib().tfq_autotune_clear()


def tfq_autotune_set(kind, m: int, n: int, k: int, kernel: int, band: int, epi=None,
                     groups: int = 0) -> None:
    """Cache launch configuration (kernel, band) for a GEMM shape on the
    current device, as tuning would (used while autotuning is on); it must be
    one of the shape's candidate configurations."""
    kd = AUTOTUNE_KIND[kind] if isinstance(kind, str) else int(kind)
    check(lib().tfq_autotune_set(kd, m, n, k, _epi(epi), int(groups), int(kernel), int(band)),
          "tfq_autotune_set")


@_on_stream
def tfq_quantize_mxfp4(x: torch.Tensor, q_out=None, scale_out=None, stream=None):
    """MXFP4 quantisation of BF16 rows x [rows, cols]: returns (packed E2M1
    codes uint8 [rows, cols/2], lower index in the low nibble; E8M0 scales
    uint8 [cols/128, rows, 4] as tfq_quantize_mx)."""
    rows, cols = _arg(x, "x", _BF16, rows=True).shape
    if q_out is None:
        q_out = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    if scale_out is None:
        scale_out = torch.empty((cols // 128, rows, 4), dtype=torch.uint8, device=x.device)
    _arg(q_out, "q_out", (torch.uint8,), shape=(rows, cols // 2))
    _mx_scales(scale_out, "scale_out", rows, cols)
    _gpu(x=x, q_out=q_out, scale_out=scale_out)
    check(lib().tfq_quantize_mxfp4(_ptr(x), rows, cols, x.stride(0), _ptr(q_out), _ptr(scale_out),
                                   _stream(stream)), "tfq_quantize_mxfp4")
    return q_out, scale_out


@_on_stream
def tfq_scaled_mm_mxfp4(a_q, a_scale, b_q, b_scale, bias=None, epi=None, y=None, stream=None):
    """y [m, n] BF16 from MXFP4 operands a_q [m, k/2], b_q [n, k/2] (packed)."""
    m, k2 = _arg(a_q, "a_q", (torch.uint8,), shape=(None, None)).shape
    n = _arg(b_q, "b_q", (torch.uint8,), shape=(None, k2)).shape[0]
    _mx_scales(a_scale, "a_scale", m, 2 * k2)
    _mx_scales(b_scale, "b_scale", n, 2 * k2)
    _opt(bias, "bias", _BF16, numel=n)
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=a_q.device)
    _arg(y, "y", _BF16, shape=(m, n))
    _gpu(a_q=a_q, a_scale=a_scale, b_q=b_q, b_scale=b_scale, bias=bias, y=y)
    check(lib().tfq_scaled_mm_mxfp4(_ptr(a_q), _ptr(a_scale), _ptr(b_q), _ptr(b_scale), m, n,
                                    2 * k2, _ptr(bias), _epi(epi), _ptr(y), _stream(stream)),
          "tfq_scaled_mm_mxfp4")
    return y


@_on_stream
def tfq_quantize_mxfp6(x: torch.Tensor, fmt="e2m3", q_out=None, scale_out=None, stream=None):
    """MXFP6 quantisation of BF16 rows x [rows, cols] (fmt "e2m3" or "e3m2"):
    returns (codes uint8 [cols/128, rows, 96], group-major: q[g, r] holds the
    128 codes of elements 128 g .. 128 g + 127 of row r as a 6-bit
    little-endian stream; E8M0 scales uint8 [cols/128, rows, 4] as
    tfq_quantize_mx)."""
    rows, cols = _arg(x, "x", _BF16, rows=True).shape
    if fmt not in FP6:
        raise ValueError(f"fmt: {fmt!r}, expected one of {list(FP6)}")
    if q_out is None:
        q_out = torch.empty((cols // 128, rows, 96), dtype=torch.uint8, device=x.device)
    if scale_out is None:
        scale_out = torch.empty((cols // 128, rows, 4), dtype=torch.uint8, device=x.device)
    _arg(q_out, "q_out", (torch.uint8,), shape=(cols // 128, rows, 96))
    _mx_scales(scale_out, "scale_out", rows, cols)
    _gpu(x=x, q_out=q_out, scale_out=scale_out)
    check(lib().tfq_quantize_mxfp6(_ptr(x), rows, cols, x.stride(0), FP6[fmt], _ptr(q_out),
                                   _ptr(scale_out), _stream(stream)), "tfq_quantize_mxfp6")
    return q_out, scale_out


@_on_stream
def tfq_scaled_mm_mxfp6(a_q, a_scale, b_q, b_scale, fmt="e2m3", bias=None, epi=None, y=None,
                        stream=None):
    """y [m, n] BF16 from MXFP6 operands a_q [k/128, m, 96], b_q [k/128, n,
    96] as tfq_quantize_mxfp6 writes them."""
    kg, m, _ = _arg(a_q, "a_q", (torch.uint8,), shape=(None, None, 96)).shape
    n = _arg(b_q, "b_q", (torch.uint8,), shape=(kg, None, 96)).shape[1]
    if fmt not in FP6:
        raise ValueError(f"fmt: {fmt!r}, expected one of {list(FP6)}")
    _mx_scales(a_scale, "a_scale", m, kg * 128)
    _mx_scales(b_scale, "b_scale", n, kg * 128)
    _opt(bias, "bias", _BF16, numel=n)
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=a_q.device)
    _arg(y, "y", _BF16, shape=(m, n))
    _gpu(a_q=a_q, a_scale=a_scale, b_q=b_q, b_scale=b_scale, bias=bias, y=y)
    check(lib().tfq_scaled_mm_mxfp6(_ptr(a_q), _ptr(a_scale), _ptr(b_q), _ptr(b_scale), m, n,
                                    kg * 128, FP6[fmt], _ptr(bias), _epi(epi), _ptr(y),
                                    _stream(stream)), "tfq_scaled_mm_mxfp6")
    return y


@_on_stream
def tfq_e4m3fn_encode_f32(x: torch.Tensor, q=None, stream=None):
    """The device's E4M3FN encoder over a float32 tensor (numel % 4 == 0)."""
    _arg(x, "x", _F32)
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _arg(q, "q", (torch.uint8,), numel=x.numel())
    _gpu(x=x, q=q)
    check(lib().tfq_e4m3fn_encode_f32(_ptr(x), _ptr(q), x.numel(), _stream(stream)),
          "tfq_e4m3fn_encode_f32")
    return q


class QuantLinear:
    """W8A8 Linear holding a BF16 weight [out, in]: the weight is quantised per
    output channel (or per 128x128 block) on the first call and kept resident,
    activations are quantised per token (or per 1x128 group) on every call
    (TeleFuser "Quantization", "tf-kernel FP8: online W8A8").  qtype "mxfp8",
    "mxfp6_e2m3", "mxfp6_e3m2" or "mxfp4" uses the MX formats instead
    (32-element blocks with E8M0 scales, weight and activations alike;
    TeleFuser "Quantization", converter section).  The weight codes are
    cached: after changing the weight in place, call requantize()."""

    MX = {"mxfp8": (tfq_quantize_mx, tfq_scaled_mm_mxfp8),
          "mxfp4": (tfq_quantize_mxfp4, tfq_scaled_mm_mxfp4),
          "mxfp6_e2m3": (lambda x, *o: tfq_quantize_mxfp6(x, "e2m3", *o),
                         lambda *a: tfq_scaled_mm_mxfp6(*a[:4], "e2m3", *a[4:])),
          "mxfp6_e3m2": (lambda x, *o: tfq_quantize_mxfp6(x, "e3m2", *o),
                         lambda *a: tfq_scaled_mm_mxfp6(*a[:4], "e3m2", *a[4:]))}

    def __init__(self, weight: torch.Tensor, bias: torch.Tensor | None = None, qtype="fp8",
                 act_qmax: float | None = None, weight_qmax: float | None = None,
                 scale_block: int = 0, epi=None):
        self.weight = weight
        self.bias = bias
        self.qtype = qtype
        self.mx = self.MX.get(qtype) if isinstance(qtype, str) else None
        default = 448.0 if self.mx or _qt(qtype) == 0 else 127.0
        self.act_qmax = default if act_qmax is None else act_qmax
        self.weight_qmax = default if weight_qmax is None else weight_qmax
        self.scale_block = scale_block
        self.epi = epi
        self.w_q = None
        self.w_scale = None
        self._ws = None
        self._act = None

    def requantize(self) -> None:
        """Drop the cached weight codes and scales: the next call quantises
        the current weight again (after the weight tensor was modified)."""
        self.w_q = None
        self.w_scale = None

    def quantized_weight(self):
        if self.w_q is None:
            if self.mx:
                self.w_q, self.w_scale = self.mx[0](self.weight)
            else:
                self.w_q, self.w_scale = tfq_quantize_weight_per_channel(
                    self.weight, self.qtype, self.weight_qmax, self.scale_block)
        return self.w_q, self.w_scale

    def __call__(self, x: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
        w_q, w_s = self.quantized_weight()
        if self.mx:
            quant, mm = self.mx
            # activation codes and scales are reused while x keeps its shape
            # (the scales are [cols/128, rows, 4] in every MX format; the
            # codes' layout differs between formats)
            if self._act is None or tuple(self._act[1].shape[:2]) != (x.shape[1] // 128, x.shape[0]):
                self._act = quant(x)
            else:
                quant(x, *self._act)
            return mm(self._act[0], self._act[1], w_q, w_s, self.bias, self.epi, y)
        need = tfq_quant_linear_workspace_bytes(x.shape[0], x.shape[1], self.qtype,
                                                self.scale_block)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=x.device)
        return tfq_quant_linear_fused(x, w_q, w_s, self.qtype, self.act_qmax, self.scale_block,
                                      self.bias, self.epi, y, self._ws)
