"""ctypes loader for libtfq.so (the HIP kernels behind the C ABI of include/tfq.h).

There is no fallback: if the library is missing or a call fails, an exception
is raised.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtfq.so")

STATUS_NAMES = {
    0: "TFQ_OK",
    1: "TFQ_ERR_NULL_POINTER",
    2: "TFQ_ERR_BAD_SHAPE",
    3: "TFQ_ERR_MISALIGNED",
    4: "TFQ_ERR_BAD_QMAX",
    5: "TFQ_ERR_WORKSPACE_TOO_SMALL",
    6: "TFQ_ERR_ALIAS",
    7: "TFQ_ERR_UNSUPPORTED",
    8: "TFQ_ERR_UNSUPPORTED_DEVICE",
    9: "TFQ_ERR_HIP",
}

# (name, restype, argtypes) of every entry point declared in include/tfq.h
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F = ctypes.c_float
SIGNATURES = [
    ("tfq_quantize_rows", _I32, [_P, _I64, _I64, _I64, _I32, _F, _I32, _P, _P, _P]),
    ("tfq_quantize_rows_gather", _I32, [_P, _I64, _I64, _I64, _P, _I64, _I32, _F, _I32, _P, _P,
                                         _P]),
    ("tfq_quantize_weight_per_channel", _I32, [_P, _I64, _I64, _I32, _F, _I32, _P, _P, _P]),
    ("tfq_grouped_scaled_mm_fp8", _I32, [_P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _P, _I32, _P,
                                         _P]),
    ("tfq_scaled_mm_fp8", _I32, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _I32, _P, _P]),
    ("tfq_scaled_mm_int8", _I32, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _I32, _P, _P, _P]),
    ("tfq_quant_linear_workspace_bytes", ctypes.c_size_t, [_I64, _I64, _I32, _I32]),
    ("tfq_quant_linear_fused", _I32, [_P, _I64, _I64, _I64, _P, _P, _I64, _I32, _F, _I32, _P,
                                      _I32, _P, _P, ctypes.c_size_t, _P]),
    ("tfq_quantize_mx", _I32, [_P, _I64, _I64, _I64, _P, _P, _P]),
    ("tfq_scaled_mm_mxfp8", _I32, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _I32, _P, _P]),
    ("tfq_quantize_mxfp4", _I32, [_P, _I64, _I64, _I64, _P, _P, _P]),
    ("tfq_scaled_mm_mxfp4", _I32, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _I32, _P, _P]),
    ("tfq_quantize_mxfp6", _I32, [_P, _I64, _I64, _I64, _I32, _P, _P, _P]),
    ("tfq_scaled_mm_mxfp6", _I32, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _I32, _P, _P]),
    ("tfq_kv_cache_store", _I32, [_P, _I64, _I64, _I64, _I64, _P, _I64, _F, _P, _P, _P]),
    ("tfq_kv_cache_load", _I32, [_P, _P, _I64, _I64, _I64, _P, _I64, _I32, _P, _P]),
    ("tfq_set_autotune", _I32, [_I32]),
    ("tfq_autotune_lookup", _I32, [_I32, _I64, _I64, _I64, _I32, _I32, _P, _P]),
    ("tfq_autotune_clear", None, []),
    ("tfq_autotune_set", _I32, [_I32, _I64, _I64, _I64, _I32, _I32, _I32, _I32]),
    ("tfq_quant_linear_fused_noalloc", _I32, [_P, _I64, _I64, _I64, _P, _P, _I64, _I32, _F, _I32,
                                              _P, _I32, _P, _P]),
    ("tfq_e4m3fn_encode_f32", _I32, [_P, _P, _I64, _P]),
    ("tfq_status_string", ctypes.c_char_p, [_I32]),
    ("tfq_last_hip_error", ctypes.c_int, []),
    ("tfq_abi_version", ctypes.c_int, []),
]


class TfqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = STATUS_NAMES.get(status, str(status))
        try:
            detail = lib().tfq_status_string(status).decode()
        except Exception:  # pragma: no cover - message only
            detail = ""
        extra = ""
        if status == 9:
            extra = f" (hipError {lib().tfq_last_hip_error()})"
        super().__init__(f"{where}: {msg}: {detail}{extra}")


_lib = None


def lib():
    """Load libtfq.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m int8_w8a8_quantized_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status: int, where: str) -> None:
    if status != 0:
        raise TfqError(status, where)
