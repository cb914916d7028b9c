"""Host-side checks of the C ABI that need no GPU.

* libtfq.so loads and exports every function include/tfq.h declares;
* every invalid-argument path returns its status before any HIP call
  (fake, never-dereferenced addresses are passed: these tests are skipped on
  a machine that has a GPU so that a validation bug can never launch a kernel
  on them);
* on a machine without a GPU a valid call reports TFQ_ERR_UNSUPPORTED_DEVICE
  instead of falling back to anything.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HAS_GPU_NODE = os.path.exists("/dev/kfd")

OK, NULL, SHAPE, ALIGN, QMAX, WS, ALIAS, UNSUP, DEV, HIP = range(10)

# fake 256-byte-aligned addresses, far apart; never dereferenced
A, B, C, D, E, F, G = (0x10_0000_0000 * (i + 1) for i in range(7))

no_gpu_only = pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer validation tests run only "
                                 "on machines without a GPU")


@pytest.fixture(scope="module")
def L():
    from int8_w8a8_quantized_amd._lib import lib

    return lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "tfq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tfq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) == 25, names
    for n in names:
        assert hasattr(L, n), n
    from int8_w8a8_quantized_amd._lib import SIGNATURES

    assert sorted(s[0] for s in SIGNATURES) == names


def test_version_and_strings(L):
    assert L.tfq_abi_version() == 9
    for s in range(10):
        assert L.tfq_status_string(s)
    assert L.tfq_last_hip_error() == 0


@no_gpu_only
def test_quantize_rows_validation(L):
    q = L.tfq_quantize_rows
    assert q(None, 4, 64, 64, 0, 448.0, 0, B, C, None) == NULL
    assert q(A, 4, 64, 64, 0, 448.0, 0, None, C, None) == NULL
    assert q(A, 0, 64, 64, 0, 448.0, 0, B, C, None) == SHAPE
    assert q(A, 4, 60, 64, 0, 448.0, 0, B, C, None) == SHAPE      # cols % 16
    assert q(A, 4, 64, 32, 0, 448.0, 0, B, C, None) == SHAPE      # ld < cols
    assert q(A, 4, 64, 68, 0, 448.0, 0, B, C, None) == ALIGN      # ld % 8
    assert q(A + 2, 4, 64, 64, 0, 448.0, 0, B, C, None) == ALIGN
    assert q(A, 4, 64, 64, 0, 448.0, 0, B + 8, C, None) == ALIGN
    assert q(A, 4, 64, 64, 2, 448.0, 0, B, C, None) == UNSUP      # qtype
    assert q(A, 4, 64, 64, 0, 448.0, 64, B, C, None) == UNSUP     # group size
    assert q(A, 4, 192, 192, 0, 448.0, 128, B, C, None) == SHAPE  # cols % 128 in group mode
    for bad in (0.0, -1.0, 449.0, 21.0, float("inf"), float("nan")):
        assert q(A, 4, 64, 64, 0, bad, 0, B, C, None) == QMAX, bad
    assert q(A, 4, 64, 64, 1, 127.5, 0, B, C, None) == QMAX
    assert q(A, 4, 64, 64, 1, 128.0, 0, B, C, None) == QMAX
    assert q(A, 4, 64, 64, 0, 448.0, 0, A + 64, C, None) == ALIAS  # codes over x
    assert q(A, 4, 64, 64, 0, 448.0, 0, B, B + 128, None) == ALIAS  # scales over codes


@no_gpu_only
def test_weight_quantize_validation(L):
    w = L.tfq_quantize_weight_per_channel
    assert w(A, 256, 256, 0, 448.0, 64, B, C, None) == UNSUP
    assert w(A, 200, 256, 0, 448.0, 128, B, C, None) == SHAPE
    assert w(A, 256, 200, 0, 448.0, 128, B, C, None) == SHAPE
    assert w(None, 256, 256, 0, 448.0, 128, B, C, None) == NULL


@no_gpu_only
def test_gemm_validation(L):
    f = L.tfq_scaled_mm_fp8
    assert f(A, B, C, D, 64, 64, 64, 0, None, 0, None, None) == NULL
    assert f(None, B, C, D, 64, 64, 64, 0, None, 0, E, None) == NULL
    assert f(A, B, C, D, 64, 60, 64, 0, None, 0, E, None) == SHAPE   # n % 8
    assert f(A, B, C, D, 64, 64, 40, 0, None, 0, E, None) == SHAPE   # k % 16
    assert f(A, B, C, D, 0, 64, 64, 0, None, 0, E, None) == SHAPE
    assert f(A, B, C, D, 64, 64, 64, 64, None, 0, E, None) == UNSUP  # scale_block
    assert f(A, B, C, D, 64, 64, 192, 128, None, 0, E, None) == SHAPE
    assert f(A, B, C, D, 64, 128, 131072 + 128, 128, None, 0, E, None) == SHAPE  # block-mode k bound
    assert f(A, B, C, D, 64, 64, 64, 0, None, 5, E, None) == UNSUP  # epilogue
    assert f(A + 4, B, C, D, 64, 64, 64, 0, None, 0, E, None) == ALIGN
    # the bias is fetched with 16-byte loads: a 2-byte-aligned slice is refused
    assert f(A, B, C, D, 64, 64, 64, 0, F + 2, 0, E, None) == ALIGN
    assert f(A, B, C, D, 64, 128, 128, 128, F + 8, 0, E, None) == ALIGN
    assert f(A, B, C, D, 64, 64, 64, 0, F + 16, 0, E, None) in (DEV, HIP)
    assert f(A, B, C, D, 64, 64, 64, 0, None, 0, A + 16, None) == ALIAS
    i = L.tfq_scaled_mm_int8
    assert i(A, B, C, D, 64, 64, 64, None, 0, None, None, None) == NULL
    assert i(A, B, C, D, 64, 64, 131072, None, 0, E, None, None) == SHAPE  # INT32 bound
    assert i(A, B, C, D, 64, 64, 64, None, 0, E, E + 64, None) == ALIAS    # y over acc
    assert i(A, B, C, D, 64, 64, 64, F + 2, 0, E, None, None) == ALIGN     # bias alignment


@no_gpu_only
def test_mx_validation(L):
    q = L.tfq_quantize_mx
    assert q(None, 4, 128, 128, B, C, None) == NULL
    assert q(A, 4, 128, 128, B, None, None) == NULL
    assert q(A, 0, 128, 128, B, C, None) == SHAPE
    assert q(A, 4, 96, 96, B, C, None) == SHAPE           # cols % 128
    assert q(A, 4, 128, 64, B, C, None) == SHAPE          # ld < cols
    assert q(A, 1 << 24, 4096, 4096, B, C, None) == SHAPE  # scale words past 2^30 bytes
    assert q(A, 4, 128, 132, B, C, None) == ALIGN         # ld % 8
    assert q(A + 2, 4, 128, 128, B, C, None) == ALIGN
    assert q(A, 4, 128, 128, B + 8, C, None) == ALIGN
    assert q(A, 4, 128, 128, B, C + 2, None) == ALIGN     # scale words: 4 bytes
    assert q(A, 4, 128, 128, A + 64, C, None) == ALIAS    # codes over x
    assert q(A, 4, 128, 128, B, B + 508, None) == ALIAS   # scales over codes
    g = L.tfq_scaled_mm_mxfp8
    assert g(A, B, C, D, 64, 64, 128, None, 0, None, None) == NULL
    assert g(A, None, C, D, 64, 64, 128, None, 0, E, None) == NULL
    assert g(A, B, C, D, 64, 64, 128, None, 2, E, None) == UNSUP   # epilogue
    assert g(A, B, C, D, 64, 64, 96, None, 0, E, None) == SHAPE    # k % 128
    assert g(A, B, C, D, 64, 60, 128, None, 0, E, None) == SHAPE   # n % 8
    assert g(A, B, C, D, 0, 64, 128, None, 0, E, None) == SHAPE
    assert g(A, B, C, D, 64, 64, (1 << 22) + 128, None, 0, E, None) == SHAPE
    assert g(A, B, C, D, 1 << 20, 64, 1 << 16, None, 0, E, None) == SHAPE  # a_scale words
    assert g(A, B + 2, C, D, 64, 64, 128, None, 0, E, None) == ALIGN  # scale words: 4 bytes
    assert g(A + 4, B, C, D, 64, 64, 128, None, 0, E, None) == ALIGN
    assert g(A, B, C, D, 64, 64, 128, None, 0, E + 8, None) == ALIGN
    assert g(A, B, C, D, 64, 64, 128, None, 0, B + 16, None) == ALIAS  # y over a_scale
    q6 = L.tfq_quantize_mxfp6
    assert q6(A, 4, 128, 128, 0, B, C, None) == DEV
    assert q6(A, 4, 128, 128, 2, B, C, None) == UNSUP           # format
    assert q6(A, 4, 160, 160, 1, B, C, None) == SHAPE           # cols % 128
    assert q6(A, 4, 128, 128, 0, B, B + 380, None) == ALIAS     # scales over the 384 code bytes
    assert q6(A, 4, 128, 128, 0, B, B + 384, None) == DEV
    g6 = L.tfq_scaled_mm_mxfp6
    assert g6(A, B, C, D, 64, 64, 128, 1, None, 0, E, None) == DEV
    assert g6(A, B, C, D, 64, 64, 128, 3, None, 0, E, None) == UNSUP
    assert g6(A, B, C, D, 64, 64, 192, 0, None, 0, E, None) == SHAPE
    assert g6(A, B, C, D, 64, 64, 128, 0, None, 0, A + 64 * 96, None) == DEV   # after a_q
    assert g6(A, B, C, D, 64, 64, 128, 0, None, 0, A + 64 * 80, None) == ALIAS
    q4 = L.tfq_quantize_mxfp4
    assert q4(A, 4, 128, 128, B, C, None) == DEV
    assert q4(A, 4, 96, 96, B, C, None) == SHAPE           # cols % 128
    assert q4(A, 4, 128, 128, B + 4, C, None) == ALIGN
    assert q4(A, 4, 128, 128, B, B + 252, None) == ALIAS   # scales over the 256 code bytes
    assert q4(A, 4, 128, 128, B, B + 256, None) == DEV
    g4 = L.tfq_scaled_mm_mxfp4
    assert g4(A, B, C, D, 64, 64, 128, None, 0, E, None) == DEV
    assert g4(A, B, C, D, 64, 64, 192, None, 0, E, None) == SHAPE  # k % 128
    assert g4(A, B, C, D, 64, 64, 128, None, 0, A + 64 * 64, None) == DEV   # after a_q's 64*64 bytes
    assert g4(A, B, C, D, 64, 64, 128, None, 0, A + 64 * 48, None) == ALIAS


@no_gpu_only
def test_moe_validation(L):
    q = L.tfq_quantize_rows_gather
    assert q(A, 10, 64, 64, None, 4, 0, 448.0, 0, B, C, None) == NULL
    assert q(A, 0, 64, 64, D, 4, 0, 448.0, 0, B, C, None) == SHAPE     # src_rows
    assert q(A, 10, 64, 64, D, 0, 0, 448.0, 0, B, C, None) == SHAPE     # rows
    assert q(A, 10, 60, 64, D, 4, 0, 448.0, 0, B, C, None) == SHAPE     # cols % 16
    assert q(A, 10, 64, 64, D + 2, 4, 0, 448.0, 0, B, C, None) == ALIGN  # index alignment
    assert q(A, 10, 64, 64, D, 4, 0, 449.0, 0, B, C, None) == QMAX
    assert q(A, 10, 64, 64, B + 64, 4, 0, 448.0, 0, B, C, None) == ALIAS  # index over codes
    assert q(A, 10, 64, 64, D, 4, 0, 448.0, 0, A + 640, C, None) == ALIAS  # codes over x row 5
    g = L.tfq_grouped_scaled_mm_fp8
    assert g(A, B, C, D, None, 4, 64, 64, 64, None, 0, E, None) == NULL
    assert g(A, B, C, D, F, 0, 64, 64, 64, None, 0, E, None) == SHAPE    # groups
    assert g(A, B, C, D, F, 257, 64, 64, 64, None, 0, E, None) == SHAPE
    assert g(A, B, C, D, F, 4, 64, 60, 64, None, 0, E, None) == SHAPE    # n % 8
    assert g(A, B, C, D, F, 4, 64, 64, 40, None, 0, E, None) == SHAPE    # k % 16
    assert g(A, B, C, D, F, 4, 64, 64, 64, None, 3, E, None) == UNSUP    # epilogue
    assert g(A, B, C, D, F + 2, 4, 64, 64, 64, None, 0, E, None) == ALIGN
    assert g(A, B, C, D, F, 4, 64, 64, 64, None, 0, E + 8, None) == ALIGN
    assert g(A, B, C, D, F, 4, 64, 64, 64, None, 0, F, None) == ALIAS    # y over offsets
    assert g(A, B, C, D, F, 4, 64, 64, 64, None, 0, C + 3 * 64 * 64, None) == ALIAS  # y over b_q[3]


@no_gpu_only
def test_kv_cache_validation(L):
    st = L.tfq_kv_cache_store
    #         kv  T  H  D    ld   slot S   qmax   cache scale
    assert st(A, 4, 2, 128, 256, B, 10, 448.0, C, D, None) == DEV
    assert st(None, 4, 2, 128, 256, B, 10, 448.0, C, D, None) == NULL
    assert st(A, 4, 2, 128, 256, None, 10, 448.0, C, D, None) == NULL
    assert st(A, 4, 2, 120, 240, B, 10, 448.0, C, D, None) == DEV      # head_dim 120 is fine
    assert st(A, 4, 2, 100, 200, B, 10, 448.0, C, D, None) == SHAPE    # head_dim % 8
    assert st(A, 4, 2, 520, 1040, B, 10, 448.0, C, D, None) == SHAPE   # head_dim > 512
    assert st(A, 4, 2, 128, 200, B, 10, 448.0, C, D, None) == SHAPE    # ld < heads * head_dim
    assert st(A, 4, 2, 128, 260, B, 10, 448.0, C, D, None) == ALIGN    # ld % 8
    assert st(A, 1 << 30, 1, 8, 1 << 40, B, 10, 448.0, C, D, None) == SHAPE  # kv span > 2^61 bytes
    assert st(A, 4, 2, 128, 256, B, 10, 448.0, C + 8, D, None) == ALIGN
    assert st(A, 4, 2, 128, 256, B + 2, 10, 448.0, C, D, None) == ALIGN
    assert st(A, 4, 2, 128, 256, B, 10, 500.0, C, D, None) == QMAX
    assert st(A, 4, 2, 128, 256, B, 10, 448.0, C, C + 2048, None) == ALIAS  # scales inside cache
    assert st(A, 4, 2, 128, 256, B, 10, 448.0, A + 512, D, None) == ALIAS   # cache over kv
    ld = L.tfq_kv_cache_load
    #         cache scale S  H  D   idx n  dtype out
    assert ld(C, D, 10, 2, 128, B, 4, 0, E, None) == DEV
    assert ld(C, D, 10, 2, 128, B, 4, 3, E, None) == UNSUP     # dtype
    assert ld(C, D, 10, 2, 128, None, 4, 0, E, None) == NULL
    assert ld(C, D, 10, 2, 96, B, 4, 0, E + 8, None) == ALIGN
    assert ld(C, D, 10, 2, 128, B, 0, 0, E, None) == SHAPE
    assert ld(C, D, 10, 2, 128, B, 4, 2, C + 1024, None) == ALIAS  # out over the cache


def test_autotune_switch_and_empty_cache(L):
    assert L.tfq_set_autotune(2) == UNSUP and L.tfq_set_autotune(-1) == UNSUP
    assert L.tfq_set_autotune(1) == OK and L.tfq_set_autotune(0) == OK
    L.tfq_autotune_clear()
    assert L.tfq_autotune_lookup(0, 4096, 4096, 4096, 0, 0, None, None) == 0
    assert L.tfq_autotune_lookup(9, 4096, 4096, 4096, 0, 0, None, None) == 0  # unknown kind


@no_gpu_only
def test_fused_validation(L):
    ws = L.tfq_quant_linear_workspace_bytes
    need = ws(100, 256, 0, 0)
    assert need == 25600 + 400  # codes (256-aligned) + scales
    assert ws(100, 256, 0, 128) == 25600 + 100 * 2 * 4
    assert ws(100, 256, 1, 128) == 0 and ws(0, 256, 0, 0) == 0 and ws(100, 250, 0, 0) == 0
    fu = L.tfq_quant_linear_fused
    assert fu(A, 100, 256, 256, B, C, 64, 0, 448.0, 0, None, 0, D, E, need - 1, None) == WS
    assert fu(A, 100, 256, 256, B, C, 64, 0, 448.0, 0, None, 0, D, E + 16, need, None) == ALIGN
    assert fu(A, 100, 256, 256, B, C, 64, 0, 449.0, 0, None, 0, D, E, need, None) == QMAX
    assert fu(A, 100, 256, 256, B, C, 64, 1, 127.0, 128, None, 0, D, E, need, None) == UNSUP
    assert fu(A, 100, 256, 256, B, C, 64, 0, 448.0, 0, None, 0, D, A, need, None) == ALIAS
    assert fu(A, 100, 256, 256, B, C, 64, 0, 448.0, 0, None, 0, A + 256, E, need, None) == ALIAS
    # K far past every limit is refused before the workspace size (m * k) is formed
    big = 1 << 60
    assert fu(A, 100, big, big, B, C, 64, 0, 448.0, 0, None, 0, D, E, need, None) == SHAPE
    assert ws(100, big, 0, 0) == 0


@no_gpu_only
def test_valid_call_without_gpu_reports_device(L):
    # everything valid: the only thing missing is a gfx950
    assert L.tfq_quantize_rows(A, 4, 64, 64, 0, 448.0, 0, B, C, None) == DEV
    assert L.tfq_scaled_mm_fp8(A, B, C, D, 64, 64, 64, 0, None, 0, E, None) == DEV
    assert L.tfq_e4m3fn_encode_f32(A, B, 64, None) == DEV
    assert L.tfq_quantize_mx(A, 4, 128, 128, B, C, None) == DEV
    assert L.tfq_scaled_mm_mxfp8(A, B, C, D, 64, 64, 128, None, 0, E, None) == DEV
    assert L.tfq_quantize_rows_gather(A, 10, 64, 64, D, 4, 0, 448.0, 0, B, C, None) == DEV
    # codes placed right after a source matrix that has fewer rows than the
    # output: adjacent, not overlapping
    x_end = A + 97 * 1024 * 2
    assert L.tfq_quantize_rows_gather(A, 97, 1024, 1024, D, 183, 0, 448.0, 0, x_end,
                                      x_end + 183 * 1024, None) == DEV
    assert L.tfq_grouped_scaled_mm_fp8(A, B, C, D, F, 4, 64, 64, 64, None, 0, E, None) == DEV


def test_python_binding_names_match_abi():
    import int8_w8a8_quantized_amd as P

    for n in declared_functions():
        if n in ("tfq_status_string", "tfq_last_hip_error"):
            continue
        assert callable(getattr(P, n)), n


def test_autotune_set_validation(L):
    s = L.tfq_autotune_set
    assert s(9, 4096, 4096, 4096, 0, 0, 2, 4) == UNSUP       # unknown kind
    assert s(0, 4096, 4096, 4096, 7, 0, 2, 4) == UNSUP       # unknown epilogue
    assert s(0, 4096, 4096, 4096, 0, 0, 3, 4) == UNSUP       # no such kernel
    assert s(0, 4096, 4096, 4096, 0, 0, 0, 3) == UNSUP       # band not a candidate
    assert s(0, 4096, 8192, 4096, 0, 0, 1, 4) == UNSUP       # two-per-CU only below 512 tiles
    assert s(2, 4096, 4096, 4096, 0, 0, 1, 4) == UNSUP       # block-scaled: kernel 0 only
    assert s(3, 4096, 4096, 4096, 0, 0, 2, 4) == UNSUP       # MXFP8: no 192-column tiles
    assert s(4, 4096, 4096, 4096, 0, 2, 2, 4) == UNSUP       # grouped: no 192-column tiles
    assert s(4, 4096, 4096, 4096, 0, 0, 0, 4) == SHAPE       # grouped needs 1..256 groups
    assert s(0, 0, 4096, 4096, 0, 0, 0, 4) == SHAPE
    if not HAS_GPU_NODE:
        # a valid candidate: only the missing device stops it
        assert s(1, 4096, 4096, 4096, 0, 0, 1, 4) == DEV
        assert s(0, 4096, 4096, 4096, 1, 0, 0, 8) == DEV
        assert s(0, 4096, 4096, 4096, 0, 0, 2, 2) == DEV


@no_gpu_only
def test_noalloc_fused_validation(L):
    f = L.tfq_quant_linear_fused_noalloc
    # (x, m, k, ld_x, w_q, w_scale, n, qtype, act_qmax, scale_block, bias, epi, y, stream)
    assert f(None, 100, 256, 256, B, C, 64, 0, 448.0, 0, None, 0, D, None) == NULL
    assert f(A, 100, 256, 256, B, C, 64, 5, 448.0, 0, None, 0, D, None) == UNSUP
    assert f(A, 100, 250, 256, B, C, 64, 0, 448.0, 0, None, 0, D, None) == SHAPE
    assert f(A, 100, 256, 256, B, C, 64, 0, 21.0, 0, None, 0, D, None) == QMAX
    assert f(A, 100, 256, 256, B, C, 64, 0, 448.0, 0, F + 2, 0, D, None) == ALIGN
    assert f(A, 100, 256, 256, B, C, 64, 0, 448.0, 0, None, 0, A + 64, None) == ALIAS
    # beyond the 64 MiB device scratch: refused before any HIP call
    assert f(A, 16384, 5120, 5120, B, C, 256, 0, 448.0, 0, None, 0, D, None) == WS
    # valid: only the missing device stops it
    assert f(A, 100, 256, 256, B, C, 64, 0, 448.0, 0, None, 0, D, None) == DEV
