// extern "C" entry points of libtfq: argument validation on the host (before
// any HIP call), a once-per-device gfx950 check, then kernel launches on the
// caller's stream.  The method each entry point implements is cited in
// include/tfq.h beside its declaration.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "tfq.h"
#include "tfq_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxDim = (int64_t)1 << 30;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) { return Range{(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes}; }

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

// qmax must be a finite positive value on the code grid: an E4M3FN value in
// (0, 448] (OCP OFP8: (1 + m/8) 2^(e-7) for e >= 1, m/8 2^-6 for e == 0), or
// an integer in [1, 127] for INT8.
bool qmax_ok(int32_t qtype, float qmax)
{
    if (!(qmax > 0.0f) || !isfinite(qmax)) return false;
    if (qtype == TFQ_QTYPE_INT8) return qmax <= 127.0f && qmax == floorf(qmax);
    if (qmax > 448.0f) return false;
    for (int e = 0; e <= 15; ++e) {
        for (int m = 0; m <= 7; ++m) {
            if (e == 15 && m == 7) continue;
            const double v = e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
            if ((double)qmax == v) return true;
        }
    }
    return false;
}

bool qtype_ok(int32_t q) { return q == TFQ_QTYPE_E4M3FN || q == TFQ_QTYPE_INT8; }
bool epi_ok(int32_t e) { return e == TFQ_EPI_NONE || e == TFQ_EPI_GELU_TANH; }

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// ---- device check: the current device must be a gfx950 ----
std::mutex g_dev_mu;
int g_dev_state[256];  // 0 unknown, 1 gfx950, -1 other

tfq_status check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) {
        (void)hipGetLastError();
        return TFQ_ERR_UNSUPPORTED_DEVICE;
    }
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_state[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return TFQ_ERR_UNSUPPORTED_DEVICE;
        }
        g_dev_state[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    return g_dev_state[dev] == 1 ? TFQ_OK : TFQ_ERR_UNSUPPORTED_DEVICE;
}

tfq_status hip_status(hipError_t e)
{
    if (e == hipSuccess) return TFQ_OK;
    g_last_hip_error = (int)e;
    return TFQ_ERR_HIP;
}

// ---- validation (pure host code, no HIP calls) ----
tfq_status validate_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld, int32_t qtype,
                             float qmax, int32_t group, const void* q, const float* s)
{
    if (!x || !q || !s) return TFQ_ERR_NULL_POINTER;
    if (!qtype_ok(qtype)) return TFQ_ERR_UNSUPPORTED;
    if (group != 0 && group != 128) return TFQ_ERR_UNSUPPORTED;
    if (rows < 1 || rows > kMaxDim || cols < 16 || cols > kMaxDim || cols % 16 != 0)
        return TFQ_ERR_BAD_SHAPE;
    if (ld < cols || ld > kMaxDim) return TFQ_ERR_BAD_SHAPE;
    if (group == 128 && cols % 128 != 0) return TFQ_ERR_BAD_SHAPE;
    if (ld % 8 != 0 || !aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4))
        return TFQ_ERR_MISALIGNED;
    if (!qmax_ok(qtype, qmax)) return TFQ_ERR_BAD_QMAX;
    const int64_t ng = group == 128 ? cols / 128 : 1;
    const Range rx = range_of(x, ((rows - 1) * ld + cols) * 2);
    const Range rq = range_of(q, rows * cols);
    const Range rs = range_of(s, rows * ng * 4);
    if (overlap(rx, rq) || overlap(rx, rs) || overlap(rq, rs)) return TFQ_ERR_ALIAS;
    return TFQ_OK;
}

tfq_status validate_gemm(const void* a, const float* sa, const void* b, const float* sb, int64_t m,
                         int64_t n, int64_t k, int32_t qtype, int32_t block, const void* bias,
                         int32_t epi, const void* y, const void* acc, int64_t kmax)
{
    if (!a || !sa || !b || !sb) return TFQ_ERR_NULL_POINTER;
    if (!y && !acc) return TFQ_ERR_NULL_POINTER;
    if (!epi_ok(epi) || (block != 0 && block != 128)) return TFQ_ERR_UNSUPPORTED;
    if (block == 128 && qtype != TFQ_QTYPE_E4M3FN) return TFQ_ERR_UNSUPPORTED;
    if (m < 1 || m > kMaxDim || n < 8 || n > kMaxDim || n % 8 != 0 || k < 16 || k > kmax ||
        k % 16 != 0)
        return TFQ_ERR_BAD_SHAPE;
    // block mode keeps one row of weight-block scales (k/128 floats) in 4 KB of LDS
    if (block == 128 && (k % 128 != 0 || n % 128 != 0 || k > 131072)) return TFQ_ERR_BAD_SHAPE;
    const int64_t tiles = ((m + 255) / 256) * ((n + 255) / 256);
    if (tiles > INT32_MAX) return TFQ_ERR_BAD_SHAPE;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(sa, 4) || !aligned(sb, 4) ||
        (bias && !aligned(bias, 16)) || (y && !aligned(y, 16)) || (acc && !aligned(acc, 16)))
        return TFQ_ERR_MISALIGNED;
    const int64_t nsa = block == 128 ? m * (k / 128) : m;
    const int64_t nsb = block == 128 ? (n / 128) * (k / 128) : n;
    const Range ins[5] = {range_of(a, m * k), range_of(b, n * k), range_of(sa, nsa * 4),
                          range_of(sb, nsb * 4), range_of(bias, bias ? n * 2 : 0)};
    const Range ry = range_of(y, y ? m * n * 2 : 0);
    const Range racc = range_of(acc, acc ? m * n * 4 : 0);
    for (const Range& r : ins)
        if (overlap(r, ry) || overlap(r, racc)) return TFQ_ERR_ALIAS;
    if (overlap(ry, racc)) return TFQ_ERR_ALIAS;
    return TFQ_OK;
}

// MXFP8 scale words [k/128, rows]: word offsets must fit the GEMM's 32-bit
// buffer offsets
bool mx_scales_fit(int64_t rows, int64_t k) { return rows * (k / 32) <= ((int64_t)1 << 30); }

size_t workspace_bytes(int64_t m, int64_t k, int32_t block)
{
    const int64_t ns = block == 128 ? m * (k / 128) : m;
    return align256((size_t)(m * k)) + (size_t)ns * 4;
}

}  // namespace

extern "C" {

const char* tfq_status_string(tfq_status s)
{
    switch (s) {
    case TFQ_OK: return "ok";
    case TFQ_ERR_NULL_POINTER: return "null pointer";
    case TFQ_ERR_BAD_SHAPE: return "bad shape";
    case TFQ_ERR_MISALIGNED: return "misaligned pointer or leading dimension";
    case TFQ_ERR_BAD_QMAX: return "qmax not finite, not positive, too large or not on the code grid";
    case TFQ_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case TFQ_ERR_ALIAS: return "output overlaps an input or another output";
    case TFQ_ERR_UNSUPPORTED: return "unsupported option";
    case TFQ_ERR_UNSUPPORTED_DEVICE: return "no HIP device or the current device is not gfx950";
    case TFQ_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

int tfq_last_hip_error(void) { return g_last_hip_error; }

int tfq_abi_version(void) { return TFQ_ABI_VERSION; }

tfq_status tfq_quantize_rows(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                             int32_t qtype, float qmax, int32_t group_cols, void* q_out,
                             float* scale_out, void* stream)
{
    tfq_status st =
        validate_quantize(x_bf16, rows, cols, ld_x, qtype, qmax, group_cols, q_out, scale_out);
    if (st != TFQ_OK) return st;
    if ((st = check_device()) != TFQ_OK) return st;
    return hip_status(tfq::launch_quantize_rows((const uint16_t*)x_bf16, rows, cols, ld_x, qtype,
                                                qmax, group_cols, (uint8_t*)q_out, scale_out,
                                                (hipStream_t)stream));
}

tfq_status tfq_quantize_rows_gather(const void* x_bf16, int64_t src_rows, int64_t cols,
                                    int64_t ld_x, const int32_t* row_index, int64_t rows,
                                    int32_t qtype, float qmax, int32_t group_cols, void* q_out,
                                    float* scale_out, void* stream)
{
    if (!x_bf16 || !row_index || !q_out || !scale_out) return TFQ_ERR_NULL_POINTER;
    if (!qtype_ok(qtype) || (group_cols != 0 && group_cols != 128)) return TFQ_ERR_UNSUPPORTED;
    if (rows < 1 || rows > kMaxDim || src_rows < 1 || src_rows > kMaxDim || cols < 16 ||
        cols > kMaxDim || cols % 16 != 0 || ld_x < cols || ld_x > kMaxDim ||
        (group_cols == 128 && cols % 128 != 0))
        return TFQ_ERR_BAD_SHAPE;
    if (ld_x % 8 != 0 || !aligned(x_bf16, 16) || !aligned(q_out, 16) || !aligned(scale_out, 4) ||
        !aligned(row_index, 4))
        return TFQ_ERR_MISALIGNED;
    if (!qmax_ok(qtype, qmax)) return TFQ_ERR_BAD_QMAX;
    const int64_t ng = group_cols == 128 ? cols / 128 : 1;
    const Range rx = range_of(x_bf16, ((src_rows - 1) * ld_x + cols) * 2);
    const Range ri = range_of(row_index, rows * 4);
    const Range rq = range_of(q_out, rows * cols), rs = range_of(scale_out, rows * ng * 4);
    if (overlap(rq, rs) || overlap(rq, rx) || overlap(rq, ri) || overlap(rs, rx) || overlap(rs, ri))
        return TFQ_ERR_ALIAS;
    tfq_status st = check_device();
    if (st != TFQ_OK) return st;
    return hip_status(tfq::launch_quantize_rows((const uint16_t*)x_bf16, rows, cols, ld_x, qtype,
                                                qmax, group_cols, (uint8_t*)q_out, scale_out,
                                                (hipStream_t)stream, row_index, src_rows));
}

tfq_status tfq_quantize_weight_per_channel(const void* w_bf16, int64_t n, int64_t k, int32_t qtype,
                                           float qmax, int32_t block, void* q_out,
                                           float* scale_out, void* stream)
{
    if (block != 0 && block != 128) return !w_bf16 || !q_out || !scale_out ? TFQ_ERR_NULL_POINTER
                                                                           : TFQ_ERR_UNSUPPORTED;
    tfq_status st = validate_quantize(w_bf16, n, k, k, qtype, qmax, 0, q_out, scale_out);
    if (st != TFQ_OK) return st;
    if (block == 128) {
        if (n % 128 != 0 || k % 128 != 0) return TFQ_ERR_BAD_SHAPE;
        const Range rw = range_of(w_bf16, n * k * 2), rq = range_of(q_out, n * k);
        const Range rs = range_of(scale_out, (n / 128) * (k / 128) * 4);
        if (overlap(rw, rs) || overlap(rq, rs)) return TFQ_ERR_ALIAS;
    }
    if ((st = check_device()) != TFQ_OK) return st;
    if (block == 128)
        return hip_status(tfq::launch_quantize_blocks((const uint16_t*)w_bf16, n, k, qtype, qmax,
                                                      (uint8_t*)q_out, scale_out,
                                                      (hipStream_t)stream));
    return hip_status(tfq::launch_quantize_rows((const uint16_t*)w_bf16, n, k, k, qtype, qmax, 0,
                                                (uint8_t*)q_out, scale_out, (hipStream_t)stream));
}

tfq_status tfq_scaled_mm_fp8(const uint8_t* a_q, const float* a_scale, const uint8_t* b_q,
                             const float* b_scale, int64_t m, int64_t n, int64_t k,
                             int32_t scale_block, const void* bias_bf16, int32_t epi, void* y_bf16,
                             void* stream)
{
    if (!y_bf16) return TFQ_ERR_NULL_POINTER;
    tfq_status st = validate_gemm(a_q, a_scale, b_q, b_scale, m, n, k, TFQ_QTYPE_E4M3FN,
                                  scale_block, bias_bf16, epi, y_bf16, nullptr, (int64_t)1 << 22);
    if (st != TFQ_OK) return st;
    if ((st = check_device()) != TFQ_OK) return st;
    tfq::GemmArgs g{a_q, b_q, a_scale, b_scale, (const uint16_t*)bias_bf16, (uint16_t*)y_bf16,
                    nullptr, m, n, k, tfq::kE4M3FN, scale_block, epi};
    return hip_status(tfq::launch_scaled_gemm(g, (hipStream_t)stream));
}

tfq_status tfq_scaled_mm_int8(const int8_t* a_q, const float* a_scale, const int8_t* b_q,
                              const float* b_scale, int64_t m, int64_t n, int64_t k,
                              const void* bias_bf16, int32_t epi, void* y_bf16, int32_t* acc_i32,
                              void* stream)
{
    tfq_status st = validate_gemm(a_q, a_scale, b_q, b_scale, m, n, k, TFQ_QTYPE_INT8, 0,
                                  bias_bf16, epi, y_bf16, acc_i32, 131071);
    if (st != TFQ_OK) return st;
    if ((st = check_device()) != TFQ_OK) return st;
    tfq::GemmArgs g{(const uint8_t*)a_q, (const uint8_t*)b_q, a_scale, b_scale,
                    (const uint16_t*)bias_bf16, (uint16_t*)y_bf16, acc_i32, m, n, k, tfq::kInt8, 0,
                    epi};
    return hip_status(tfq::launch_scaled_gemm(g, (hipStream_t)stream));
}

tfq_status tfq_grouped_scaled_mm_fp8(const uint8_t* a_q, const float* a_scale, const uint8_t* b_q,
                                     const float* b_scale, const int32_t* group_offsets,
                                     int32_t groups, int64_t m, int64_t n, int64_t k,
                                     const void* bias_bf16, int32_t epi, void* y_bf16, void* stream)
{
    if (!a_q || !a_scale || !b_q || !b_scale || !group_offsets || !y_bf16)
        return TFQ_ERR_NULL_POINTER;
    if (!epi_ok(epi)) return TFQ_ERR_UNSUPPORTED;
    if (groups < 1 || groups > 256 || m < 1 || m > kMaxDim || n < 8 || n > kMaxDim || n % 8 != 0 ||
        k < 16 || k > ((int64_t)1 << 22) || k % 16 != 0)
        return TFQ_ERR_BAD_SHAPE;
    if (((m + 255) / 256 + groups) * ((n + 255) / 256) > INT32_MAX) return TFQ_ERR_BAD_SHAPE;
    if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(a_scale, 4) || !aligned(b_scale, 4) ||
        !aligned(group_offsets, 4) || (bias_bf16 && !aligned(bias_bf16, 16)) || !aligned(y_bf16, 16))
        return TFQ_ERR_MISALIGNED;
    const Range ry = range_of(y_bf16, m * n * 2);
    const Range ins[6] = {range_of(a_q, m * k), range_of(b_q, groups * n * k),
                          range_of(a_scale, m * 4), range_of(b_scale, groups * n * 4),
                          range_of(bias_bf16, bias_bf16 ? groups * n * 2 : 0),
                          range_of(group_offsets, (groups + 1) * 4)};
    for (const Range& r : ins)
        if (overlap(r, ry)) return TFQ_ERR_ALIAS;
    tfq_status st = check_device();
    if (st != TFQ_OK) return st;
    tfq::GemmArgs g{a_q, b_q, a_scale, b_scale, (const uint16_t*)bias_bf16, (uint16_t*)y_bf16,
                    nullptr, m, n, k, tfq::kE4M3FN, 0, epi, nullptr, nullptr, group_offsets,
                    groups};
    return hip_status(tfq::launch_scaled_gemm(g, (hipStream_t)stream));
}

size_t tfq_quant_linear_workspace_bytes(int64_t m, int64_t k, int32_t qtype, int32_t scale_block)
{
    if (!qtype_ok(qtype) || m < 1 || m > kMaxDim || k < 16 || k > kMaxDim || k % 16 != 0)
        return 0;
    if (scale_block != 0 && scale_block != 128) return 0;
    if (scale_block == 128 && (qtype != TFQ_QTYPE_E4M3FN || k % 128 != 0)) return 0;
    return workspace_bytes(m, k, scale_block);
}

tfq_status tfq_quant_linear_fused(const void* x_bf16, int64_t m, int64_t k, int64_t ld_x,
                                  const void* w_q, const float* w_scale, int64_t n, int32_t qtype,
                                  float act_qmax, int32_t scale_block, const void* bias_bf16,
                                  int32_t epi, void* y_bf16, void* workspace,
                                  size_t workspace_bytes_given, void* stream)
{
    if (!x_bf16 || !w_q || !w_scale || !y_bf16 || !workspace) return TFQ_ERR_NULL_POINTER;
    if (!qtype_ok(qtype) || !epi_ok(epi) || (scale_block != 0 && scale_block != 128) ||
        (scale_block == 128 && qtype != TFQ_QTYPE_E4M3FN))
        return TFQ_ERR_UNSUPPORTED;
    // (k bounded before workspace_bytes multiplies it by m)
    if (m < 1 || m > kMaxDim || k < 16 || k > kMaxDim || k % 16 != 0 || ld_x < k ||
        ld_x > kMaxDim)
        return TFQ_ERR_BAD_SHAPE;
    if (scale_block == 128 && k % 128 != 0) return TFQ_ERR_BAD_SHAPE;
    if (!aligned(workspace, 256)) return TFQ_ERR_MISALIGNED;
    const size_t need = workspace_bytes(m, k, scale_block);
    if (workspace_bytes_given < need) return TFQ_ERR_WORKSPACE_TOO_SMALL;
    uint8_t* codes = (uint8_t*)workspace;
    float* scales = (float*)((uint8_t*)workspace + align256((size_t)(m * k)));
    tfq_status st = validate_quantize(x_bf16, m, k, ld_x, qtype, act_qmax, scale_block, codes,
                                      scales);
    if (st != TFQ_OK) return st;
    st = validate_gemm(codes, scales, w_q, w_scale, m, n, k, qtype, scale_block, bias_bf16, epi,
                       y_bf16, nullptr, qtype == TFQ_QTYPE_INT8 ? 131071 : ((int64_t)1 << 22));
    if (st != TFQ_OK) return st;
    // the workspace must not overlap the caller's inputs or output
    const Range rws = range_of(workspace, (int64_t)need);
    const int64_t nsb = scale_block == 128 ? (n / 128) * (k / 128) : n;
    if (overlap(rws, range_of(x_bf16, ((m - 1) * ld_x + k) * 2)) ||
        overlap(rws, range_of(w_q, n * k)) || overlap(rws, range_of(w_scale, nsb * 4)) ||
        overlap(rws, range_of(y_bf16, m * n * 2)) ||
        (bias_bf16 && overlap(rws, range_of(bias_bf16, n * 2))) ||
        overlap(range_of(y_bf16, m * n * 2), range_of(x_bf16, ((m - 1) * ld_x + k) * 2)))
        return TFQ_ERR_ALIAS;
    if ((st = check_device()) != TFQ_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    st = hip_status(tfq::launch_quantize_rows((const uint16_t*)x_bf16, m, k, ld_x, qtype, act_qmax,
                                              scale_block, codes, scales, s));
    if (st != TFQ_OK) return st;
    tfq::GemmArgs g{codes, (const uint8_t*)w_q, scales, w_scale, (const uint16_t*)bias_bf16,
                    (uint16_t*)y_bf16, nullptr, m, n, k, qtype, scale_block, epi};
    return hip_status(tfq::launch_scaled_gemm(g, s));
}

tfq_status tfq_quant_linear_fused_noalloc(const void* x_bf16, int64_t m, int64_t k, int64_t ld_x,
                                          const void* w_q, const float* w_scale, int64_t n,
                                          int32_t qtype, float act_qmax, int32_t scale_block,
                                          const void* bias_bf16, int32_t epi, void* y_bf16,
                                          void* stream)
{
    static_assert(TFQ_NOALLOC_WORKSPACE_BYTES == tfq::kNoAllocScratchBytes, "one scratch size");
    if (!x_bf16 || !w_q || !w_scale || !y_bf16) return TFQ_ERR_NULL_POINTER;
    if (!qtype_ok(qtype) || !epi_ok(epi) || (scale_block != 0 && scale_block != 128) ||
        (scale_block == 128 && qtype != TFQ_QTYPE_E4M3FN))
        return TFQ_ERR_UNSUPPORTED;
    if (m < 1 || m > kMaxDim || k < 16 || k > kMaxDim || k % 16 != 0 || ld_x < k ||
        ld_x > kMaxDim)
        return TFQ_ERR_BAD_SHAPE;
    if (scale_block == 128 && k % 128 != 0) return TFQ_ERR_BAD_SHAPE;
    const size_t need = workspace_bytes(m, k, scale_block);
    if (need > tfq::kNoAllocScratchBytes) return TFQ_ERR_WORKSPACE_TOO_SMALL;
    // host-side checks of the caller's buffers before any HIP call (the
    // scratch is the library's own: placeholders stand in for it here)
    const uintptr_t fake = (uintptr_t)1 << 62;  // far from any caller buffer; never used
    tfq_status st = validate_quantize(x_bf16, m, k, ld_x, qtype, act_qmax, scale_block,
                                      (void*)fake, (float*)(fake + align256((size_t)(m * k))));
    if (st != TFQ_OK) return st;
    st = validate_gemm((void*)fake, (const float*)(fake + align256((size_t)(m * k))), w_q, w_scale, m,
                       n, k, qtype, scale_block, bias_bf16, epi, y_bf16, nullptr,
                       qtype == TFQ_QTYPE_INT8 ? 131071 : ((int64_t)1 << 22));
    if (st != TFQ_OK) return st;
    if (overlap(range_of(y_bf16, m * n * 2), range_of(x_bf16, ((m - 1) * ld_x + k) * 2)))
        return TFQ_ERR_ALIAS;
    if ((st = check_device()) != TFQ_OK) return st;
    void* ws = nullptr;
    if ((st = hip_status(tfq::noalloc_scratch(&ws))) != TFQ_OK) return st;
    uint8_t* codes = (uint8_t*)ws;
    float* scales = (float*)((uint8_t*)ws + align256((size_t)(m * k)));
    hipStream_t s = (hipStream_t)stream;
    st = hip_status(tfq::launch_quantize_rows((const uint16_t*)x_bf16, m, k, ld_x, qtype, act_qmax,
                                              scale_block, codes, scales, s));
    if (st != TFQ_OK) return st;
    tfq::GemmArgs g{codes, (const uint8_t*)w_q, scales, w_scale, (const uint16_t*)bias_bf16,
                    (uint16_t*)y_bf16, nullptr, m, n, k, qtype, scale_block, epi};
    return hip_status(tfq::launch_scaled_gemm_with(g, tfq::config_without_tuning(g), s));
}

tfq_status tfq_quantize_mx(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                           void* q_out, uint32_t* scale_out, void* stream)
{
    if (!x_bf16 || !q_out || !scale_out) return TFQ_ERR_NULL_POINTER;
    if (rows < 1 || rows > kMaxDim || cols < 128 || cols > kMaxDim || cols % 128 != 0 ||
        ld_x < cols || ld_x > kMaxDim || !mx_scales_fit(rows, cols))
        return TFQ_ERR_BAD_SHAPE;
    if (ld_x % 8 != 0 || !aligned(x_bf16, 16) || !aligned(q_out, 16) || !aligned(scale_out, 4))
        return TFQ_ERR_MISALIGNED;
    const Range rx = range_of(x_bf16, ((rows - 1) * ld_x + cols) * 2);
    const Range rq = range_of(q_out, rows * cols), rs = range_of(scale_out, rows * (cols / 32));
    if (overlap(rx, rq) || overlap(rx, rs) || overlap(rq, rs)) return TFQ_ERR_ALIAS;
    tfq_status st = check_device();
    if (st != TFQ_OK) return st;
    return hip_status(tfq::launch_quantize_mx((const uint16_t*)x_bf16, rows, cols, ld_x,
                                              (uint8_t*)q_out, scale_out, (hipStream_t)stream));
}

tfq_status tfq_quantize_mxfp4(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                              void* q_out, uint32_t* scale_out, void* stream)
{
    if (!x_bf16 || !q_out || !scale_out) return TFQ_ERR_NULL_POINTER;
    if (rows < 1 || rows > kMaxDim || cols < 128 || cols > kMaxDim || cols % 128 != 0 ||
        ld_x < cols || ld_x > kMaxDim || !mx_scales_fit(rows, cols))
        return TFQ_ERR_BAD_SHAPE;
    if (ld_x % 8 != 0 || !aligned(x_bf16, 16) || !aligned(q_out, 16) || !aligned(scale_out, 4))
        return TFQ_ERR_MISALIGNED;
    const Range rx = range_of(x_bf16, ((rows - 1) * ld_x + cols) * 2);
    const Range rq = range_of(q_out, rows * cols / 2), rs = range_of(scale_out, rows * (cols / 32));
    if (overlap(rx, rq) || overlap(rx, rs) || overlap(rq, rs)) return TFQ_ERR_ALIAS;
    tfq_status st = check_device();
    if (st != TFQ_OK) return st;
    return hip_status(tfq::launch_quantize_mx((const uint16_t*)x_bf16, rows, cols, ld_x,
                                              (uint8_t*)q_out, scale_out, (hipStream_t)stream, 4));
}

tfq_status tfq_scaled_mm_mxfp4(const uint8_t* a_q, const uint32_t* a_scale, const uint8_t* b_q,
                               const uint32_t* b_scale, int64_t m, int64_t n, int64_t k,
                               const void* bias_bf16, int32_t epi, void* y_bf16, void* stream)
{
    if (!a_q || !a_scale || !b_q || !b_scale || !y_bf16) return TFQ_ERR_NULL_POINTER;
    if (!epi_ok(epi)) return TFQ_ERR_UNSUPPORTED;
    if (m < 1 || m > kMaxDim || n < 8 || n > kMaxDim || n % 8 != 0 || k < 128 ||
        k > ((int64_t)1 << 23) || k % 128 != 0 || !mx_scales_fit(m, k) || !mx_scales_fit(n, k))
        return TFQ_ERR_BAD_SHAPE;
    if (((m + 255) / 256) * ((n + 255) / 256) > INT32_MAX) return TFQ_ERR_BAD_SHAPE;
    if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(a_scale, 4) || !aligned(b_scale, 4) ||
        (bias_bf16 && !aligned(bias_bf16, 16)) || !aligned(y_bf16, 16))
        return TFQ_ERR_MISALIGNED;
    const Range ry = range_of(y_bf16, m * n * 2);
    const Range ins[5] = {range_of(a_q, m * k / 2), range_of(b_q, n * k / 2),
                          range_of(a_scale, m * (k / 32)), range_of(b_scale, n * (k / 32)),
                          range_of(bias_bf16, bias_bf16 ? n * 2 : 0)};
    for (const Range& r : ins)
        if (overlap(r, ry)) return TFQ_ERR_ALIAS;
    tfq_status st = check_device();
    if (st != TFQ_OK) return st;
    tfq::GemmArgs g{a_q, b_q, nullptr, nullptr, (const uint16_t*)bias_bf16, (uint16_t*)y_bf16,
                    nullptr, m, n, k, tfq::kMxE2M1, 0, epi, a_scale, b_scale};
    return hip_status(tfq::launch_scaled_gemm(g, (hipStream_t)stream));
}

tfq_status tfq_quantize_mxfp6(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                              int32_t fmt, void* q_out, uint32_t* scale_out, void* stream)
{
    if (!x_bf16 || !q_out || !scale_out) return TFQ_ERR_NULL_POINTER;
    if (fmt != 0 && fmt != 1) return TFQ_ERR_UNSUPPORTED;
    if (rows < 1 || rows > kMaxDim || cols < 128 || cols > kMaxDim || cols % 128 != 0 ||
        ld_x < cols || ld_x > kMaxDim || !mx_scales_fit(rows, cols))
        return TFQ_ERR_BAD_SHAPE;
    if (ld_x % 8 != 0 || !aligned(x_bf16, 16) || !aligned(q_out, 16) || !aligned(scale_out, 4))
        return TFQ_ERR_MISALIGNED;
    const Range rx = range_of(x_bf16, ((rows - 1) * ld_x + cols) * 2);
    const Range rq = range_of(q_out, rows * (cols / 4 * 3)), rs = range_of(scale_out, rows * (cols / 32));
    if (overlap(rx, rq) || overlap(rx, rs) || overlap(rq, rs)) return TFQ_ERR_ALIAS;
    tfq_status st = check_device();
    if (st != TFQ_OK) return st;
    return hip_status(tfq::launch_quantize_mx((const uint16_t*)x_bf16, rows, cols, ld_x,
                                              (uint8_t*)q_out, scale_out, (hipStream_t)stream,
                                              fmt == 0 ? 62 : 63));
}

tfq_status tfq_scaled_mm_mxfp6(const uint8_t* a_q, const uint32_t* a_scale, const uint8_t* b_q,
                               const uint32_t* b_scale, int64_t m, int64_t n, int64_t k, int32_t fmt,
                               const void* bias_bf16, int32_t epi, void* y_bf16, void* stream)
{
    if (!a_q || !a_scale || !b_q || !b_scale || !y_bf16) return TFQ_ERR_NULL_POINTER;
    if (!epi_ok(epi) || (fmt != 0 && fmt != 1)) return TFQ_ERR_UNSUPPORTED;
    if (m < 1 || m > kMaxDim || n < 8 || n > kMaxDim || n % 8 != 0 || k < 128 ||
        k > ((int64_t)1 << 22) || k % 128 != 0 || !mx_scales_fit(m, k) || !mx_scales_fit(n, k))
        return TFQ_ERR_BAD_SHAPE;
    if (((m + 255) / 256) * ((n + 255) / 256) > INT32_MAX) return TFQ_ERR_BAD_SHAPE;
    if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(a_scale, 4) || !aligned(b_scale, 4) ||
        (bias_bf16 && !aligned(bias_bf16, 16)) || !aligned(y_bf16, 16))
        return TFQ_ERR_MISALIGNED;
    const Range ry = range_of(y_bf16, m * n * 2);
    const Range ins[5] = {range_of(a_q, m * (k / 4 * 3)), range_of(b_q, n * (k / 4 * 3)),
                          range_of(a_scale, m * (k / 32)), range_of(b_scale, n * (k / 32)),
                          range_of(bias_bf16, bias_bf16 ? n * 2 : 0)};
    for (const Range& r : ins)
        if (overlap(r, ry)) return TFQ_ERR_ALIAS;
    tfq_status st = check_device();
    if (st != TFQ_OK) return st;
    tfq::GemmArgs g{a_q, b_q, nullptr, nullptr, (const uint16_t*)bias_bf16, (uint16_t*)y_bf16,
                    nullptr, m, n, k, fmt == 0 ? tfq::kMxE2M3 : tfq::kMxE3M2, 0, epi, a_scale,
                    b_scale};
    return hip_status(tfq::launch_scaled_gemm(g, (hipStream_t)stream));
}

tfq_status tfq_scaled_mm_mxfp8(const uint8_t* a_q, const uint32_t* a_scale, const uint8_t* b_q,
                               const uint32_t* b_scale, int64_t m, int64_t n, int64_t k,
                               const void* bias_bf16, int32_t epi, void* y_bf16, void* stream)
{
    if (!a_q || !a_scale || !b_q || !b_scale || !y_bf16) return TFQ_ERR_NULL_POINTER;
    if (!epi_ok(epi)) return TFQ_ERR_UNSUPPORTED;
    if (m < 1 || m > kMaxDim || n < 8 || n > kMaxDim || n % 8 != 0 || k < 128 ||
        k > ((int64_t)1 << 22) || k % 128 != 0 || !mx_scales_fit(m, k) || !mx_scales_fit(n, k))
        return TFQ_ERR_BAD_SHAPE;
    if (((m + 255) / 256) * ((n + 255) / 256) > INT32_MAX) return TFQ_ERR_BAD_SHAPE;
    if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(a_scale, 4) || !aligned(b_scale, 4) ||
        (bias_bf16 && !aligned(bias_bf16, 16)) || !aligned(y_bf16, 16))
        return TFQ_ERR_MISALIGNED;
    const Range ry = range_of(y_bf16, m * n * 2);
    const Range ins[5] = {range_of(a_q, m * k), range_of(b_q, n * k), range_of(a_scale, m * (k / 32)),
                          range_of(b_scale, n * (k / 32)), range_of(bias_bf16, bias_bf16 ? n * 2 : 0)};
    for (const Range& r : ins)
        if (overlap(r, ry)) return TFQ_ERR_ALIAS;
    tfq_status st = check_device();
    if (st != TFQ_OK) return st;
    tfq::GemmArgs g{a_q, b_q, nullptr, nullptr, (const uint16_t*)bias_bf16, (uint16_t*)y_bf16,
                    nullptr, m, n, k, tfq::kMxE4M3, 0, epi, a_scale, b_scale};
    return hip_status(tfq::launch_scaled_gemm(g, (hipStream_t)stream));
}

tfq_status tfq_kv_cache_store(const void* kv_bf16, int64_t tokens, int64_t heads, int64_t head_dim,
                              int64_t ld_token, const int32_t* slot_index, int64_t slots,
                              float qmax, uint8_t* cache, float* cache_scale, void* stream)
{
    if (!kv_bf16 || !slot_index || !cache || !cache_scale) return TFQ_ERR_NULL_POINTER;
    if (tokens < 1 || tokens > kMaxDim || heads < 1 || heads > 65536 || head_dim < 8 ||
        head_dim > 512 || head_dim % 8 != 0 || slots < 1 || slots > kMaxDim ||
        ld_token < heads * head_dim || ld_token > ((int64_t)1 << 40) || tokens * heads > kMaxDim ||
        slots * heads > kMaxDim || tokens - 1 > ((int64_t)1 << 61) / ld_token)
        return TFQ_ERR_BAD_SHAPE;  // (the last bound keeps the input's byte span in range)
    if (ld_token % 8 != 0 || !aligned(kv_bf16, 16) || !aligned(cache, 16) ||
        !aligned(cache_scale, 4) || !aligned(slot_index, 4))
        return TFQ_ERR_MISALIGNED;
    if (!qmax_ok(TFQ_QTYPE_E4M3FN, qmax)) return TFQ_ERR_BAD_QMAX;
    const Range rkv = range_of(kv_bf16, ((tokens - 1) * ld_token + heads * head_dim) * 2);
    const Range rsl = range_of(slot_index, tokens * 4);
    const Range rc = range_of(cache, slots * heads * head_dim);
    const Range rs = range_of(cache_scale, slots * heads * 4);
    if (overlap(rc, rs) || overlap(rc, rkv) || overlap(rc, rsl) || overlap(rs, rkv) ||
        overlap(rs, rsl))
        return TFQ_ERR_ALIAS;
    tfq_status st = check_device();
    if (st != TFQ_OK) return st;
    return hip_status(tfq::launch_kv_store((const uint16_t*)kv_bf16, tokens, (int)heads,
                                           (int)head_dim, ld_token, slot_index, slots, qmax, cache,
                                           cache_scale, (hipStream_t)stream));
}

tfq_status tfq_kv_cache_load(const uint8_t* cache, const float* cache_scale, int64_t slots,
                             int64_t heads, int64_t head_dim, const int32_t* slot_index, int64_t n,
                             int32_t out_dtype, void* out, void* stream)
{
    if (!cache || !cache_scale || !slot_index || !out) return TFQ_ERR_NULL_POINTER;
    if (out_dtype < 0 || out_dtype > 2) return TFQ_ERR_UNSUPPORTED;
    if (n < 1 || n > kMaxDim || heads < 1 || heads > 65536 || head_dim < 8 || head_dim > 512 ||
        head_dim % 8 != 0 || slots < 1 || slots > kMaxDim || n * heads > kMaxDim ||
        slots * heads > kMaxDim)
        return TFQ_ERR_BAD_SHAPE;
    if (!aligned(cache, 16) || !aligned(cache_scale, 4) || !aligned(slot_index, 4) ||
        !aligned(out, 16))
        return TFQ_ERR_MISALIGNED;
    const int64_t esize = out_dtype == 2 ? 4 : 2;
    const Range ro = range_of(out, n * heads * head_dim * esize);
    if (overlap(ro, range_of(cache, slots * heads * head_dim)) ||
        overlap(ro, range_of(cache_scale, slots * heads * 4)) ||
        overlap(ro, range_of(slot_index, n * 4)))
        return TFQ_ERR_ALIAS;
    tfq_status st = check_device();
    if (st != TFQ_OK) return st;
    return hip_status(tfq::launch_kv_load(cache, cache_scale, slots, (int)heads, (int)head_dim,
                                          slot_index, n, out_dtype, out, (hipStream_t)stream));
}

tfq_status tfq_set_autotune(int32_t mode)
{
    if (mode != 0 && mode != 1) return TFQ_ERR_UNSUPPORTED;
    tfq::set_autotune(mode);
    return TFQ_OK;
}

// the GEMM kind codes of tfq_autotune_lookup / tfq_autotune_set
static bool gemm_kind(int32_t kind, int64_t m, int64_t n, int64_t k, int32_t epi, int32_t groups,
                      tfq::GemmArgs* out)
{
    tfq::GemmArgs g{};
    g.m = m;
    g.n = n;
    g.k = k;
    g.epi = epi;
    switch (kind) {
    case 0: g.qtype = tfq::kE4M3FN; break;
    case 1: g.qtype = tfq::kInt8; break;
    case 2: g.qtype = tfq::kE4M3FN; g.scale_block = 128; break;
    case 3: g.qtype = tfq::kMxE4M3; break;
    case 5: g.qtype = tfq::kMxE2M1; break;
    case 6: g.qtype = tfq::kMxE2M3; break;
    case 7: g.qtype = tfq::kMxE3M2; break;
    case 4: g.qtype = tfq::kE4M3FN; g.groups = groups; break;
    default: return false;
    }
    *out = g;
    return true;
}

tfq_status tfq_autotune_set(int32_t kind, int64_t m, int64_t n, int64_t k, int32_t epi, int32_t groups,
                            int32_t kernel, int32_t band)
{
    tfq::GemmArgs g{};
    if (!gemm_kind(kind, m, n, k, epi, groups, &g) || !epi_ok(epi)) return TFQ_ERR_UNSUPPORTED;
    if (kind == 4 && (groups < 1 || groups > 256)) return TFQ_ERR_BAD_SHAPE;
    if (m < 1 || n < 1 || k < 1) return TFQ_ERR_BAD_SHAPE;
    if (!tfq::config_is_candidate(g, tfq::GemmConfig{kernel, band})) return TFQ_ERR_UNSUPPORTED;
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return TFQ_ERR_UNSUPPORTED_DEVICE;
    }
    tfq::autotune_set(dev, g, tfq::GemmConfig{kernel, band});
    return TFQ_OK;
}

int32_t tfq_autotune_lookup(int32_t kind, int64_t m, int64_t n, int64_t k, int32_t epi,
                            int32_t groups, int32_t* kernel, int32_t* band)
{
    tfq::GemmArgs g{};
    if (!gemm_kind(kind, m, n, k, epi, groups, &g)) return 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    tfq::GemmConfig c;
    if (!tfq::autotune_lookup(dev, g, &c)) return 0;
    if (kernel) *kernel = c.kernel;
    if (band) *band = c.band;
    return 1;
}

void tfq_autotune_clear(void) { tfq::autotune_clear(); }

tfq_status tfq_e4m3fn_encode_f32(const float* x, uint8_t* q, int64_t n, void* stream)
{
    if (!x || !q) return TFQ_ERR_NULL_POINTER;
    if (n < 1 || n % 4 != 0 || n > ((int64_t)1 << 40)) return TFQ_ERR_BAD_SHAPE;
    if (!aligned(x, 16) || !aligned(q, 16)) return TFQ_ERR_MISALIGNED;
    if (overlap(range_of(x, n * 4), range_of(q, n))) return TFQ_ERR_ALIAS;
    tfq_status st = check_device();
    if (st != TFQ_OK) return st;
    return hip_status(tfq::launch_e4m3fn_encode(x, q, n, (hipStream_t)stream));
}

}  // extern "C"
