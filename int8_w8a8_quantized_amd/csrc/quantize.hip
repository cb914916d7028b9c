// Dynamic absmax quantisation kernels for gfx950 (CDNA4, wave64).
//
// Method: TeleFuser "Quantization", "Core ideas" (symmetric INT8,
// s = max|x|/127, q = clamp(round(x/s), -128, 127)) and "Scaled FP8
// checkpoints: W8A8" (per input row, s = max|x| / max(E4M3FN),
// q = cast_E4M3FN(clamp(x/s))); LightX2V "模型量化技术", "MiniMax-H3 FP8 FP16
// 累加" (scale = max(abs(x))/qmax with reduced qmax) and table "量化模式"
// (fp8-b128-deepgemm: 1x128 activation groups, 128x128 weight blocks).
//
// The kernels are HBM-bound (2 bytes in, 1 byte out per element):
//  * one wavefront per row, the whole row held in VGPRs between the absmax
//    pass and the encode pass (single HBM read), 128-bit loads, 64-bit code
//    stores, fully coalesced across the wave;
//  * the absmax is taken on the BF16 bit patterns with the sign cleared
//    (non-negative finite floats order like integers) using packed 16-bit
//    max, then reduced with DPP row operations and four readlanes;
//  * x / s is evaluated as q0 = x*r, e = fma(q0, s, -x), q = fma(-e, r, q0)
//    with r = RN(1/s) (Markstein's correction step, with the remainder
//    negated so that a zero x keeps its sign through every step).  For 2^-90 <= s <=
//    2^126 this equals the correctly rounded quotient whenever |x/s| >=
//    2^-12, and smaller quotients encode to zero either way (the sign is
//    restored from x): checked on the host for every BF16 amax and every BF16
//    x with |x| <= amax, both signs, at qmax 448, 14, 12, 7 and 127
//    (tests/test_divide_exhaustive.py); Markstein's theorem (a correctly
//    rounded reciprocal, a first quotient within one ulp, no underflow of the
//    remainder) covers the other accepted qmax values.  Rows with s < 2^-90
//    or s > 2^126 (including an overflowed s = inf, where x / s = +-0) use a
//    true division.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tfq_internal.h"

namespace tfq {
namespace {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b)
{
    us2 x = __builtin_bit_cast(us2, a), y = __builtin_bit_cast(us2, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

__device__ __forceinline__ uint32_t abs_max_chunk(uint32_t m, const uint4& v)
{
    m = pk_max_u16(m, v.x & 0x7FFF7FFFu);
    m = pk_max_u16(m, v.y & 0x7FFF7FFFu);
    m = pk_max_u16(m, v.z & 0x7FFF7FFFu);
    m = pk_max_u16(m, v.w & 0x7FFF7FFFu);
    return m;
}

// max over the 16 lanes of a DPP row; every lane of the row gets the result
__device__ __forceinline__ uint32_t row16_max(uint32_t m)
{
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xF, 0xF, false)); // row_half_mirror
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x140, 0xF, 0xF, false)); // row_mirror
    return m;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t m)
{
    m = row16_max(m);
    uint32_t a = __builtin_amdgcn_readlane(m, 0), b = __builtin_amdgcn_readlane(m, 16);
    uint32_t c = __builtin_amdgcn_readlane(m, 32), d = __builtin_amdgcn_readlane(m, 48);
    return max(max(a, b), max(c, d));
}

// RN(x / s) for the quantiser; see the file comment.  How a wave evaluates
// it: kFast, Markstein's step with no clamp needed; kFastClamp, the same
// step and the clamp to +-qmax; kDivide, an IEEE division and the clamp.
enum : int { kFast = 0, kFastClamp = 1, kDivide = 2 };

struct Quotient {
    float s, r;
    __device__ __forceinline__ explicit Quotient(float scale)
        : s(scale), r(scale == 0.0f ? 0.0f : 1.0f / scale)  // correctly rounded reciprocal
    {
    }
    template <int MODE>
    __device__ __forceinline__ float eval(float x) const
    {
        if constexpr (MODE == kDivide) {
            // a true division keeps the sign of a zero quotient; a lane with
            // s = 0 (an all-zero row or group in a wave that divides) takes
            // x * 0 = +-0, as Markstein's step gives it
            return s != 0.0f ? x / s : x * 0.0f;
        } else {
            // e = RN(q0 s - x) = -RN(x - q0 s), so q = RN(q0 + RN(x - q0 s) r)
            // as in the textbook form; every step is odd in x, and for x = -0
            // (or s = 0, r = 0) the last sum is -0 + -0, so q keeps the sign
            const float q0 = x * r;
            const float e = __builtin_fmaf(q0, s, -x);
            return __builtin_fmaf(-e, r, q0);
        }
    }
    // This lane's mode for a row or group with absmax amax.  Inside the
    // window the quotient is monotone in |x| (correctly rounded for |x/s| >=
    // 2^-12, below 2^-10 otherwise, and qmax >= 2^-9), so the largest is that
    // of amax; when it is <= qmax the clamp changes no element.
    __device__ __forceinline__ int lane_mode(float amax, float qmax) const
    {
        if (!((s >= 0x1p-90f && s <= 0x1p126f) || s == 0.0f)) return kDivide;
        return eval<kFast>(amax) <= qmax ? kFast : kFastClamp;
    }
};

// One mode for the whole wave (a wave-uniform value, so the encode loops
// branch once): the largest of its lanes' modes.  Every lane gets the same
// codes as under its own mode: the clamp is exact where it is not needed,
// and inside the window the division equals Markstein's step wherever
// |x/s| >= 2^-12, while smaller quotients encode to a signed zero either way.
__device__ __forceinline__ int wave_mode(int lane_mode)
{
    if (__ballot(lane_mode == kDivide)) return kDivide;
    return __ballot(lane_mode == kFastClamp) ? kFastClamp : kFast;
}

// f(std::integral_constant<int, MODE>) for the wave's mode
template <typename F>
__device__ __forceinline__ void with_mode(int mode, F&& f)
{
    if (mode == kFast)
        f(std::integral_constant<int, kFast>());
    else if (mode == kFastClamp)
        f(std::integral_constant<int, kFastClamp>());
    else
        f(std::integral_constant<int, kDivide>());
}

template <int QT, bool CLAMP = true>
__device__ __forceinline__ uint32_t encode4(float t0, float t1, float t2, float t3, float qmax)
{
    if constexpr (CLAMP) {
        t0 = __builtin_amdgcn_fmed3f(t0, -qmax, qmax);
        t1 = __builtin_amdgcn_fmed3f(t1, -qmax, qmax);
        t2 = __builtin_amdgcn_fmed3f(t2, -qmax, qmax);
        t3 = __builtin_amdgcn_fmed3f(t3, -qmax, qmax);
    }
    if constexpr (QT == kE4M3FN) {
        // gfx950 converts to OCP E4M3FN with round-to-nearest-even
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(t0, t1, 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(t2, t3, v, true);
        return (uint32_t)v;
    } else {
        // |t| <= qmax <= 127 after the clamp: round half to even, then pack
        uint32_t b0 = (uint32_t)(int)__builtin_rintf(t0) & 0xFFu;
        uint32_t b1 = (uint32_t)(int)__builtin_rintf(t1) & 0xFFu;
        uint32_t b2 = (uint32_t)(int)__builtin_rintf(t2) & 0xFFu;
        uint32_t b3 = (uint32_t)(int)__builtin_rintf(t3) & 0xFFu;
        return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
    }
}

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

template <int QT, int MODE>
__device__ __forceinline__ uint2 encode_chunk(const uint4& v, const Quotient& d, float qmax)
{
    constexpr bool C = MODE != kFast;
    uint2 o;
    o.x = encode4<QT, C>(d.eval<MODE>(bf_lo(v.x)), d.eval<MODE>(bf_hi(v.x)),
                         d.eval<MODE>(bf_lo(v.y)), d.eval<MODE>(bf_hi(v.y)), qmax);
    o.y = encode4<QT, C>(d.eval<MODE>(bf_lo(v.z)), d.eval<MODE>(bf_hi(v.z)),
                         d.eval<MODE>(bf_lo(v.w)), d.eval<MODE>(bf_hi(v.w)), qmax);
    return o;
}

// Streaming reads of the per-row quantisers and the KV-cache store: every
// input element is read once, so the loads are marked non-temporal and the
// caches (L2, Infinity Cache) may drop those lines first.  Quantising X and
// G of the video-DiT FFN pair ran 12% and 7% faster so; the MX and 1x128
// group kernels ran 2-4% slower and keep plain loads.  The codes are stored
// normally: the GEMM that follows reads them, and non-temporal stores made
// it ~3% slower.  Values are unaffected.
typedef uint32_t nt_u4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p)
{
    const nt_u4 t = __builtin_nontemporal_load(reinterpret_cast<const nt_u4*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

constexpr int kRowsPerBlock = 4;  // one wave per row, 4 waves per workgroup

// Source of output row `row`: the row itself, or row gather[row] of x for a
// routed quantisation (TeleFuser "Quantization", "Other quantized data
// paths": MoE activations are quantised per row after routing).  An index
// outside [0, src_rows) reads as a row of zeros (ok = false: every load of
// the row is masked).
__device__ __forceinline__ const uint4* source_row(const uint16_t* x, int64_t row, int64_t ld,
                                                  const int32_t* gather, int64_t src_rows,
                                                  bool& ok)
{
    const int64_t r = gather != nullptr ? (int64_t)gather[row] : row;
    ok = r >= 0 && r < src_rows;
    return reinterpret_cast<const uint4*>(x + (ok ? r : 0) * ld);
}

// Per-row quantisation with the row resident in registers (cols <= CH*512).
template <int QT, int CH>
__global__ __launch_bounds__(256) void quantize_rows_resident(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, float qmax,
    uint8_t* __restrict__ q, float* __restrict__ scale, const int32_t* __restrict__ gather,
    int64_t src_rows)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= rows) return;
    bool ok;
    const uint4* xr = source_row(x, row, ld, gather, src_rows, ok);
    const int nchunk = ok ? (int)(cols >> 3) : 0;
    uint4 v[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int idx = c * 64 + lane;
        v[c] = (idx < nchunk) ? load_stream(xr + idx) : make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t m = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) m = abs_max_chunk(m, v[c]);
    m = max(m & 0xFFFFu, m >> 16);
    const uint32_t mw = wave_max(m);
    const float amax = __uint_as_float(mw << 16);
    const float s = amax / qmax;  // correctly rounded (IEEE division)
    if (lane == 0) scale[row] = s;
    const Quotient d(s);
    uint2* qr = reinterpret_cast<uint2*>(q + row * cols);
    const int nout = (int)(cols >> 3);
    with_mode(wave_mode(d.lane_mode(amax, qmax)), [&](auto mode) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = c * 64 + lane;
            if (idx < nout) qr[idx] = encode_chunk<QT, decltype(mode)::value>(v[c], d, qmax);
        }
    });
}

// Long rows resident in registers, WPR waves per row: each wave holds CH
// chunks of 64 x 8 elements of its part of the row; the row absmax is
// combined across the row's waves through LDS.  Shorter per-wave register
// footprints than one wave per row keep more rows in flight.  Arithmetic as
// in quantize_rows_resident, so results are identical.
template <int QT, int CH, int WPR>
__global__ __launch_bounds__(256) void quantize_rows_split(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, float qmax,
    uint8_t* __restrict__ q, float* __restrict__ scale, const int32_t* __restrict__ gather,
    int64_t src_rows)
{
    __shared__ uint32_t part_max[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int part = wave % WPR;
    // Row blocks in eight equal slices, each walked from its end: workgroup b
    // (dispatched to XCD b % 8) takes block S (b % 8) + S - 1 - b / 8.  A
    // GEMM's tile order gives each XCD its own eighth of the rows and walks
    // it forwards, so the rows a GEMM wrote last (the ends of the eighths)
    // are read first, while still in the Infinity Cache, and the codes
    // written last are the ones the next GEMM reads first.  Measured on the
    // video-DiT FFN pair: quantise X -4%, quantise G -3%.
    const int64_t nblk = (rows + (4 / WPR) - 1) / (4 / WPR);
    const int64_t S = (nblk + 7) / 8;
    const int64_t blk = (int64_t)(blockIdx.x & 7) * S + (S - 1 - (int64_t)(blockIdx.x >> 3));
    if (blk >= nblk) return;  // the whole workgroup, before any barrier
    const int64_t row = blk * (4 / WPR) + wave / WPR;
    const bool valid = row < rows;  // every wave reaches the barrier
    bool ok = false;
    const uint4* xr = valid ? source_row(x, row, ld, gather, src_rows, ok)
                            : reinterpret_cast<const uint4*>(x);
    const int nchunk = (int)(cols >> 3);
    uint4 v[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int idx = (part * CH + c) * 64 + lane;
        v[c] = (ok && idx < nchunk) ? load_stream(xr + idx) : make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t m = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) m = abs_max_chunk(m, v[c]);
    m = max(m & 0xFFFFu, m >> 16);
    m = wave_max(m);
    if (lane == 0) part_max[wave] = m;
    __syncthreads();
    uint32_t mw = 0;
#pragma unroll
    for (int w = 0; w < WPR; ++w) mw = max(mw, part_max[wave - part + w]);
    if (!valid) return;
    const float amax = __uint_as_float(mw << 16);
    const float s = amax / qmax;  // correctly rounded (IEEE division)
    if (part == 0 && lane == 0) scale[row] = s;
    const Quotient d(s);
    uint2* qr = reinterpret_cast<uint2*>(q + row * cols);
    with_mode(wave_mode(d.lane_mode(amax, qmax)), [&](auto mode) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = (part * CH + c) * 64 + lane;
            if (idx < nchunk) qr[idx] = encode_chunk<QT, decltype(mode)::value>(v[c], d, qmax);
        }
    });
}

// Per-row quantisation of long rows: an absmax pass, then a second read.
template <int QT>
__global__ __launch_bounds__(256) void quantize_rows_two_pass(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, float qmax,
    uint8_t* __restrict__ q, float* __restrict__ scale, const int32_t* __restrict__ gather,
    int64_t src_rows)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= rows) return;
    bool ok;
    const uint4* xr = source_row(x, row, ld, gather, src_rows, ok);
    const int64_t nchunk = cols >> 3;
    uint32_t m = 0;
    if (ok)
        for (int64_t idx = lane; idx < nchunk; idx += 64) m = abs_max_chunk(m, xr[idx]);
    m = max(m & 0xFFFFu, m >> 16);
    const float amax = __uint_as_float(wave_max(m) << 16);
    const float s = amax / qmax;
    if (lane == 0) scale[row] = s;
    const Quotient d(s);
    uint2* qr = reinterpret_cast<uint2*>(q + row * cols);
    with_mode(wave_mode(d.lane_mode(amax, qmax)), [&](auto mode) {
        for (int64_t idx = lane; idx < nchunk; idx += 64)
            qr[idx] = encode_chunk<QT, decltype(mode)::value>(
                ok ? xr[idx] : make_uint4(0u, 0u, 0u, 0u), d, qmax);
    });
}

// 1x128 groups: 16 lanes x 8 elements cover one group, so every chunk of a
// wave holds 4 whole groups and no row needs to stay resident.
template <int QT>
__global__ __launch_bounds__(256) void quantize_groups128(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, float qmax,
    uint8_t* __restrict__ q, float* __restrict__ scale, const int32_t* __restrict__ gather,
    int64_t src_rows)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= rows) return;
    bool ok;
    const uint4* xr = source_row(x, row, ld, gather, src_rows, ok);
    const int nchunk = (int)(cols >> 3);  // multiple of 16
    const int ngroups = (int)(cols >> 7);
    uint2* qr = reinterpret_cast<uint2*>(q + row * cols);
    float* sr = scale + row * ngroups;
    constexpr int U = 4;
    for (int base = 0; base < nchunk; base += 64 * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = base + u * 64 + lane;
            v[u] = (ok && idx < nchunk) ? xr[idx] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = base + u * 64 + lane;
            uint32_t m = abs_max_chunk(0u, v[u]);
            m = max(m & 0xFFFFu, m >> 16);
            m = row16_max(m);  // the group's absmax in every lane of the group
            const float amax = __uint_as_float(m << 16);
            const float s = amax / qmax;
            const Quotient d(s);
            // (lanes past the row end hold zeros: amax 0, mode kFast)
            with_mode(wave_mode(d.lane_mode(amax, qmax)), [&](auto mode) {
                if (idx < nchunk) {
                    if ((lane & 15) == 0) sr[idx >> 4] = s;
                    qr[idx] = encode_chunk<QT, decltype(mode)::value>(v[u], d, qmax);
                }
            });
        }
    }
}

// MXFP8: E4M3FN elements with one E8M0 scale per 32 consecutive elements of
// a row (TeleFuser "Quantization", converter section: MXFP4/6/8 use 32-value
// blocks and E8M0 scales).  Block rule of the OCP MX v1.0 format: shared
// exponent floor(log2(amax)) - 8 (8 = exponent of E4M3's largest normal,
// 448 = 1.75 * 2^8), clamped to [-127, 127]; E8M0 byte = shared + 127.  For a
// BF16 amax with exponent field e that byte is max(e - 8, 0) (a subnormal or
// zero amax has e = 0).  Elements are x * 2^-shared -- an exact power-of-two
// scaling -- clamped to +-448 and encoded E4M3FN (RNE).  One wave per row; a
// lane holds 8 elements, 4 lanes one block, 16 lanes one 128-wide K group.
// The scale bytes of a group go out as one 32-bit word holding blocks
// 4 g + 0, 4 g + 2, 4 g + 1, 4 g + 3 in bytes 0..3, stored group-major --
// word (g, row) at g * rows + row -- the layout the MXFP8 GEMM loads whole
// per K stage (each half of the word is what one half of an MFMA's lanes
// needs).
//
// MXFP4 (F == 4): E2M1 elements (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), shared
// exponent floor(log2(amax)) - 2 (6 = 1.5 * 2^2), so the byte is
// max(e - 2, 0); elements x * 2^-shared clamped to +-6 and rounded to the
// nearest E2M1 value, ties to the even code, the sign kept (-0 -> 0x8).  Two
// codes per byte, the lower index in the low nibble: a lane's 8 elements are
// one 32-bit store.  gfx950 converts BF16 pairs this way in one instruction,
// v_cvt_scalef32_pk_fp4_bf16, which divides by the scale operand (the
// power of two 2^shared): on every finite BF16 input, under each scale
// tried from 2^-127 to 2^125, it gives the E2M1 codes of that rule (the
// MXFP4 quantiser tests check it against the oracle on every finite BF16
// value under eight such scales).
typedef __bf16 v2bf_mx __attribute__((ext_vector_type(2)));

// 2^(code - 127) for an E8M0 byte (2^-127, the byte 0, is a binary32 subnormal)
__device__ __forceinline__ float e8m0_value(int code)
{
    return __uint_as_float(code > 0 ? (uint32_t)code << 23 : 0x00400000u);
}

__device__ __forceinline__ uint32_t e2m1_pack8(const uint4& w, float scale)
{
    uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(v2bf_mx, w.x), scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf_mx, w.y), scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf_mx, w.z), scale, 2);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf_mx, w.w), scale, 3);
}

// MXFP6 (F == 62: E2M3, bias 1, largest 7.5; F == 63: E3M2, bias 3, largest
// 28): shared exponent floor(log2(amax)) - emax (2 / 4); elements
// x * 2^-shared clamped to the largest value and rounded to the nearest grid
// point, ties to the even code, the sign kept.  Six-bit codes are stored
// group-major: the 128 codes of group g of row r are a 96-byte
// little-endian bit stream (four codes in three bytes) at byte
// (g rows + r) 96, so the groups of one K range of all rows lie together (a
// GEMM stage reads a contiguous panel).  gfx950 converts 32 BF16 values this
// way in one instruction, v_cvt_scalef32_pk32_fp6_bf16 (E2M3) /
// v_cvt_scalef32_pk32_bf6_bf16 (E3M2), dividing by the scale operand (the
// power of two 2^shared) and writing the 32 codes as 24 bytes of that bit
// stream: on every finite BF16 input, under each scale tried from 2^-127 to
// 2^125, it gives the codes of the rule above (the MXFP6 quantiser tests
// check it against the oracle on every finite BF16 value under eight such
// scales).
typedef __bf16 v32bf_mx __attribute__((ext_vector_type(32)));
typedef int v6i_mx __attribute__((ext_vector_type(6)));

template <int F>  // 8: MXFP8 (E4M3FN), 4: MXFP4 (E2M1)
__global__ __launch_bounds__(256) void quantize_mx_kernel(const uint16_t* __restrict__ x,
                                                          int64_t rows, int64_t cols, int64_t ld,
                                                          uint8_t* __restrict__ q,
                                                          uint32_t* __restrict__ scale)
{
    // exponent of the element type's largest normal
    constexpr int kEmax = F == 8 ? 8 : 2;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= rows) return;
    const uint4* xr = reinterpret_cast<const uint4*>(x + row * ld);
    uint8_t* qrow = q + row * (F == 8 ? cols : cols / 2);
    const int nchunk = (int)(cols >> 3);  // a multiple of 16: whole groups only
    constexpr int U = 4;
    for (int base = 0; base < nchunk; base += 64 * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = base + u * 64 + lane;
            v[u] = idx < nchunk ? xr[idx] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = base + u * 64 + lane;
            uint32_t m = abs_max_chunk(0u, v[u]);
            m = max(m & 0xFFFFu, m >> 16);
            // block max over the 4 lanes of the quad
            m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));
            m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));
            const int code = max((int)((m >> 7) & 0xFFu) - kEmax, 0);
            const float inv = __uint_as_float((uint32_t)(254 - code) << 23);  // 2^(127 - code)
            // the codes of the group's other 3 blocks (lanes +4, +8, +12 of the
            // 16-lane DPP row) into the group's first lane
            const uint32_t word = (uint32_t)code |
                                  ((uint32_t)__builtin_amdgcn_update_dpp(0, code, 0x108, 0xF, 0xF, false) << 8) |
                                  ((uint32_t)__builtin_amdgcn_update_dpp(0, code, 0x104, 0xF, 0xF, false) << 16) |
                                  ((uint32_t)__builtin_amdgcn_update_dpp(0, code, 0x10C, 0xF, 0xF, false) << 24);
            if (idx < nchunk) {
                const uint4 w = v[u];
                if constexpr (F == 8) {
                    uint2 o;
                    o.x = encode4<kE4M3FN>(bf_lo(w.x) * inv, bf_hi(w.x) * inv, bf_lo(w.y) * inv,
                                           bf_hi(w.y) * inv, 448.0f);
                    o.y = encode4<kE4M3FN>(bf_lo(w.z) * inv, bf_hi(w.z) * inv, bf_lo(w.w) * inv,
                                           bf_hi(w.w) * inv, 448.0f);
                    reinterpret_cast<uint2*>(qrow)[idx] = o;
                } else {
                    reinterpret_cast<uint32_t*>(qrow)[idx] = e2m1_pack8(w, e8m0_value(code));
                }
                if ((lane & 15) == 0) scale[(int64_t)(idx >> 4) * rows + row] = word;
            }
        }
    }
}

// One round of a 4 x 4 transpose across a lane quad: element u of lane q
// takes element u ^ R of lane q ^ R where bit R of q ^ u is set.
template <int R>
__device__ __forceinline__ void quad_exchange(uint32_t (&a)[4][4], int qd)
{
    constexpr int kPerm = R == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
    uint32_t b[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t p = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a[u ^ R][k], kPerm, 0xF, 0xF, false);
            b[u][k] = ((qd ^ u) & R) ? p : a[u][k];
        }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) a[u][k] = b[u][k];
}

// MXFP6: 16 rows per workgroup, four 128-element groups of each at a time.
// Lane l of wave w takes row 4 w + (l >> 4) and loads chunk c = l & 15 (8
// elements) of each of the four groups, so a 16-lane DPP row reads a row's
// groups as whole 256-byte pieces.  A 4 x 4 transpose inside each lane quad
// (two DPP exchange rounds) then gives lane q of quad j the four chunks of
// block j of group q: one 32-element block per lane, as the conversion
// takes them.  The workgroup writes a group's codes for its 16 rows as one
// contiguous 1536-byte run of the group-major array (one wave per row
// scattered 96-byte pieces over every group's region: 22% slower on a
// 75600 x 13824 input).
template <int F>  // 62: E2M3, 63: E3M2
__global__ __launch_bounds__(256) void quantize_mx6_kernel(const uint16_t* __restrict__ x,
                                                           int64_t rows, int64_t cols, int64_t ld,
                                                           uint8_t* __restrict__ q,
                                                           uint32_t* __restrict__ scale)
{
    constexpr int kEmax = F == 63 ? 4 : 2;
    const int lane = threadIdx.x & 63, c = lane & 15, qd = lane & 3, blk = c >> 2;
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const bool live = row < rows;
    const uint4* xr = reinterpret_cast<const uint4*>(x + (live ? row : 0) * ld);
    const int groups = (int)(cols >> 7);
    for (int g0 = 0; g0 < groups; g0 += 4) {
        uint32_t a[4][4];  // [group u][dword] of the lane's chunk
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint4 t = live && g0 + u < groups ? xr[(g0 + u) * 16 + c] : make_uint4(0u, 0u, 0u, 0u);
            a[u][0] = t.x, a[u][1] = t.y, a[u][2] = t.z, a[u][3] = t.w;
        }
        // transpose: element u of lane q <- element q of lane u, in two
        // rounds (lanes and elements paired by xor 1, then by xor 2)
        quad_exchange<1>(a, qd);
        quad_exchange<2>(a, qd);
        // the lane now holds chunks 0..3 (a[0..3]) of block blk of group g0 + qd
        const int g = g0 + qd;
        uint32_t m = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) m = abs_max_chunk(m, make_uint4(a[i][0], a[i][1], a[i][2], a[i][3]));
        m = max(m & 0xFFFFu, m >> 16);
        const int code = max((int)((m >> 7) & 0xFFu) - kEmax, 0);
        // the group's scale word into its block-0 lane: blocks 0, 2, 1, 3 (lanes
        // +0, +8, +4, +12 of the 16-lane DPP row) in bytes 0..3
        const uint32_t word = (uint32_t)code |
                              ((uint32_t)__builtin_amdgcn_update_dpp(0, code, 0x108, 0xF, 0xF, false) << 8) |
                              ((uint32_t)__builtin_amdgcn_update_dpp(0, code, 0x104, 0xF, 0xF, false) << 16) |
                              ((uint32_t)__builtin_amdgcn_update_dpp(0, code, 0x10C, 0xF, 0xF, false) << 24);
        v32bf_mx e;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const v2bf_mx pr = __builtin_bit_cast(v2bf_mx, a[i][k]);
                e[8 * i + 2 * k] = pr[0];
                e[8 * i + 2 * k + 1] = pr[1];
            }
        v6i_mx r6;
        if constexpr (F == 62)
            r6 = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(e, e8m0_value(code));
        else
            r6 = __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(e, e8m0_value(code));
        if (live && g < groups) {
            // 24 bytes at block offset 24 blk: an even block starts 16-byte
            // aligned (16 + 8 bytes), an odd one 8 bytes past (8 + 16)
            uint8_t* qb = q + ((int64_t)g * rows + row) * 96 + blk * 24;
            const bool odd = blk & 1;
            *reinterpret_cast<uint4*>(qb + (odd ? 8 : 0)) =
                odd ? make_uint4(r6[2], r6[3], r6[4], r6[5]) : make_uint4(r6[0], r6[1], r6[2], r6[3]);
            *reinterpret_cast<uint2*>(qb + (odd ? 0 : 16)) =
                odd ? make_uint2(r6[0], r6[1]) : make_uint2(r6[4], r6[5]);
            if (blk == 0) scale[(int64_t)g * rows + row] = word;
        }
    }
}

// FP8 KV cache (TeleFuser "Quantization", "Other quantized data paths":
// LiveAct stores K and V as E4M3FN with one FP32 scale per last-dimension
// vector and dequantises them to the attention's dtype on load).
//
// Store: each (token, head) vector of head_dim elements is quantised as an
// FP8 activation row (absmax / qmax, the same division and encoding) and
// written to cache row slot[token] * heads + head.  P lanes (a power of two,
// 8 elements each, P * 8 >= head_dim) hold one vector; a workgroup takes
// KV_U rounds of 256 / P vectors, all loads first so that KV_U are in
// flight per lane.  The absmax is combined over the vector's lanes by DPP
// within a 16-lane row (P == 16, head_dim 128: 5% faster than shuffles) or
// by shuffles.  A slot outside [0, slots) is not written.
constexpr int KV_U = 4;

template <int P>
__global__ __launch_bounds__(256) void kv_store_kernel(
    const uint16_t* __restrict__ kv, int64_t tokens, int heads, int hd, int64_t ld_token,
    const int32_t* __restrict__ slot, int64_t slots, float qmax, uint8_t* __restrict__ cache,
    float* __restrict__ scale)
{
    // (tokens * heads <= 2^30: 32-bit vector indices)
    const int nv = (int)(tokens * heads);
    const int li = threadIdx.x % P;
    const bool lane_on = li < (hd >> 3);
    uint4 x[KV_U];
    int tok[KV_U], h[KV_U];
    bool in[KV_U];
#pragma unroll
    for (int u = 0; u < KV_U; ++u) {
        const int v = ((int)blockIdx.x * KV_U + u) * (256 / P) + (int)threadIdx.x / P;
        in[u] = v < nv;
        tok[u] = in[u] ? v / heads : 0;
        h[u] = in[u] ? v - tok[u] * heads : 0;
        x[u] = (in[u] && lane_on)
                   ? load_stream(reinterpret_cast<const uint4*>(kv + (int64_t)tok[u] * ld_token + (int64_t)h[u] * hd) + li)
                   : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < KV_U; ++u) {
        uint32_t m = abs_max_chunk(0u, x[u]);
        m = max(m & 0xFFFFu, m >> 16);
        if constexpr (P == 16) {
            m = row16_max(m);
        } else {
#pragma unroll
            for (int o = 1; o < P; o <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
        }
        const float amax = __uint_as_float(m << 16);
        const float s = amax / qmax;  // correctly rounded (IEEE division)
        const Quotient d(s);
        const int mode = wave_mode(d.lane_mode(amax, qmax));
        const int64_t sl = in[u] ? (int64_t)slot[tok[u]] : -1;
        if (lane_on && sl >= 0 && sl < slots) {
            const int64_t row = sl * heads + h[u];
            with_mode(mode, [&](auto md) {
                reinterpret_cast<uint2*>(cache + row * hd)[li] =
                    encode_chunk<kE4M3FN, decltype(md)::value>(x[u], d, qmax);
            });
            if (li == 0) scale[row] = s;
        }
    }
}

// Load: output vector (i, head) = scale * value of cache row
// index[i] * heads + head -- the E4M3FN decode is exact, the product is one
// binary32 multiplication (RNE), then one conversion to the output type
// (RNE).  An index outside [0, slots) gives a zero vector.  P threads (a
// power of two, 8 elements each) per vector, KV_LOAD_U rounds per workgroup
// with all loads first (2 rounds measured 10% faster than 4 at head_dim 128,
// 8 rounds 20% slower).
constexpr int KV_LOAD_U = 2;
typedef float v2f_q __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_q __attribute__((ext_vector_type(2)));
typedef _Float16 v2h_q __attribute__((ext_vector_type(2)));

template <int OUT, int P>  // OUT: 0 BF16, 1 FP16, 2 FP32
__global__ __launch_bounds__(256) void kv_load_kernel(
    const uint8_t* __restrict__ cache, const float* __restrict__ scale, int64_t slots, int heads,
    int hd, const int32_t* __restrict__ index, int64_t n, void* __restrict__ out)
{
    // (n * heads <= 2^30: 32-bit vector indices)
    const int nv = (int)(n * heads);
    const int ci = threadIdx.x % P;
    if (ci >= (hd >> 3)) return;
    int vec[KV_LOAD_U];
    uint2 q[KV_LOAD_U];
    float s[KV_LOAD_U];
#pragma unroll
    for (int u = 0; u < KV_LOAD_U; ++u) {
        vec[u] = ((int)blockIdx.x * KV_LOAD_U + u) * (256 / P) + (int)threadIdx.x / P;
        q[u] = make_uint2(0u, 0u);
        s[u] = 0.0f;
        if (vec[u] < nv) {
            const int i = vec[u] / heads;
            const int h = vec[u] - i * heads;
            const int64_t sl = index[i];
            if (sl >= 0 && sl < slots) {
                const int64_t row = sl * heads + h;
                q[u] = reinterpret_cast<const uint2*>(cache + row * hd)[ci];
                s[u] = scale[row];
            }
        }
    }
#pragma unroll
    for (int u = 0; u < KV_LOAD_U; ++u) {
        if (vec[u] >= nv) continue;
        // (a zero vector: codes 0 times scale 0)
        v2f_q f[4];
        f[0] = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[u].x, false) * s[u];
        f[1] = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[u].x, true) * s[u];
        f[2] = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[u].y, false) * s[u];
        f[3] = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[u].y, true) * s[u];
        const int64_t e0 = (int64_t)vec[u] * hd + ci * 8;
        if constexpr (OUT == 2) {
            float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + e0);
            o[0] = make_float4(f[0].x, f[0].y, f[1].x, f[1].y);
            o[1] = make_float4(f[2].x, f[2].y, f[3].x, f[3].y);
        } else {
            uint32_t w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (OUT == 0)
                    w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f[k], v2bf_q));
                else
                    w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f[k], v2h_q));
            }
            *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + e0) =
                make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

// 128x128 weight blocks: one workgroup (256 threads) per block.
template <int QT>
__global__ __launch_bounds__(256) void quantize_blocks128(
    const uint16_t* __restrict__ w, int64_t /* n: the grid covers its n/128 blocks */, int64_t k,
    float qmax, uint8_t* __restrict__ q,
    float* __restrict__ scale)
{
    __shared__ uint32_t red[4];
    const int64_t kb_count = k >> 7;
    const int64_t nb = blockIdx.x / kb_count, kb = blockIdx.x % kb_count;
    const int t = threadIdx.x;
    // 128 rows x 16 chunks of 8 elements; thread t takes chunk t%16 of rows t/16 + 16 i
    const int cc = t & 15, r0 = t >> 4;
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t row = nb * 128 + r0 + 16 * i;
        v[i] = reinterpret_cast<const uint4*>(w + row * k + kb * 128)[cc];
    }
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = abs_max_chunk(m, v[i]);
    m = max(m & 0xFFFFu, m >> 16);
    m = wave_max(m);
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    const float amax = __uint_as_float(m << 16);
    const float s = amax / qmax;
    if (t == 0) scale[nb * kb_count + kb] = s;
    const Quotient d(s);
    with_mode(wave_mode(d.lane_mode(amax, qmax)), [&](auto mode) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t row = nb * 128 + r0 + 16 * i;
            reinterpret_cast<uint2*>(q + row * k + kb * 128)[cc] =
                encode_chunk<QT, decltype(mode)::value>(v[i], d, qmax);
        }
    });
}

__global__ __launch_bounds__(256) void e4m3fn_encode_kernel(const float4* __restrict__ x,
                                                            uint32_t* __restrict__ q, int64_t n4)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const float4 v = x[i];
    q[i] = encode4<kE4M3FN>(v.x, v.y, v.z, v.w, 448.0f);
}

// source rows of a launch: an optional gather index and the number of rows
// of x it may name
struct Src {
    const int32_t* gather;
    int64_t rows;
};

template <int QT, int CH>
hipError_t launch_resident(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float qmax,
                           uint8_t* q, float* s, Src src, hipStream_t st)
{
    const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL((quantize_rows_resident<QT, CH>), dim3((unsigned)blocks), dim3(256), 0, st,
                       x, rows, cols, ld, qmax, q, s, src.gather, src.rows);
    return hipGetLastError();
}

// wg_per_cu > 0 caps the workgroups resident on a CU by giving each one an
// unused share of the CU's 160 KB of LDS.  With two waves per row (rows of
// 8K-16K columns) two workgroups per CU -- four rows, ~110 KB of loads in
// flight per CU -- stream best: quantising the video-DiT G [75600, 13824]
// went from 5.69 to 6.00 TB/s right after the GEMM that writes G, and from
// 5.41 to 5.90 TB/s on its own (1, 3 or more per CU, or 4 waves per row at
// 2-6 per CU: 4.7-5.96 TB/s; a persistent double-buffered variant: 5.0-5.5).
template <int QT, int CH, int WPR>
hipError_t launch_split(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float qmax,
                        uint8_t* q, float* s, Src src, hipStream_t st, int wg_per_cu = 0)
{
    constexpr unsigned kLdsPerCu = 160u << 10;
    const int64_t rpb = 4 / WPR;
    const int64_t blocks = 8 * (((rows + rpb - 1) / rpb + 7) / 8);  // eight equal slices
    const unsigned pad = wg_per_cu > 0 ? kLdsPerCu / (unsigned)wg_per_cu - 1024u : 0u;
    hipLaunchKernelGGL((quantize_rows_split<QT, CH, WPR>), dim3((unsigned)blocks), dim3(256), pad,
                       st, x, rows, cols, ld, qmax, q, s, src.gather, src.rows);
    return hipGetLastError();
}

template <int QT>
hipError_t launch_rows_qt(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float qmax,
                          uint8_t* q, float* s, Src src, hipStream_t st)
{
    const int64_t chunks = (cols >> 3);
    const int64_t per_lane = (chunks + 63) / 64;
    if (per_lane <= 2) return launch_resident<QT, 2>(x, rows, cols, ld, qmax, q, s, src, st);
    if (per_lane <= 4) return launch_resident<QT, 4>(x, rows, cols, ld, qmax, q, s, src, st);
    if (per_lane <= 6) return launch_resident<QT, 6>(x, rows, cols, ld, qmax, q, s, src, st);
    if (per_lane <= 8) return launch_resident<QT, 8>(x, rows, cols, ld, qmax, q, s, src, st);
    // 4097..6144 columns: 4 waves per row (3% faster at 5120 than one wave;
    // at 3072 one wave per row is 17% faster)
    if (per_lane <= 12) return launch_split<QT, 3, 4>(x, rows, cols, ld, qmax, q, s, src, st);
    // longer rows: 2 waves per row up to 16384 columns (two workgroups per
    // CU, see launch_split), 4 up to 32768
    if (per_lane <= 16) return launch_split<QT, 8, 2>(x, rows, cols, ld, qmax, q, s, src, st, 2);
    if (per_lane <= 20) return launch_split<QT, 10, 2>(x, rows, cols, ld, qmax, q, s, src, st, 2);
    if (per_lane <= 24) return launch_split<QT, 12, 2>(x, rows, cols, ld, qmax, q, s, src, st, 2);
    if (per_lane <= 28) return launch_split<QT, 14, 2>(x, rows, cols, ld, qmax, q, s, src, st, 2);
    if (per_lane <= 32) return launch_split<QT, 16, 2>(x, rows, cols, ld, qmax, q, s, src, st, 2);
    if (per_lane <= 48) return launch_split<QT, 12, 4>(x, rows, cols, ld, qmax, q, s, src, st);
    if (per_lane <= 64) return launch_split<QT, 16, 4>(x, rows, cols, ld, qmax, q, s, src, st);
    const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL((quantize_rows_two_pass<QT>), dim3((unsigned)blocks), dim3(256), 0, st, x,
                       rows, cols, ld, qmax, q, s, src.gather, src.rows);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                                int qtype, float qmax, int group_cols, uint8_t* q, float* scale,
                                hipStream_t stream, const int32_t* gather, int64_t src_rows)
{
    const Src src{gather, gather != nullptr ? src_rows : rows};
    if (group_cols == 128) {
        const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
        if (qtype == kE4M3FN)
            hipLaunchKernelGGL((quantize_groups128<kE4M3FN>), dim3((unsigned)blocks), dim3(256), 0,
                               stream, x, rows, cols, ld, qmax, q, scale, src.gather, src.rows);
        else
            hipLaunchKernelGGL((quantize_groups128<kInt8>), dim3((unsigned)blocks), dim3(256), 0,
                               stream, x, rows, cols, ld, qmax, q, scale, src.gather, src.rows);
        return hipGetLastError();
    }
    if (qtype == kE4M3FN) return launch_rows_qt<kE4M3FN>(x, rows, cols, ld, qmax, q, scale, src, stream);
    return launch_rows_qt<kInt8>(x, rows, cols, ld, qmax, q, scale, src, stream);
}

hipError_t launch_quantize_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                              uint8_t* q, uint32_t* scale, hipStream_t stream, int elem_bits)
{
    const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
    if (elem_bits == 4)
        hipLaunchKernelGGL((quantize_mx_kernel<4>), dim3((unsigned)blocks), dim3(256), 0, stream, x,
                           rows, cols, ld, q, scale);
    else if (elem_bits == 62 || elem_bits == 63)
        hipLaunchKernelGGL((elem_bits == 62 ? quantize_mx6_kernel<62> : quantize_mx6_kernel<63>),
                           dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, x, rows, cols, ld,
                           q, scale);
    else
        // MXFP8: 52 KB of unused LDS per workgroup caps residency at 3
        // workgroups per CU, which measured 4-5% faster on 75600-row inputs
        // (2 per CU, or none: slower; MXFP4 and MXFP6 gain nothing)
        hipLaunchKernelGGL((quantize_mx_kernel<8>), dim3((unsigned)blocks), dim3(256), 52u << 10,
                           stream, x, rows, cols, ld, q, scale);
    return hipGetLastError();
}

hipError_t launch_quantize_blocks(const uint16_t* w, int64_t n, int64_t k, int qtype, float qmax,
                                  uint8_t* q, float* scale, hipStream_t stream)
{
    const int64_t blocks = (n >> 7) * (k >> 7);
    if (qtype == kE4M3FN)
        hipLaunchKernelGGL((quantize_blocks128<kE4M3FN>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, w, n, k, qmax, q, scale);
    else
        hipLaunchKernelGGL((quantize_blocks128<kInt8>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, w, n, k, qmax, q, scale);
    return hipGetLastError();
}

hipError_t launch_kv_store(const uint16_t* kv, int64_t tokens, int heads, int hd, int64_t ld_token,
                           const int32_t* slot, int64_t slots, float qmax, uint8_t* cache,
                           float* scale, hipStream_t stream)
{
    const int lanes = (hd + 7) / 8;
    const int64_t nvec = tokens * heads;
#define TFQ_KV_STORE(P)                                                                           \
    hipLaunchKernelGGL((kv_store_kernel<P>), dim3((unsigned)((nvec + KV_U * 256 / P - 1) / (KV_U * 256 / P))), \
                       dim3(256), 0, stream, kv, tokens, heads, hd, ld_token, slot, slots, qmax,    \
                       cache, scale)
    if (lanes <= 4)
        TFQ_KV_STORE(4);
    else if (lanes <= 8)
        TFQ_KV_STORE(8);
    else if (lanes <= 16)
        TFQ_KV_STORE(16);
    else if (lanes <= 32)
        TFQ_KV_STORE(32);
    else
        TFQ_KV_STORE(64);
#undef TFQ_KV_STORE
    return hipGetLastError();
}

hipError_t launch_kv_load(const uint8_t* cache, const float* scale, int64_t slots, int heads, int hd,
                          const int32_t* index, int64_t n, int out_dtype, void* out,
                          hipStream_t stream)
{
    const int lanes = (hd + 7) / 8;
    const int64_t nvec = n * heads;
#define TFQ_KV_LOAD(O, P)                                                                         \
    hipLaunchKernelGGL((kv_load_kernel<O, P>), dim3((unsigned)((nvec + KV_LOAD_U * 256 / P - 1) / (KV_LOAD_U * 256 / P))), \
                       dim3(256), 0, stream, cache, scale, slots, heads, hd, index, n, out)
#define TFQ_KV_LOAD_P(O)       \
    if (lanes <= 4)            \
        TFQ_KV_LOAD(O, 4);     \
    else if (lanes <= 8)       \
        TFQ_KV_LOAD(O, 8);     \
    else if (lanes <= 16)      \
        TFQ_KV_LOAD(O, 16);    \
    else if (lanes <= 32)      \
        TFQ_KV_LOAD(O, 32);    \
    else                       \
        TFQ_KV_LOAD(O, 64)
    if (out_dtype == 0) {
        TFQ_KV_LOAD_P(0);
    } else if (out_dtype == 1) {
        TFQ_KV_LOAD_P(1);
    } else {
        TFQ_KV_LOAD_P(2);
    }
#undef TFQ_KV_LOAD_P
#undef TFQ_KV_LOAD
    return hipGetLastError();
}

hipError_t launch_e4m3fn_encode(const float* x, uint8_t* q, int64_t n, hipStream_t stream)
{
    const int64_t n4 = n >> 2;
    const int64_t blocks = (n4 + 255) / 256;
    hipLaunchKernelGGL(e4m3fn_encode_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const float4*>(x), reinterpret_cast<uint32_t*>(q), n4);
    return hipGetLastError();
}

}  // namespace tfq
