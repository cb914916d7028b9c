// Scaled W8A8 GEMM for gfx950 (CDNA4): y = (a . b^T) * s_a[m] * s_b[n] -> BF16.
//
// Method: TeleFuser "Quantization", "tf-kernel FP8: online W8A8" (per-token
// FP8 activations x per-output-channel FP8 weights -> BF16 via a scaled
// GEMM) and "Core ideas" (symmetric INT8, x_hat = s q, so the product of the
// dequantised operands factors into s_a s_b (q_a . q_b)); block mode follows
// LightX2V "模型量化技术", table "量化模式" (fp8-b128-deepgemm): one scale per
// 1x128 activation group and per 128x128 weight block, applied per K-block.
//
// Design (MI355X):
//  * both operands are K-contiguous ("TN"), the layout MFMA operands want;
//  * the K order inside an MFMA does not change the sum as long as A and B
//    use the same one, so each lane group reads 32 contiguous bytes;
//  * main kernel: operands go from global memory straight into LDS with
//    buffer loads carrying the LDS modifier (no VGPR staging, no LDS write
//    instructions), in 128-byte K stages so that every row load is one whole
//    cache line; out-of-range rows and the K tail read as zero, so ragged
//    M/N/K need no branches; LDS rows are chunk-swizzled to be free of bank
//    conflicts for the MFMA fragment reads;
//  * the block-scaled and two-workgroups-per-CU kernels stage 64-byte K
//    stages through a ring of VGPRs (128-bit buffer loads) into LDS;
//  * the weights are the first MFMA operand, so each lane finishes with four
//    consecutive output columns of one row; the epilogue scales in FP32,
//    stages BF16 rows in LDS and writes whole row segments with 16-byte
//    stores;
//  * tile order: consecutive workgroup ids go round-robin over the 8 XCDs,
//    so ids are remapped to give each XCD a contiguous slice of the tile
//    sequence, which walks bands of 2 or 4 tile rows so that the tiles in flight
//    on one XCD share A and B panels in that XCD's L2;
//  * epilogue arithmetic: FP32 (acc * s_a) * s_b [+ bias] [GELU-tanh] -> BF16
//    (RNE), each step rounded on its own; the INT8 path converts the exact
//    INT32 sum to FP32 first (bit-reproducible); raw INT32 output optional.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#include <type_traits>

#include "tfq_internal.h"

namespace tfq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256;  // output tile of the per-token / per-channel kernel

struct Params {
    const uint8_t* a;
    const uint8_t* b;
    const float* sa;
    const float* sb;
    const uint32_t* ea;  // MXFP8 E8M0 scale words [k/128, m]
    const uint32_t* eb;  // MXFP8 E8M0 scale words [k/128, n]
    const uint16_t* bias;
    uint16_t* y;
    int32_t* acc;
    int m, n, k;
    int tiles_m, tiles_n;
    int group_m;           // tile rows per band of the tile order
    const int32_t* goff;   // grouped (MoE) mode: row offsets [groups + 1]
    int groups;            // grouped mode: number of weight groups (<= 256)
};

__device__ __forceinline__ void map_tile(int bid, int tiles_m, int tiles_n, int group_m, int& tm, int& tn)
{
    const int total = tiles_m * tiles_n;
    const int full = total & ~7;
    int id = bid;
    if (bid < full) id = (bid & 7) * (full >> 3) + (bid >> 3);
    const int band_tiles = group_m * tiles_n;
    const int band = id / band_tiles;
    const int first = band * group_m;
    const int gm = min(tiles_m - first, group_m);
    const int in = id - band * band_tiles;
    tm = first + in % gm;
    tn = in / gm;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }


// two floats -> two BF16 (round to nearest even) in one 32-bit word, lo in
// the low half: one v_cvt_pk_bf16_f32
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{lo, hi}, v2bf));
}

// (v * s_row) * s_col and + bias, each rounded on its own (never fused into
// an FMA): the fixed order that makes the INT8 BF16 output reproducible.
__device__ __forceinline__ float scale_out(float v, float srow, float scol)
{
#pragma clang fp contract(off)
    const float t = v * srow;
    return t * scol;
}

__device__ __forceinline__ float add_bias(float v, float b)
{
#pragma clang fp contract(off)
    return v + b;
}

// GELU, tanh form: 0.5 h (1 + tanh(u)) = h / (1 + exp(-2u)),
// u = sqrt(2/pi) (h + 0.044715 h^3)
__device__ __forceinline__ float gelu_tanh(float h)
{
    const float c1 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
    const float c2 = c1 * 0.044715f;
    const float z = h * __builtin_fmaf(c2, h * h, c1);
    const float e = __builtin_amdgcn_exp2f(z);
    return h * __builtin_amdgcn_rcpf(1.0f + e);
}

// ---------------------------------------------------------------------------
// Main kernel for per-token / per-channel scales: 256x256 output tile, 4
// waves x (128 x 128) with v_mfma_f32_32x32x64_f8f6f4 (FP8) or 2x
// v_mfma_i32_32x32x32_i8 (INT8), accumulators in AGPRs (one wave per SIMD).
// 128 K-bytes per stage, 2 LDS buffers of 64 KB filled by LDS-DMA loads one
// stage ahead, one barrier per stage.
// ---------------------------------------------------------------------------
constexpr int PK = 128;               // K bytes per stage: whole 128-byte lines
constexpr int PA = BM * PK;           // 32 KB of A per stage
constexpr int PSTAGE = PA + BN * PK;  // 64 KB per LDS buffer
constexpr int EPITCH = 272;           // bytes per staged output row (256 + 16)
constexpr int PBUF = 2;               // LDS buffers: stages in flight
// the tile's row scales, column scales and BF16 bias (1 KB each) sit past
// both the pipeline buffers and the output staging area
constexpr int PSCL = (PBUF * PSTAGE > 4 * 128 * EPITCH) ? PBUF * PSTAGE : 4 * 128 * EPITCH;
// MXFP8: the E8M0 scale words of two stages (A rows, then B rows; one word =
// the stage's 4 K blocks of a row)
constexpr int PMXS = PSCL + 3 * 1024;
constexpr int PMXRING = 2;
constexpr int PSMEM = PMXS + PMXRING * 2048;
// MXFP6: three stages of packed 96-byte rows (A's three 24 KB stages, then
// B's), then the bias (and the unused scale slots), then a 4-slot ring of
// E8M0 scale words
constexpr int P6OP = BM * 96;        // one operand's stage
constexpr int P6B = 3 * P6OP;        // where B's stages start
constexpr int P6SCL = 6 * P6OP;
constexpr int P6MXS = P6SCL + 3 * 1024;
constexpr int P6SMEM = P6MXS + 4 * 2048;

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v16i __attribute__((ext_vector_type(16)));

// all of this wave's LDS operations are complete, then a workgroup barrier
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Buffer resource of `records` bytes from `base` (raw, no swizzle, loads
// past the end return zero): word 3 is the gfx950 data-format word of an
// untyped 32-bit buffer.
__device__ __forceinline__ v4i buffer_rsrc(const void* base, int records)
{
    // readfirstlane: the inline-asm loads need the descriptor in SGPRs even
    // where the compiler cannot prove the value uniform
    const uint64_t a = (uint64_t)base;
    return v4i{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)),
               __builtin_amdgcn_readfirstlane(records), 0x00020000};
}

// 64 lanes x 16 bytes from the buffer at per-lane byte offset `off` straight
// into LDS [lds, lds + 1024), lane l at lds + 16 l.  The compiler does not see
// this load: the caller orders it with explicit vmcnt waits.
__device__ __forceinline__ void lds_dma16(const v4i& rsrc, int off, uint32_t lds)
{
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(rsrc),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}

// Lane id (0..63) computed in place by an asm block the compiler cannot hoist
// or merge: values derived from it are rebuilt where they are used instead of
// being kept live (and spilled) across long loops.
__device__ __forceinline__ int lane_id_here()
{
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// 64 lanes x 4 bytes from the buffer at per-lane byte offset `off` straight
// into LDS [lds, lds + 256), lane l at lds + 4 l (caller orders with vmcnt)
__device__ __forceinline__ void lds_dma4(const v4i& rsrc, int off, uint32_t lds)
{
    asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(off), "s"(rsrc),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}

template <int QT>
struct PipeAcc;
template <>
struct PipeAcc<kE4M3FN> {
    typedef v16f type;
};
template <>
struct PipeAcc<kInt8> {
    typedef v16i type;
};
template <>
struct PipeAcc<kMxE4M3> {
    typedef v16f type;
};
template <>
struct PipeAcc<kMxE2M1> {
    typedef v16f type;
};
template <>
struct PipeAcc<kMxE2M3> {
    typedef v16f type;
};
template <>
struct PipeAcc<kMxE3M2> {
    typedef v16f type;
};

// NB: 32-column B fragments per wave, so the tile is 256 x (64 NB): NB = 4
// (256 columns) for every type, NB = 3 (192 columns) for per-channel FP8 and
// INT8, whose tile counts can then end on a whole wave of CUs.  Both widths
// run the same MFMAs over the same K steps for every output, so they give
// the same bits.
template <int QT, int EPI, bool WANT_Y, bool WANT_ACC, bool GROUPED = false, int NB = 4>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void gemm_pipe_kernel(const Params p)
{
    static_assert(NB == 4 || (NB == 3 && (QT == kE4M3FN || QT == kInt8) && !GROUPED),
                  "192-column tiles: per-channel FP8 / INT8");
    constexpr int TBN = 64 * NB;  // tile columns
    constexpr int WNC = 32 * NB;  // columns per wave
    // MXFP4 rows hold two codes per byte: K counts bytes below, and a stage
    // (128 bytes) holds 256 elements = two 128-element scale groups
    constexpr bool FP4 = QT == kMxE2M1;
    // MXFP6 rows hold 3 bytes per 4 codes: a stage is 128 elements = 96
    // bytes, kept as packed 96-byte LDS rows (a pipeline of its own below)
    constexpr bool FP6 = QT == kMxE2M3 || QT == kMxE3M2;
    constexpr int SK = FP6 ? 96 : PK;  // K bytes per stage
    __shared__ __attribute__((aligned(16))) uint8_t smem[FP6 ? P6SMEM : FP4 ? PSMEM + 2 * 2048 : PSMEM];
    constexpr int SCL = FP6 ? P6SCL : PSCL;  // the tile's row / column scales and bias

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    int tm, tn, m0, m_end = p.m;
    const uint8_t* b_grp = p.b;
    const float* sb_grp = p.sb;
    const uint16_t* bias_grp = p.bias;
    if constexpr (GROUPED) {
        // Routed (MoE) rows (TeleFuser "Quantization", "Other quantized data
        // paths": routed activations per row, expert weights per output
        // channel): group g owns rows goff[g] .. goff[g+1] and weight matrix
        // g; its ceil(rows / 256) x tiles_n tiles run in bands of group_m
        // tile rows.  Workgroup b runs on XCD b % 8 as that XCD's
        // (b / 8)-th workgroup.  Each XCD takes its own eighth of every
        // group's tiles, group after group, so that all XCDs work on the same
        // experts' weights at a time (they stay in the Infinity Cache) while
        // each XCD's tiles are neighbours (its L2 shares their panels).
        // Thread g reads group g's offsets, clamped to [0, m] so that any
        // offsets keep every access in bounds; a scan over the threads of
        // the slice sizes finds the group of this workgroup's tile.
        int* gs = reinterpret_cast<int*>(smem + PMXS);
        if (t == 0) gs[256] = gs[257] = gs[258] = 0;  // (kept only if no tile is found)
        const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
        int lo = 0, hi = 0, cnt = 0, s0 = 0, sz = 0;
        if (t < p.groups) {
            lo = min(max(p.goff[t], 0), p.m);
            hi = max(lo, min(max(p.goff[t + 1], 0), p.m));
            cnt = (hi - lo + BM - 1) / BM;
            const int64_t tiles = (int64_t)cnt * p.tiles_n;
            s0 = (int)(tiles * xcd / 8);
            sz = (int)(tiles * (xcd + 1) / 8) - s0;
        }
        int v = sz;
        gs[t] = v;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {
            const int add = t >= d ? gs[t - d] : 0;
            __syncthreads();
            v += add;
            gs[t] = v;
            __syncthreads();
        }
        if (t < p.groups && v - sz <= j && j < v) {
            // tile s0 + (j - start) of group t, in bands of group_m tile rows
            const int local = s0 + (j - (v - sz));
            const int band_tiles = p.group_m * p.tiles_n;
            const int band = local / band_tiles;
            const int first = band * p.group_m;
            const int gm = min(cnt - first, p.group_m);
            const int in = local - band * band_tiles;
            gs[256] = t;
            gs[257] = lo + (first + in % gm) * BM;
            gs[258] = hi;
            gs[259] = in / gm;
        }
        __syncthreads();
        if (gs[258] == 0) return;  // no tile for this workgroup (uniform)
        const int g = gs[256];
        m0 = gs[257];
        m_end = gs[258];
        tn = gs[259];
        tm = 0;
        b_grp += (int64_t)g * p.n * p.k;
        sb_grp += (int64_t)g * p.n;
        if (bias_grp != nullptr) bias_grp += (int64_t)g * p.n;
    } else {
        map_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
        m0 = tm * BM;
    }
    const int n0 = tn * TBN;
    const int K = FP4 ? p.k / 2 : FP6 ? p.k / 4 * 3 : p.k;
    const int rows_a = min(BM, m_end - m0), rows_b = min(TBN, p.n - n0);
    const v4i ra = buffer_rsrc(p.a + (int64_t)m0 * K, rows_a * K);
    const v4i rb = buffer_rsrc(b_grp + (int64_t)n0 * K, rows_b * K);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);

    // LDS rows are 128 bytes (one stage of K); the 16-byte chunk index is
    // XOR-swizzled with (row >> 1) & 7.  The LDS serves a ds_read_b128 16
    // lanes per cycle from 64 banks; the 16 lanes of a fragment read take 16
    // consecutive rows at one logical chunk, and with the swizzle row parity
    // and physical chunk together name 16 different 16-byte bank groups.
    //
    // global -> LDS: each wave moves 8-row groups 8 w + j (j = 0..7) of A
    // and 2 NB w + j (j < 2 NB) of B with one 1 KB LDS-DMA load each; every
    // row of a group is one whole 128-byte line of the operand.  Lane l
    // lands at byte 16 l of the group -- row l >> 3, physical chunk l & 7 --
    // so it fetches logical chunk (l & 7) ^ ((row >> 1) & 7), which is
    // (l & 7) ^ (l >> 4) in even groups and that ^ 4 in odd ones.
    const int lc_e = (lane & 7) ^ (lane >> 4), lc_o = lc_e ^ 4;
    const int row_off = (64 * wave + (lane >> 3)) * K;
    const int b_row_off = (16 * NB * wave + (lane >> 3)) * K;
    const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
    // LDS -> fragments: for K step ks (0, 1) of a stage, lane reads row
    // (lane & 31), logical chunks 4 ks + 2 h and 4 ks + 2 h + 1 into
    // registers 0-3 and 4-7.  MXFP8 reads chunks 4 ks + h and 4 ks + 2 + h
    // instead: the scaled MFMA applies one block scale to registers 0-3 of
    // both lane halves and another to registers 4-7 (the scale of the first
    // comes from lanes 0-31, of the second from lanes 32-63), so each of
    // those register groups must hold one whole 32-element block.
    const int fr = lane & 31, h = lane >> 5, sw = (fr >> 1) & 7;
    int rd[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int ch = QT == kMxE4M3 ? 4 * ks + h + 2 * e : 4 * ks + 2 * h + e;
            rd[ks][e] = fr * PK + ((ch ^ sw) << 4);
        }
    const int a_rd = wm * 128 * PK;
    const int b_rd = PA + wn * WNC * PK;
    const int KT = (K + SK - 1) / SK;

    typedef typename PipeAcc<QT>::type acc_t;
    acc_t acc[4][NB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

    // Load of group j (0..7) of A (ab = 0) or B (ab = 1) of stage kt into
    // LDS buffer kt & 1.  Loads past the end of K (the K tail and the
    // padding stages up to an even count) get bit 31 set in their offset:
    // out of range, they write zeros.
    auto dma = [&](int kt, int ab, int j) {
        const int k0 = kt * SK;
        const int lc = (j & 1) ? lc_o : lc_e;
        const bool oob = k0 + lc * 16 >= K;
        const int off = ((ab ? b_row_off : row_off) + j * 8 * K + k0 + lc * 16) | (int)((unsigned)oob << 31);
        const int grp = ab ? 2 * NB * wave_u + j : 8 * wave_u + j;
        const uint32_t dst = lds_base + (uint32_t)((kt & 1) * PSTAGE + ab * PA + grp * 1024);
        lds_dma16(ab ? rb : ra, off, dst);
    };
    // the stage's loads in issue order: A and B groups alternating, then the
    // rest of A (8 + 2 NB loads per wave)
    constexpr int kLoads = 8 + 2 * NB;
    auto dma_nth = [&](int kt, int t) {
        if (t < 4 * NB)
            dma(kt, t & 1, t >> 1);
        else
            dma(kt, 0, t - 2 * NB);
    };
    // fragments of one K step: B of the NB column tiles, A of the 4 row tiles
    struct Frags {
        v8i b[NB], a[4];
    };
    // half e of fragment q (B tiles 0..NB-1, then A tiles 0..3) of K step ks
    auto read_part = [&](int buf, int ks, Frags& f, int q, int e) {
        const uint8_t* s = smem + buf * PSTAGE + (q < NB ? b_rd + q * 32 * PK : a_rd + (q - NB) * 32 * PK);
        const v4i v = *reinterpret_cast<const v4i*>(s + rd[ks][e]);
        v8i& d = q < NB ? f.b[q] : f.a[q - NB];
#pragma unroll
        for (int i = 0; i < 4; ++i) d[4 * e + i] = v[i];
    };
    // the fragment reads that go with MFMA i (of 4 NB) of a K step: the
    // 2 (NB + 4) 16-byte halves spread evenly (one each for NB = 4)
    constexpr int kMfmas = 4 * NB, kHalves = 2 * (NB + 4);
    auto read_slots = [&](int buf, int ks, Frags& f, int i) {
        // fragment order A0, B0..B(NB-1), A1..A3: the order the next K
        // step's MFMAs first use them
        auto ord = [](int k) { return k == 0 ? NB : (k <= NB ? k - 1 : k); };
#pragma unroll
        for (int hh = kHalves * i / kMfmas; hh < kHalves * (i + 1) / kMfmas; ++hh)
            read_part(buf, ks, f, ord(hh >> 1), hh & 1);
    };
    // weights as the first operand: the 32x32 result is the transposed
    // output tile, so each lane ends up with 4 consecutive columns
    // MXFP8: the block scales of K step ks are blocks 2 ks (registers 0-3,
    // taken from lanes 0-31) and 2 ks + 1 (registers 4-7, from lanes 32-63):
    // lane half h passes the scale of block 2 ks + h of its row.  A scale
    // word holds the group's blocks in the byte order 0, 2, 1, 3, so lane
    // half h reads the 16 bits at byte 2 h -- blocks h and 2 + h -- and the
    // MFMA's byte select is ks for every lane (operand order as the data).
    constexpr bool MX = QT == kMxE4M3 || FP4 || FP6;
    // MFMA operand format: 0 E4M3, 2 E2M3, 3 E3M2 (4 E2M1 in the MXFP4 loop)
    constexpr int FMT = QT == kMxE2M3 ? 2 : QT == kMxE3M2 ? 3 : 0;
    int scA[2][4], scB[2][4];
    auto mfma_one = [&](int mi, int ni, const Frags& f, int set = 0, int ks = 0) {
        if constexpr (QT == kE4M3FN) {
            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                f.b[ni], f.a[mi], acc[mi][ni], 0, 0, 0, 0, 0, 0);
        } else if constexpr (MX) {
            if (ks == 0)
                acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    f.b[ni], f.a[mi], acc[mi][ni], FMT, FMT, 0, scB[set][ni], 0, scA[set][mi]);
            else
                acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    f.b[ni], f.a[mi], acc[mi][ni], FMT, FMT, 1, scB[set][ni], 1, scA[set][mi]);
        } else {
            const v8i b8 = f.b[ni], a8 = f.a[mi];
            acc[mi][ni] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                v4i{b8[0], b8[1], b8[2], b8[3]}, v4i{a8[0], a8[1], a8[2], a8[3]}, acc[mi][ni],
                0, 0, 0);
            acc[mi][ni] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                v4i{b8[4], b8[5], b8[6], b8[7]}, v4i{a8[4], a8[5], a8[6], a8[7]}, acc[mi][ni],
                0, 0, 0);
        }
    };
    // MXFP8 scale loads of stage kt: the scale words of a 128-wide K group
    // are stored group-major, so a tile's 256 row words of one stage are 1 KB
    // in one piece (lane l loads rows 4 l .. 4 l + 3).  Rows past the end of
    // A or B read the next group's words (finite scales of zero data, in
    // outputs that are never stored) or zeros past the tensor: the buffer's
    // range check takes each dword of a 16-byte load on its own, so a lane
    // that straddles the end still gets its in-range words (the row scales
    // of a ragged last tile rely on the same).
    // (MXFP4: a stage takes the words of groups 2 kt and 2 kt + 1, 4 KB per
    // ring slot: A and B of the first group, then of the second)
    const int KG = p.k / 128;  // 128-element scale groups
    const v4i rea = MX ? buffer_rsrc(p.ea + m0, (KG * p.m - m0) * 4) : v4i{};
    const v4i reb = MX ? buffer_rsrc(p.eb + n0, (KG * p.n - n0) * 4) : v4i{};
    auto dma_mx = [&](int kt) {
        // one 16-byte-per-lane load moves a whole 1 KB row of a stage's
        // scale words, one load per wave and stage (against two or four
        // 4-byte loads: MXFP4 2.5% faster, MXFP8/6 under 1%).  MXFP4 has
        // four rows per stage (A and B of its two groups), wave w loads row
        // w.  MXFP8/6 have two: waves 0 and 2 load A's, 1 and 3 B's, the
        // same bytes to the same place twice (a branch on the wave made the
        // compiler spill in the loop)
        constexpr int GPS = FP4 ? 2 : 1;
        const int gi = FP4 ? wave_u >> 1 : 0;
        const int ab = wave_u & 1;
        const int grp = kt * GPS + gi;
        const uint32_t dst =
            lds_base + PMXS + (kt & (PMXRING - 1)) * (2048 * GPS) + gi * 2048 + ab * 1024;
        const int off = grp >= KG ? (int)0x80000000u : grp * (ab ? p.n : p.m) * 4 + lane * 16;
        lds_dma16(ab ? reb : rea, off, dst);
    };
    // (straight from LDS into the MFMA's scale operand: no VALU work, so the
    // reads need not complete before the MFMAs that do not use them)
    auto read_mx = [&](int kt, int set) {
        const uint16_t* sm =
            reinterpret_cast<const uint16_t*>(smem + PMXS + (kt & (PMXRING - 1)) * 2048);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            scA[set][i] = sm[2 * (wm * 128 + i * 32 + fr) + h];
            scB[set][i] = sm[2 * (256 + wn * 128 + i * 32 + fr) + h];
        }
    };
    // MXFP4: the scale halves of both groups of a stage (group g = ks / 2 for
    // K step ks; lane half h holds blocks h and 2 + h of the group, the
    // MFMA's byte select is ks & 1)
    int s4A[2][2][4], s4B[2][2][4];
    auto read_mx4 = [&](int kt, int set) {
        const uint16_t* sm =
            reinterpret_cast<const uint16_t*>(smem + PMXS + (kt & (PMXRING - 1)) * 4096);
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s4A[set][g][i] = sm[1024 * g + 2 * (wm * 128 + i * 32 + fr) + h];
                s4B[set][g][i] = sm[1024 * g + 2 * (256 + wn * 128 + i * 32 + fr) + h];
            }
    };
#define TFQ_FENCE() __builtin_amdgcn_sched_barrier(0)

    // Stage s (128 bytes of K) lives in LDS buffer s & 1 and is computed as
    // two K steps of 16 MFMAs.  One barrier per stage, between its K steps:
    // by then every wave has read all of stage s's fragments (the second K
    // step's were read during the first) and has received its own loads of
    // stage s + 1, so buffer s & 1 is free and stage s + 1 complete.  The
    // second K step then reads stage s + 1's first fragments, one 16-byte
    // read after each MFMA, and issues the 16 loads of stage s + 2 into the
    // freed buffer, one after each MFMA: a stage's 64 KB per CU spread over
    // the K step rather than in a burst, which filled the address FIFO and
    // stalled the wave's in-order issue, MFMAs included (6-7% faster).  The
    // loop runs an even number of stages (a stage past K reads zeros).
    //
    // MXFP8 scale words ride along, two 4-byte loads per wave per stage into
    // a 2-slot ring: stage s + 2's go out first in the second K step of
    // stage s (into the slot of stage s, whose words every wave has read
    // before the barrier of stage s).  Issued ahead of the data loads they
    // measured faster than behind them.
    Frags f0, f1;
    // waves 0, 1, 2 fetch the tile's row scales, column scales and bias into
    // LDS (past the end: zeros); issued first, so the prologue's wait covers them
    if (wave_u == 0 && !MX) {
        lds_dma16(buffer_rsrc(p.sa + m0, rows_a * 4), lane * 16, lds_base + SCL);
    } else if (wave_u == 1 && !MX) {
        lds_dma16(buffer_rsrc(sb_grp + n0, rows_b * 4), lane * 16, lds_base + SCL + 1024);
    } else if (wave_u == 2 && bias_grp != nullptr) {
        lds_dma16(buffer_rsrc(bias_grp + n0, rows_b * 2), lane * 16, lds_base + SCL + 2048);
    }
    if constexpr (!FP6) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int t = 0; t < kLoads; ++t) dma_nth(u, t);
            if constexpr (MX) dma_mx(u);
        }
    }
    if constexpr (FP4) {
        // MXFP4: a stage is four K steps of 64 elements.  In K step ks lane
        // half h holds row (lane & 31)'s 16-byte chunk 2 ks + h -- one whole
        // 32-element block, whose scale the lane passes (the MFMA reads
        // registers 0-3 of each lane for E2M1).  K step j computes from
        // fragment set g_j.  K step 0 reads step 1's fragments, step 1 reads
        // steps 2 and 3's (one 16-byte read after each MFMA), so the
        // stage's barrier comes before its third K step: steps 2 and 3 then
        // issue the next stage's 16 loads, one after every other MFMA, and
        // step 2 reads the next stage's first fragments.  (Measured 2% faster
        // than a barrier before the last step with the loads all in it.)
        struct Frags4 {
            v4i b[4], a[4];
        };
        int rd4[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) rd4[ks] = fr * PK + (((2 * ks + h) ^ sw) << 4);
        auto read4 = [&](int buf, int ks, Frags4& f, int q) {
            const uint8_t* sp =
                smem + buf * PSTAGE + (q < 4 ? b_rd + q * 32 * PK : a_rd + (q - 4) * 32 * PK);
            const v4i v = *reinterpret_cast<const v4i*>(sp + rd4[ks]);
            if (q < 4)
                f.b[q] = v;
            else
                f.a[q - 4] = v;
        };
        auto mfma4 = [&](int mi, int ni, const Frags4& f, int set, int ks) {
            const v8i bb = __builtin_shufflevector(f.b[ni], f.b[ni], 0, 1, 2, 3, -1, -1, -1, -1);
            const v8i aa = __builtin_shufflevector(f.a[mi], f.a[mi], 0, 1, 2, 3, -1, -1, -1, -1);
            const int g = ks >> 1;
            if ((ks & 1) == 0)
                acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    bb, aa, acc[mi][ni], 4, 4, 0, s4B[set][g][ni], 0, s4A[set][g][mi]);
            else
                acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    bb, aa, acc[mi][ni], 4, 4, 1, s4B[set][g][ni], 1, s4A[set][g][mi]);
        };
        Frags4 g0, g1, g2, g3;
        // stage 0 complete: stage 1's 16 data loads and 1 scale load may
        // still be in flight
        asm volatile("s_waitcnt vmcnt(17)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int q = 0; q < 8; ++q) read4(0, 0, g0, q);
        read_mx4(0, 0);
        for (int kt = 0; kt < KT; kt += 2) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    mfma4(i >> 2, i & 3, g0, u, 0);
                    TFQ_FENCE();
                    if ((i & 1) == 0) read4(u, 1, g1, i >> 1);
                    TFQ_FENCE();
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    mfma4(i >> 2, i & 3, g1, u, 1);
                    TFQ_FENCE();
                    if ((i & 1) == 0)
                        read4(u, 2, g2, i >> 1);
                    else
                        read4(u, 3, g3, i >> 1);
                    TFQ_FENCE();
                }
                // own loads of stage kt+u+1 are done; every wave has read all
                // of stage kt+u
                asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                read_mx4(kt + u + 1, u ^ 1);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    mfma4(i >> 2, i & 3, g2, u, 2);
                    TFQ_FENCE();
                    if ((i & 1) == 0) read4(u ^ 1, 0, g0, i >> 1);
                    if (i == 0) dma_mx(kt + u + 2);
                    if ((i & 1) == 1) dma(kt + u + 2, 0, i >> 1);
                    TFQ_FENCE();
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    mfma4(i >> 2, i & 3, g3, u, 3);
                    TFQ_FENCE();
                    if ((i & 1) == 1) dma(kt + u + 2, 1, i >> 1);
                    TFQ_FENCE();
                }
            }
        }
    } else if constexpr (FP6) {
        // MXFP6: the rows of a stage (128 elements, 96 bytes) lie back to back
        // in LDS, 24 KB per operand and stage, so three stages fit
        // and the loads run two stages ahead (stage s + 3 goes out in stage
        // s's second K step; the barrier of stage s waits for stage s + 1
        // only).  The codes are stored group-major, so a stage of the tile's
        // rows is one contiguous 24 KB panel in memory too: loads read whole
        // cache lines (row-major 96-byte row pieces straddle 128-byte lines
        // and cost the loads about 16% more time).  Load i of wave w moves
        // chunks L = 64 (6 w + i) + lane of an operand's 1536 16-byte chunks
        // (row L / 6, slot L % 6), landing contiguously as LDS-DMA writes them.  Row r keeps its six chunks
        // rotated by (r >> 3) & 3 slots: rows 8 apart start 768 bytes apart
        // (the same banks), and the rotation spreads the 8-byte fragment
        // reads of a 32-row tile over the banks.  In K step ks lane half h
        // reads the 24 bytes at row byte 48 ks + 24 h (one 32-element block)
        // as three 8-byte pieces into registers 0-5.
        // per-lane byte offsets of the pieces (wave's rows and the lane's
        // row, rotated chunk and byte) for A and B; the stage and the 32-row
        // tile add constants below 64 KB, so every read takes an immediate
        const int rot6 = (fr >> 3) & 3;
        int r6a[2][3], r6b[2][3];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int pc = 0; pc < 3; ++pc) {
                const int bo = 48 * ks + 24 * h + 8 * pc;
                int ph = (bo >> 4) + rot6;
                ph -= ph >= 6 ? 6 : 0;
                const int r = fr * 96 + ph * 16 + (bo & 15);
                r6a[ks][pc] = wm * 128 * 96 + r;
                r6b[ks][pc] = P6B + wn * WNC * 96 + r;
            }
        auto read6p = [&](int buf, int ks, Frags& f, int q, int pc) {
            const uint8_t* sp = q < NB ? smem + r6b[ks][pc] + buf * P6OP + q * 32 * 96
                                       : smem + r6a[ks][pc] + buf * P6OP + (q - NB) * 32 * 96;
            const v2i vv = *reinterpret_cast<const v2i*>(sp);
            v8i& d = q < NB ? f.b[q] : f.a[q - NB];
            d[2 * pc] = vv[0];
            d[2 * pc + 1] = vv[1];
        };
        // the 3 (NB + 4) pieces of a K step spread over its MFMAs, in the
        // order the next K step's MFMAs first use the fragments
        auto slots6 = [&](int buf, int ks, Frags& f, int i) {
            auto ord = [](int k) { return k == 0 ? NB : (k <= NB ? k - 1 : k); };
            constexpr int kPieces = 3 * (NB + 4);
#pragma unroll
            for (int sl = kPieces * i / kMfmas; sl < kPieces * (i + 1) / kMfmas; ++sl)
                read6p(buf, ks, f, ord(sl / 3), sl % 3);
        };
        // load i (0..5) of operand ab (0 A, 1 B) of stage kt into buffer
        // buf; the lane's row and source chunk of each load are fixed
        int src6[6];
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            const int L = (6 * wave_u + i) * 64 + lane_id_here();
            const int row = L / 6, c = L - row * 6;
            int g = c - ((row >> 3) & 3);
            g += g < 0 ? 6 : 0;
            src6[i] = row * 96 + 16 * g;
        }
        // the tile's rows of stage kt (past the end of K or of the operand's
        // rows: zeros)
        auto panel6 = [&](int ab, int kt) {
            const int64_t first = (int64_t)kt * (ab ? p.n : p.m) + (ab ? n0 : m0);
            return buffer_rsrc((ab ? p.b : p.a) + first * 96, kt < KT ? (ab ? rows_b : rows_a) * 96 : 0);
        };
        auto dma6 = [&](int kt, int buf, int ab, int i) {
            lds_dma16(panel6(ab, kt), src6[i],
                      lds_base + (uint32_t)(ab * P6B + buf * P6OP + (6 * wave_u + i) * 1024));
        };
        constexpr int kLoads6 = 12;  // per wave and stage (plus one scale load)
        auto dma6_nth = [&](int kt, int buf, int tt) { dma6(kt, buf, tt & 1, tt >> 1); };
        // E8M0 scale words of stage kt into ring slot kt % 4 (as dma_mx)
        auto dma_mx6 = [&](int kt) {
            const int ab = wave_u & 1;
            const uint32_t dst = lds_base + P6MXS + (kt & 3) * 2048 + ab * 1024;
            const int off = (kt * (ab ? p.n : p.m) * 4 + lane * 16) | (int)((unsigned)(kt >= KG) << 31);
            lds_dma16(ab ? reb : rea, off, dst);
        };
        auto read_mx6 = [&](int kt, int set) {
            const uint16_t* sm = reinterpret_cast<const uint16_t*>(smem + P6MXS + (kt & 3) * 2048);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                scA[set][i] = sm[2 * (wm * 128 + i * 32 + fr) + h];
                scB[set][i] = sm[2 * (256 + wn * 128 + i * 32 + fr) + h];
            }
        };
        // stages 0, 1, 2; then stage 0 complete (stages 1 and 2 may be in flight)
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            dma_mx6(u);
#pragma unroll
            for (int tt = 0; tt < kLoads6; ++tt) dma6_nth(u, u, tt);
        }
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * (kLoads6 + 1)) : "memory");
#pragma unroll
        for (int i = 0; i < kMfmas; ++i) slots6(0, 0, f0, i);
        read_mx6(0, 0);
        // stage s in buffer BUF = s % 3; the current stage's scales in set 0
        auto stage6 = [&](int st, auto bufc) {
            constexpr int BUF = decltype(bufc)::value;
            constexpr int NBUF = BUF == 2 ? 0 : BUF + 1;
#pragma unroll
            for (int i = 0; i < kMfmas; ++i) {
                mfma_one(i / NB, i % NB, f0, 0, 0);
                TFQ_FENCE();
                slots6(BUF, 1, f1, i);
                TFQ_FENCE();
            }
            // stage st + 1 has arrived (stage st + 2's loads may still be in
            // flight) and every wave has read all of stage st
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(kLoads6 + 1)
                         : "memory");
            read_mx6(st + 1, 1);
#pragma unroll
            for (int i = 0; i < kMfmas; ++i) {
                mfma_one(i / NB, i % NB, f1, 0, 1);
                TFQ_FENCE();
                slots6(NBUF, 0, f0, i);
                if (i == 0) dma_mx6(st + 3);
#pragma unroll
                for (int tt = kLoads6 * i / kMfmas; tt < kLoads6 * (i + 1) / kMfmas; ++tt)
                    dma6_nth(st + 3, BUF, tt);
                TFQ_FENCE();
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                scA[0][i] = scA[1][i];
                scB[0][i] = scB[1][i];
            }
        };
        int st = 0;
        for (; st + 3 <= KT; st += 3) {
            stage6(st, std::integral_constant<int, 0>());
            stage6(st + 1, std::integral_constant<int, 1>());
            stage6(st + 2, std::integral_constant<int, 2>());
        }
        if (st < KT) stage6(st, std::integral_constant<int, 0>());
        if (st + 1 < KT) stage6(st + 1, std::integral_constant<int, 1>());
    } else {
        // stage 0 complete: the loads of stage 1 (8 + 2 NB, plus 1 scale load
        // for MXFP8) may still be in flight
        if constexpr (MX)
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kLoads + 1) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kLoads) : "memory");
    #pragma unroll
        for (int i = 0; i < kMfmas; ++i) read_slots(0, 0, f0, i);
        if constexpr (MX) read_mx(0, 0);

        for (int kt = 0; kt < KT; kt += 2) {
    #pragma unroll
            for (int u = 0; u < 2; ++u) {
                // K step 0 of stage kt+u from f0; K step 1's fragments into f1
    #pragma unroll
                for (int i = 0; i < kMfmas; ++i) {
                    mfma_one(i / NB, i % NB, f0, u, 0);
                    TFQ_FENCE();
                    read_slots(u, 1, f1, i);
                    TFQ_FENCE();
                }
                // own loads of stage kt+u+1 (the only ones in flight) are done
                asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                // K step 1 from f1; stage kt+u+1's first fragments into f0 and
                // the loads of stage kt+u+2
                if constexpr (MX) read_mx(kt + u + 1, u ^ 1);
    #pragma unroll
                for (int i = 0; i < kMfmas; ++i) {
                    mfma_one(i / NB, i % NB, f1, u, 1);
                    TFQ_FENCE();
                    read_slots(u ^ 1, 0, f0, i);
                    if constexpr (MX)
                        if (i == 0) dma_mx(kt + u + 2);
    #pragma unroll
                    for (int t = kLoads * i / kMfmas; t < kLoads * (i + 1) / kMfmas; ++t)
                        dma_nth(kt + u + 2, t);
                    TFQ_FENCE();
                }
            }
        }
    }
#undef TFQ_FENCE
    // the loads of the padding stages past the loop are still in flight
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- epilogue ----
    // With the weights as the first MFMA operand, lane (fr, h) holds, for row
    // tile mi and column tile ni, output row  wm*128 + mi*32 + fr  and the
    // four consecutive output columns  wn*128 + ni*32 + 8q + 4h + (0..3)  in
    // registers 4q..4q+3 (q = 0..3).
    const float* lds_sa = reinterpret_cast<const float*>(smem + SCL);
    const float* lds_sb = reinterpret_cast<const float*>(smem + SCL + 1024);
    const uint16_t* lds_bias = reinterpret_cast<const uint16_t*>(smem + SCL + 2048);
    // (MXFP8: the sums are already scaled; no row or column scales)
    float srow[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) srow[mi] = MX ? 1.0f : lds_sa[wm * 128 + mi * 32 + fr];
    if constexpr (WANT_ACC) {
        // raw INT32 sums: 16-byte stores of 4 consecutive columns
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int row = m0 + wm * 128 + mi * 32 + fr;
            if (row >= m_end) continue;
#pragma unroll
            for (int ni = 0; ni < NB; ++ni)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c0 = n0 + wn * WNC + ni * 32 + 8 * q + 4 * h;
                    if (c0 < p.n)
                        *reinterpret_cast<v4i*>(p.acc + (int64_t)row * p.n + c0) =
                            v4i{(int)acc[mi][ni][4 * q], (int)acc[mi][ni][4 * q + 1],
                                (int)acc[mi][ni][4 * q + 2], (int)acc[mi][ni][4 * q + 3]};
                }
        }
    }
    if constexpr (WANT_Y) {
        // BF16 results are staged per wave in LDS (128 rows x 256 bytes, rows
        // padded to 272 bytes) and written back as whole 256-byte row segments
        // with 16-byte stores.
        lds_barrier();  // every wave is done with the pipeline buffers
        uint8_t* stg = smem + wave * 128 * EPITCH;
        // The column scales and bias values of a column tile are read from LDS
        // together, with one wait, so that the arithmetic is not broken up by
        // waits (LDS operations complete in order: a wait for a read also
        // waits for the staging writes issued before it).  The loop is built
        // twice, with and without the bias add, and a uniform branch picks one
        // (without a bias there is nothing to read or add).
        auto stage_out = [&](auto with_bias) {
            constexpr bool HB = decltype(with_bias)::value;
#pragma unroll
            for (int ni = 0; ni < NB; ++ni) {
                v4f sc[4];
                uint2 braw[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int lc0 = wn * WNC + ni * 32 + 8 * q + 4 * h;
                    if constexpr (!MX) sc[q] = *reinterpret_cast<const v4f*>(lds_sb + lc0);
                    if constexpr (HB) braw[q] = *reinterpret_cast<const uint2*>(lds_bias + lc0);
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float bc[4] = {};
                    if constexpr (HB) {
                        bc[0] = __uint_as_float(braw[q].x << 16);
                        bc[1] = __uint_as_float(braw[q].x & 0xffff0000u);
                        bc[2] = __uint_as_float(braw[q].y << 16);
                        bc[3] = __uint_as_float(braw[q].y & 0xffff0000u);
                    }
#pragma unroll
                    for (int mi = 0; mi < 4; ++mi) {
                        float v[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            if constexpr (MX)
                                v[j] = acc[mi][ni][4 * q + j];
                            else
                                v[j] = scale_out((float)acc[mi][ni][4 * q + j], srow[mi], sc[q][j]);
                            if constexpr (HB) v[j] = add_bias(v[j], bc[j]);
                            if constexpr (EPI == 1) v[j] = gelu_tanh(v[j]);
                        }
                        *reinterpret_cast<uint2*>(stg + (mi * 32 + fr) * EPITCH + (ni * 32 + 8 * q + 4 * h) * 2) =
                            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                    }
                }
            }
        };
        if (bias_grp != nullptr)
            stage_out(std::true_type{});
        else
            stage_out(std::false_type{});
        // the wave reads back only what it wrote itself: 128 rows of 4 NB
        // 16-byte chunks (WNC columns)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        constexpr int CPR = 4 * NB;
#pragma unroll
        for (int j = 0; j < 2 * CPR; ++j) {
            const int idx = j * 64 + lane;
            const int lrow = idx / CPR, ch = idx - lrow * CPR;
            const v4u d = *reinterpret_cast<const v4u*>(stg + lrow * EPITCH + ch * 16);
            const int grow = m0 + wm * 128 + lrow;
            const int gcol = n0 + wn * WNC + ch * 8;
            if (grow < m_end && gcol < p.n)
                *reinterpret_cast<v4u*>(p.y + (int64_t)grow * p.n + gcol) = d;
        }
    }
}

// ---------------------------------------------------------------------------
// Block-scaled FP8 kernel: 1x128 activation groups and 128x128 weight blocks
// (LightX2V "模型量化技术", table "量化模式", fp8-b128-deepgemm).  256x128
// output tile, 8 waves (4x2) of 64x64, two per SIMD: every wave's 64 columns
// lie in one 128-wide weight block and -- with the weights as the first MFMA
// operand -- every lane's output row is fixed per 32-row tile, so the scale
// of a (row, K-block) pair is one float per row tile.  One stage is one
// 128-deep K block (two K steps of MFMAs into a temporary); the next block's
// first K step folds it in, acc += temp * (s_a[row, kb] * s_b[nb, kb]), just
// before each tile's first MFMA.  A wave's sums and temporaries (2 x 64
// registers) both stay in VGPRs, so the fold is one FMA per element, and the
// two waves of a SIMD hide each other's fold, barrier and memory waits.
// Operands go straight into LDS (LDS-DMA loads, whole 128-byte lines), 3
// LDS buffers, loads 3 stages ahead, one barrier per stage; the row scales
// of each block come with the stage (4-byte LDS-DMA loads), the weight
// block's scales once per tile.
// ---------------------------------------------------------------------------
constexpr int QK = 64;                     // K bytes per stage
constexpr int QA = BM * QK;                // 16 KB of A per stage
constexpr int QBN = 128;                   // output columns per workgroup
constexpr int QSTAGE = QA + QBN * QK;      // 24 KB per LDS buffer
constexpr int QEPITCH = 144;               // staged output row: 64 columns * 2 B + 16
constexpr int DSMEM = (3 * QSTAGE > 4 * 128 * QEPITCH) ? 3 * QSTAGE : 4 * 128 * QEPITCH;
constexpr int XB_A = BM * 128;                 // 32 KB of A per stage
constexpr int XB_STAGE = XB_A + QBN * 128;      // 48 KB per LDS buffer
constexpr int XB_BUF = 3;
constexpr int XB_SA = XB_BUF * XB_STAGE;        // row-scale ring: 3 x 1 KB
constexpr int XB_BIAS = XB_SA + XB_BUF * 1024;  // the tile's 128 BF16 bias values
constexpr int XB_SB = XB_BIAS + 256;            // the weight block's scales, K/128 <= 1024
constexpr int XB_SMEM = XB_SB + 4096;


template <int EPI>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void gemm_block_kernel(const Params p)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[XB_SMEM];

    const int wave_u = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int wm = wave_u & 3, wn = wave_u >> 2;  // rows wm*64 .. +63, columns wn*64 .. +63
    const int lane = lane_id_here();
    int tm, tn;
    map_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * QBN;
    const int K = p.k;
    const int KT = K >> 7;  // K blocks = stages (K % 128 == 0)
    const int rows_a = min(BM, p.m - m0), rows_b = min(QBN, p.n - n0);
    const v4i ra = buffer_rsrc(p.a + (int64_t)m0 * K, rows_a * K);
    const v4i rb = buffer_rsrc(p.b + (int64_t)n0 * K, rows_b * K);
    const v4i rsa = buffer_rsrc(p.sa + (int64_t)m0 * KT, rows_a * KT * 4);
    const uint32_t lds_base = (uint32_t)(uintptr_t)smem;

    // global -> LDS: wave w moves 8-row groups 4 w + j (j < 4) of A and
    // 2 w + j (j < 2) of B per stage, one 1 KB LDS-DMA load each; lane l
    // lands at row l >> 3, physical chunk l & 7 of its group and fetches
    // logical chunk (l & 7) ^ ((row >> 1) & 7) (the LDS swizzle for 128-byte
    // rows), which is (l & 7) ^ (l >> 4) in even groups and that ^ 4 in odd.
    const int lc_e = (lane & 7) ^ (lane >> 4), lc_o = lc_e ^ 4;
    const int a_off = (32 * wave_u + (lane >> 3)) * K;
    const int b_off = (16 * wave_u + (lane >> 3)) * K;
    // the row scales of block kb: waves w and w + 4 both fetch rows
    // 64 (w & 3) + lane (the same bytes to the same LDS place), so every wave
    // issues the same number of loads per stage
    const int sa_off = (64 * (wave_u & 3) + lane) * KT * 4;
    // load d (0..6) of stage kt into LDS buffer bf: 4 of A, 2 of B, row scales
    auto dma_op = [&](int kt, int bf, int d) {
        const int k0 = kt * 128;
        const uint32_t dst = lds_base + (uint32_t)(bf * XB_STAGE);
        if (d < 6) {
            const int j = d < 4 ? d : d - 4;
            const int lc = (j & 1) ? lc_o : lc_e;
            const int oob = (int)((unsigned)(k0 + lc * 16 >= K) << 31);
            if (d < 4)
                lds_dma16(ra, (a_off + j * 8 * K + k0 + lc * 16) | oob, dst + (4 * wave_u + j) * 1024);
            else
                lds_dma16(rb, (b_off + j * 8 * K + k0 + lc * 16) | oob,
                          dst + XB_A + (2 * wave_u + j) * 1024);
        } else {
            lds_dma4(rsa, (sa_off + kt * 4) | (int)((unsigned)(kt >= KT) << 31),
                     lds_base + XB_SA + bf * 1024 + (wave_u & 3) * 256);
        }
    };

    // LDS -> fragments: K step ks (0, 1) of a stage, lane reads row
    // (lane & 31), logical chunks 4 ks + 2 h and 4 ks + 2 h + 1
    const int fr = lane & 31, h = lane >> 5, sw = (fr >> 1) & 7;
    int rd[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 2; ++e) rd[ks][e] = fr * 128 + (((4 * ks + 2 * h + e) ^ sw) << 4);
    const int a_rd = wm * 64 * 128;
    const int b_rd = XB_A + wn * 64 * 128;
    struct Frags {
        v8i b[2], a[2];
    };
    // fragment q (B tiles 0, 1, then A tiles 0, 1) of K step ks, both halves
    auto read_frag = [&](int buf, int ks, Frags& f, int q) {
        const uint8_t* s = smem + buf * XB_STAGE + (q < 2 ? b_rd + q * 32 * 128 : a_rd + (q - 2) * 32 * 128);
        v8i& d = q < 2 ? f.b[q] : f.a[q - 2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const v4i v = *reinterpret_cast<const v4i*>(s + rd[ks][e]);
#pragma unroll
            for (int i = 0; i < 4; ++i) d[4 * e + i] = v[i];
        }
    };
    // fragments in the order the K step's MFMAs first use them: A0, B0, B1, A1
    constexpr int ord[4] = {2, 0, 1, 3};

    v16f acc[2][2], tmp[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    float f_prev[2] = {0.0f, 0.0f};  // block scale factors of the previous stage

    // prologue: bias and the weight block's scales of every K block (wave
    // 7; the tile's 128 columns are one weight block), stages 0, 1, 2
    if (wave_u == 7) {
        if (p.bias != nullptr) lds_dma4(buffer_rsrc(p.bias + n0, rows_b * 2), lane * 4, lds_base + XB_BIAS);
        const v4i rsb = buffer_rsrc(p.sb + (int64_t)(n0 >> 7) * KT, KT * 4);
        for (int c = 0; c < KT; c += 64) lds_dma4(rsb, (c + lane) * 4, lds_base + XB_SB + c * 4);
    }
#pragma unroll
    for (int st = 0; st < 3; ++st)
#pragma unroll
        for (int d = 0; d < 7; ++d) dma_op(st, st, d);
    // bias, block scales and stage 0 complete: 14 loads (stages 1, 2) may be in flight
    asm volatile("s_waitcnt vmcnt(14)\n\ts_barrier" ::: "memory");
    Frags f0, f1;
#pragma unroll
    for (int q = 0; q < 4; ++q) read_frag(0, 0, f0, ord[q]);

    auto mfma = [&](const v16f& c, const Frags& f, int mi, int ni) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[ni], f.a[mi], c, 0, 0, 0, 0, 0, 0);
    };

#define TFQ_FENCE() __builtin_amdgcn_sched_barrier(0)
    // Stage kt lives in LDS buffer kt % 3.  Its barrier sits between its two
    // K steps: by then every wave has read all of its fragments and row
    // scales and has received its own loads of stage kt + 1 (loads issued
    // after those: the 7 of stage kt + 2), so the buffer is free for stage
    // kt + 3, whose loads go out during the second K step together with the
    // reads of stage kt + 1's first fragments.
    int buf = 0;
    for (int kt = 0; kt < KT; ++kt) {
        const int nbuf = buf == XB_BUF - 1 ? 0 : buf + 1;
        const float sbv = reinterpret_cast<const float*>(smem + XB_SB)[kt];
        const float* sa_l = reinterpret_cast<const float*>(smem + XB_SA + buf * 1024);
        float f_cur[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) f_cur[mi] = sa_l[wm * 64 + mi * 32 + fr];
        // K step 0: fold the previous block's temporary of each tile into acc
        // just before the tile's first MFMA of this block; K step 1's
        // fragments into f1, one after each MFMA
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int mi = i >> 1, ni = i & 1;
            if (kt > 0) {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    acc[mi][ni][e] = __builtin_fmaf(tmp[mi][ni][e], f_prev[mi], acc[mi][ni][e]);
            }
            tmp[mi][ni] = mfma(v16f{}, f0, mi, ni);
            TFQ_FENCE();
            read_frag(buf, 1, f1, ord[i]);
            TFQ_FENCE();
        }
        asm volatile("s_waitcnt vmcnt(7)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // K step 1; stage kt+1's K step 0 fragments into f0; stage kt+3's loads
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int mi = i >> 1, ni = i & 1;
            tmp[mi][ni] = mfma(tmp[mi][ni], f1, mi, ni);
            TFQ_FENCE();
            read_frag(nbuf, 0, f0, ord[i]);
#pragma unroll
            for (int d = (7 * i) / 4; d < (7 * (i + 1)) / 4; ++d) dma_op(kt + 3, buf, d);
            TFQ_FENCE();
        }
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) f_prev[mi] = f_cur[mi] * sbv;
        buf = nbuf;
    }
#undef TFQ_FENCE
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[mi][ni][e] = __builtin_fmaf(tmp[mi][ni][e], f_prev[mi], acc[mi][ni][e]);

    // ---- epilogue: lane holds row wm*64 + mi*32 + fr and columns
    // wn*64 + ni*32 + 8q + 4h + (0..3) in registers 4q..4q+3.  Bias is always
    // added (-0.0 without one leaves every value unchanged). ----
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // loads past the last block
    lds_barrier();
    const bool has_bias = p.bias != nullptr;
    const uint16_t* lds_bias = reinterpret_cast<const uint16_t*>(smem + XB_BIAS);
    uint8_t* stg = smem + wave_u * 64 * QEPITCH;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int lc0 = wn * 64 + ni * 32 + 8 * q + 4 * h;
            const uint2 b2 = *reinterpret_cast<const uint2*>(lds_bias + lc0);
            const float bc[4] = {has_bias ? __uint_as_float(b2.x << 16) : -0.0f,
                                 has_bias ? __uint_as_float(b2.x & 0xffff0000u) : -0.0f,
                                 has_bias ? __uint_as_float(b2.y << 16) : -0.0f,
                                 has_bias ? __uint_as_float(b2.y & 0xffff0000u) : -0.0f};
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                float v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[j] = add_bias(acc[mi][ni][4 * q + j], bc[j]);
                    if constexpr (EPI == 1) v[j] = gelu_tanh(v[j]);
                }
                *reinterpret_cast<uint2*>(stg + (mi * 32 + fr) * QEPITCH + (ni * 32 + 8 * q + 4 * h) * 2) =
                    make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // a wave reads back only its own rows
    const int ch = lane & 7;
    const int gcol = n0 + wn * 64 + ch * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int lrow = j * 8 + (lane >> 3);
        const v4u d = *reinterpret_cast<const v4u*>(stg + lrow * QEPITCH + ch * 16);
        const int grow = m0 + wm * 64 + lrow;
        if (grow < p.m && gcol < p.n)
            *reinterpret_cast<v4u*>(p.y + (int64_t)grow * p.n + gcol) = d;
    }
}

// ---------------------------------------------------------------------------
// Two-workgroups-per-CU kernel for per-token / per-channel scales: a
// 256x128 tile and 4 waves of 128x64, with at most 256
// registers per wave and 72 KB of LDS per workgroup so that two workgroups
// share every CU; each SIMD then interleaves the MFMAs of two independent
// waves, which hides one workgroup's barrier and memory waits behind the
// other's MFMAs.
// ---------------------------------------------------------------------------
template <int QT, int EPI, bool WANT_Y, bool WANT_ACC>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void gemm_dual_kernel(const Params p)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[DSMEM];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    int tm, tn;
    map_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * QBN;
    const int K = p.k;
    const int rows_a = min(BM, p.m - m0), rows_b = min(QBN, p.n - n0);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.a + (int64_t)m0 * K), (short)0, rows_a * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.b + (int64_t)n0 * K), (short)0, rows_b * K, 0x00020000);

    const int lc = t & 3, lr = t >> 2;
    const int voff = lr * K + lc * 16;
    const int stride64 = 64 * K;
    const int lds_w = lr * QK + ((lc ^ ((lr >> 2) & 3)) << 4);
    const int fr = lane & 31, h = lane >> 5, sw = (fr >> 2) & 3;
    const int rd0 = fr * QK + (((2 * h) ^ sw) << 4);
    const int rd1 = fr * QK + (((2 * h + 1) ^ sw) << 4);
    const int a_rd = wm * 128 * QK;
    const int b_rd = QA + wn * 64 * QK;
    const int KT = (K + QK - 1) / QK;

    typedef typename PipeAcc<QT>::type acc_t;
    v4u ga[3][4], gb[3][2];
    acc_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

    auto gload = [&](int kt, v4u (&da)[4], v4u (&db)[2]) {
        const int k0 = kt * QK;
        const int oob = (int)((unsigned)(k0 + lc * 16 >= K) << 31);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int off = (voff + j * stride64 + k0) | oob;
            da[j] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
            if (j < 2) db[j] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
        }
    };
    auto lstore = [&](int buf, const v4u (&da)[4], const v4u (&db)[2]) {
        uint8_t* s = smem + buf * QSTAGE;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *reinterpret_cast<v4u*>(s + lds_w + j * 64 * QK) = da[j];
            if (j < 2) *reinterpret_cast<v4u*>(s + QA + lds_w + j * 64 * QK) = db[j];
        }
    };
    auto frag = [&](const uint8_t* s) -> v8i {
        const v4i lo = *reinterpret_cast<const v4i*>(s + rd0);
        const v4i hi = *reinterpret_cast<const v4i*>(s + rd1);
        return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto compute = [&](int buf) {
        const uint8_t* s = smem + buf * QSTAGE;
        v8i bf[2];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) bf[ni] = frag(s + b_rd + ni * 32 * QK);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const v8i af = frag(s + a_rd + mi * 32 * QK);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                if constexpr (QT == kE4M3FN) {
                    acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        bf[ni], af, acc[mi][ni], 0, 0, 0, 0, 0, 0);
                } else {
                    const v8i b8 = bf[ni];
                    acc[mi][ni] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                        v4i{b8[0], b8[1], b8[2], b8[3]}, v4i{af[0], af[1], af[2], af[3]},
                        acc[mi][ni], 0, 0, 0);
                    acc[mi][ni] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                        v4i{b8[4], b8[5], b8[6], b8[7]}, v4i{af[4], af[5], af[6], af[7]},
                        acc[mi][ni], 0, 0, 0);
                }
            }
        }
    };

    // 3-slot register ring and 3 LDS buffers (stage s in slot and buffer
    // s % 3), one barrier per stage: step s writes stage s+1 into the buffer
    // of stage s-2, loads stage s+3 into the slot it just emptied and
    // computes stage s.  The loop runs a multiple of 3 stages (stages past K
    // read zeros).
    gload(0, ga[0], gb[0]);
    gload(1, ga[1], gb[1]);
    gload(2, ga[2], gb[2]);
    lstore(0, ga[0], gb[0]);
#define TFQ_DUAL_STEP(U)                                                       \
    {                                                                          \
        lds_barrier();                                                         \
        lstore(((U) + 1) % 3, ga[((U) + 1) % 3], gb[((U) + 1) % 3]);          \
        gload(kt + (U) + 3, ga[(U)], gb[(U)]);                                 \
        compute((U));                                                          \
    }
    for (int kt = 0; kt < KT; kt += 3) {
        TFQ_DUAL_STEP(0)
        TFQ_DUAL_STEP(1)
        TFQ_DUAL_STEP(2)
    }
#undef TFQ_DUAL_STEP

    // ---- epilogue: lane holds row wm*128 + mi*32 + fr and columns
    // wn*64 + ni*32 + 8q + 4h + (0..3) in registers 4q..4q+3 ----
    float srow[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int row = m0 + wm * 128 + mi * 32 + fr;
        srow[mi] = row < p.m ? p.sa[row] : 0.0f;
    }
    if constexpr (WANT_ACC) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int row = m0 + wm * 128 + mi * 32 + fr;
            if (row >= p.m) continue;
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c0 = n0 + wn * 64 + ni * 32 + 8 * q + 4 * h;
                    if (c0 < p.n)
                        *reinterpret_cast<v4i*>(p.acc + (int64_t)row * p.n + c0) =
                            v4i{(int)acc[mi][ni][4 * q], (int)acc[mi][ni][4 * q + 1],
                                (int)acc[mi][ni][4 * q + 2], (int)acc[mi][ni][4 * q + 3]};
                }
        }
    }
    if constexpr (WANT_Y) {
        lds_barrier();
        uint8_t* stg = smem + wave * 128 * QEPITCH;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c0 = n0 + wn * 64 + ni * 32 + 8 * q + 4 * h;
                float sc[4], bc[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool ok = c0 + j < p.n;
                    sc[j] = ok ? p.sb[c0 + j] : 0.0f;
                    bc[j] = (p.bias != nullptr && ok) ? bf16_to_f32(p.bias[c0 + j]) : 0.0f;
                }
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    float v[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        v[j] = scale_out((float)acc[mi][ni][4 * q + j], srow[mi], sc[j]);
                        if (p.bias != nullptr) v[j] = add_bias(v[j], bc[j]);
                        if constexpr (EPI == 1) v[j] = gelu_tanh(v[j]);
                    }
                    const uint32_t lo = pack_bf16x2(v[0], v[1]);
                    const uint32_t hi = pack_bf16x2(v[2], v[3]);
                    *reinterpret_cast<uint2*>(stg + (mi * 32 + fr) * QEPITCH +
                                              (ni * 32 + 8 * q + 4 * h) * 2) = make_uint2(lo, hi);
                }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int ch = lane & 7;
        const int gcol = n0 + wn * 64 + ch * 8;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int lrow = j * 8 + (lane >> 3);
            const v4u d = *reinterpret_cast<const v4u*>(stg + lrow * QEPITCH + ch * 16);
            const int grow = m0 + wm * 128 + lrow;
            if (grow < p.m && gcol < p.n)
                *reinterpret_cast<v4u*>(p.y + (int64_t)grow * p.n + gcol) = d;
        }
    }
}

template <int QT, int EPI, bool WANT_Y, bool WANT_ACC>
hipError_t launch_dual(Params p, hipStream_t st)
{
    p.tiles_n = (p.n + QBN - 1) / QBN;
    const unsigned grid = (unsigned)(p.tiles_m * p.tiles_n);
    hipLaunchKernelGGL((gemm_dual_kernel<QT, EPI, WANT_Y, WANT_ACC>), dim3(grid), dim3(256), 0, st,
                       p);
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_block(Params p, hipStream_t st)
{
    p.tiles_n = (p.n + QBN - 1) / QBN;
    const unsigned grid = (unsigned)(p.tiles_m * p.tiles_n);
    hipLaunchKernelGGL((gemm_block_kernel<EPI>), dim3(grid), dim3(512), 0, st, p);
    return hipGetLastError();
}

template <int QT, int EPI, bool WANT_Y, bool WANT_ACC, bool GROUPED = false, int NB = 4>
hipError_t launch_pipe(Params p, hipStream_t st)
{
    p.tiles_n = (p.n + 64 * NB - 1) / (64 * NB);
    const unsigned grid = (unsigned)(p.tiles_m * p.tiles_n);
    hipLaunchKernelGGL((gemm_pipe_kernel<QT, EPI, WANT_Y, WANT_ACC, GROUPED, NB>), dim3(grid),
                       dim3(256), 0, st, p);
    return hipGetLastError();
}

// INT8 outputs of the LDS kernel: BF16 and / or raw INT32 sums
template <int EPI, int NB>
hipError_t launch_pipe_int8(const Params& p, bool y, bool a, hipStream_t st)
{
    if (y && a) return launch_pipe<kInt8, EPI, true, true, false, NB>(p, st);
    if (y) return launch_pipe<kInt8, EPI, true, false, false, NB>(p, st);
    return launch_pipe<kInt8, EPI, false, true, false, NB>(p, st);
}

// Tile rows per band of the tile order (see map_tile).  The 32 tiles in
// flight on one XCD cover about band x (32 / band) tiles; their A row panels
// stream from HBM while the B (weight) panels mostly hit the Infinity Cache.
// With long K (a 256-row A panel of 2 MB or more) fewer concurrent A panels
// win: measured on MI355X, K = 13824 runs best with bands of 2 (2.44 vs 2.34
// PFLOP/s with 4), K = 3072 and 5120 with bands of 4.
int band_rows(int64_t m, int64_t n, int64_t k)
{
    (void)m;
    (void)n;
    return k >= 8192 ? 2 : 4;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device (256 on MI355X).
int64_t device_cus()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        return 256;
    }
    return cus;
}

// 256- or 192-column tiles for a per-channel FP8 / INT8 grid: the width
// whose grid ends closer to a whole number of waves over the CUs, the cost
// taken as waves x tile width (one tile per CU at a time), 256 on a tie.
// E.g. image-DiT FFN-up 7145 x 12288: 1344 tiles of 256 (5.25 waves) or
// exactly 1792 of 192 (7 waves); INT8 4096 x 3072: 192 tiles of 256 (0.75
// of a wave) or exactly 256 of 192.
bool prefer_192(int64_t m, int64_t n)
{
    const int64_t cus = device_cus(), tm = ceil_div(m, BM);
    return 3 * ceil_div(tm * ceil_div(n, 192), cus) < 4 * ceil_div(tm * ceil_div(n, 256), cus);
}

}  // namespace

// Heuristic launch configuration: the 256x256 kernel, or for per-channel
// FP8 / INT8 the 256x192 one where its grid fills the last wave better
// (prefer_192); for grids of fewer than 64 256x256 tiles, the 256x128
// two-per-CU kernel, which keeps twice as many CUs busy; band height by K
// (band_rows).  Measured on MI355X: from 108 tiles up (FP8 and INT8, up to
// 240 tiles) the 256x256 kernel is 3-38% faster than the two-per-CU one
// even with CUs idle; at 16 tiles the two-per-CU kernel is slightly ahead.
GemmConfig default_config(const GemmArgs& g)
{
    const int64_t tiles = ((g.m + BM - 1) / BM) * ((g.n + BN - 1) / BN);
    const bool dual_ok = g.groups == 0 && g.scale_block == 0 && (g.qtype == kE4M3FN || g.qtype == kInt8);
    const int band = band_rows(g.m, g.n, g.k);
    if (dual_ok && tiles < 64) return GemmConfig{1, band};
    if (dual_ok && prefer_192(g.m, g.n)) return GemmConfig{2, band};
    return GemmConfig{0, band};
}

int candidate_configs(const GemmArgs& g, GemmConfig* out, int max_out)
{
    static const int bands[4] = {1, 2, 4, 8};
    int n = 0;
    const int64_t tiles = ((g.m + BM - 1) / BM) * ((g.n + BN - 1) / BN);
    const bool dual_ok = g.groups == 0 && g.scale_block == 0 && (g.qtype == kE4M3FN || g.qtype == kInt8);
    for (int kernel = 0; kernel < 3; ++kernel) {
        // the two-per-CU kernel only where the grid is small enough to gain
        if (kernel == 1 && !(dual_ok && tiles < 512)) continue;
        // 192-column tiles: per-channel FP8 and INT8
        if (kernel == 2 && !dual_ok) continue;
        for (int b : bands)
            if (n < max_out) out[n++] = GemmConfig{kernel, b};
    }
    return n;
}

bool config_is_candidate(const GemmArgs& g, GemmConfig c)
{
    GemmConfig cand[32];
    const int n = candidate_configs(g, cand, 32);
    for (int i = 0; i < n; ++i)
        if (cand[i].kernel == c.kernel && cand[i].band == c.band) return true;
    return false;
}

// Every configuration sums every output in the same order (same MFMAs, same
// K stages, only the tile order or tile shape differs), so the choice never
// changes a result bit.
hipError_t launch_scaled_gemm_with(const GemmArgs& g, GemmConfig c, hipStream_t stream)
{
    Params p;
    p.a = g.a;
    p.b = g.b;
    p.sa = g.sa;
    p.sb = g.sb;
    p.ea = g.ea;
    p.eb = g.eb;
    p.bias = g.bias;
    p.y = g.y;
    p.acc = g.acc;
    p.m = (int)g.m;
    p.n = (int)g.n;
    p.k = (int)g.k;
    p.tiles_m = (int)((g.m + BM - 1) / BM);
    p.tiles_n = (int)((g.n + BN - 1) / BN);
    p.group_m = c.band;
    p.goff = g.group_offsets;
    p.groups = g.groups;
    if (g.groups > 0) {
        // grouped (MoE) FP8: at most ceil(m / 256) + groups tile rows; each
        // XCD's share of a group's tiles rounds up by at most one, so 8 more
        // workgroups per group (and 8 spare) cover every tile
        p.tiles_m += g.groups;
        const unsigned grid = (unsigned)(p.tiles_m * p.tiles_n + 8 * g.groups + 8);
        if (g.epi == 1)
            hipLaunchKernelGGL((gemm_pipe_kernel<kE4M3FN, 1, true, false, true>), dim3(grid),
                               dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((gemm_pipe_kernel<kE4M3FN, 0, true, false, true>), dim3(grid),
                               dim3(256), 0, stream, p);
        return hipGetLastError();
    }
    if (g.scale_block == 128)
        return g.epi == 1 ? launch_block<1>(p, stream) : launch_block<0>(p, stream);
    // MXFP8 and MXFP4 always take the 256x256 kernel (its scale ring lives there)
    if (g.qtype == kMxE4M3)
        return g.epi == 1 ? launch_pipe<kMxE4M3, 1, true, false>(p, stream)
                          : launch_pipe<kMxE4M3, 0, true, false>(p, stream);
    if (g.qtype == kMxE2M1)
        return g.epi == 1 ? launch_pipe<kMxE2M1, 1, true, false>(p, stream)
                          : launch_pipe<kMxE2M1, 0, true, false>(p, stream);
    if (g.qtype == kMxE2M3)
        return g.epi == 1 ? launch_pipe<kMxE2M3, 1, true, false>(p, stream)
                          : launch_pipe<kMxE2M3, 0, true, false>(p, stream);
    if (g.qtype == kMxE3M2)
        return g.epi == 1 ? launch_pipe<kMxE3M2, 1, true, false>(p, stream)
                          : launch_pipe<kMxE3M2, 0, true, false>(p, stream);
    const bool dual = c.kernel == 1;
    const bool y = g.y != nullptr, a = g.acc != nullptr;
    if (g.qtype == kE4M3FN) {
        if (dual)
            return g.epi == 1 ? launch_dual<kE4M3FN, 1, true, false>(p, stream)
                              : launch_dual<kE4M3FN, 0, true, false>(p, stream);
        if (c.kernel == 2)
            return g.epi == 1 ? launch_pipe<kE4M3FN, 1, true, false, false, 3>(p, stream)
                              : launch_pipe<kE4M3FN, 0, true, false, false, 3>(p, stream);
        return g.epi == 1 ? launch_pipe<kE4M3FN, 1, true, false>(p, stream)
                          : launch_pipe<kE4M3FN, 0, true, false>(p, stream);
    }
    if (c.kernel == 2)
        return g.epi == 1 ? launch_pipe_int8<1, 3>(p, y, a, stream) : launch_pipe_int8<0, 3>(p, y, a, stream);
    if (dual) {
        if (g.epi == 1) {
            if (y && a) return launch_dual<kInt8, 1, true, true>(p, stream);
            if (y) return launch_dual<kInt8, 1, true, false>(p, stream);
            return launch_dual<kInt8, 1, false, true>(p, stream);
        }
        if (y && a) return launch_dual<kInt8, 0, true, true>(p, stream);
        if (y) return launch_dual<kInt8, 0, true, false>(p, stream);
        return launch_dual<kInt8, 0, false, true>(p, stream);
    }
    if (g.epi == 1) {
        if (y && a) return launch_pipe<kInt8, 1, true, true>(p, stream);
        if (y) return launch_pipe<kInt8, 1, true, false>(p, stream);
        return launch_pipe<kInt8, 1, false, true>(p, stream);
    }
    if (y && a) return launch_pipe<kInt8, 0, true, true>(p, stream);
    if (y) return launch_pipe<kInt8, 0, true, false>(p, stream);
    return launch_pipe<kInt8, 0, false, true>(p, stream);
}

}  // namespace tfq
