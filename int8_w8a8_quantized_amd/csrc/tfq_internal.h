// Internal declarations shared by the host dispatch (abi.cpp) and the HIP
// kernel launchers.  Not part of the public ABI (include/tfq.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tfq {

// kMxE4M3: E4M3FN codes with one E8M0 scale per 32 elements along K (MXFP8);
// kMxE2M1: E2M1 codes, two per byte, with the same scales (MXFP4);
// kMxE2M3 / kMxE3M2: 6-bit codes, a little-endian bit stream (MXFP6)
enum QType : int { kE4M3FN = 0, kInt8 = 1, kMxE4M3 = 2, kMxE2M1 = 3, kMxE2M3 = 4, kMxE3M2 = 5 };

// Launchers enqueue kernels on `stream` and return the launch status.  They
// assume the arguments already passed the host-side validation.

// Row-wise (group_cols == 0) or 1x128-group (group_cols == 128) quantisation.
// With `gather`, output row r quantises row gather[r] of x (x has src_rows
// rows; an index outside [0, src_rows) reads as a zero row).
hipError_t launch_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                                int qtype, float qmax, int group_cols, uint8_t* q, float* scale,
                                hipStream_t stream, const int32_t* gather = nullptr,
                                int64_t src_rows = 0);

// MX rows (cols % 128 == 0): E8M0 scale words [cols/128, rows] (bytes 0..3
// of word (g, r) = blocks 4 g + 0, 2, 1, 3 of row r); elem_bits 8: MXFP8 codes [rows, cols]; 4: MXFP4 codes [rows, cols/2], two
// per byte (lower index in the low nibble); 62 / 63: MXFP6 E2M3 / E3M2 codes
// [cols/128, rows, 96]: the 128 codes of group g of row r as a little-endian
// 6-bit stream at byte (g rows + r) 96
hipError_t launch_quantize_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                              uint8_t* q, uint32_t* scale, hipStream_t stream, int elem_bits = 8);

// FP8 KV cache: store kv [tokens, heads, hd] (token stride ld_token) into
// cache rows slot[t] * heads + h; load rows index[i] dequantised to
// out_dtype (0 BF16, 1 FP16, 2 FP32) as [n, heads, hd].
hipError_t launch_kv_store(const uint16_t* kv, int64_t tokens, int heads, int hd, int64_t ld_token,
                           const int32_t* slot, int64_t slots, float qmax, uint8_t* cache,
                           float* scale, hipStream_t stream);
hipError_t launch_kv_load(const uint8_t* cache, const float* scale, int64_t slots, int heads, int hd,
                          const int32_t* index, int64_t n, int out_dtype, void* out,
                          hipStream_t stream);

// 128x128 block weight quantisation (n % 128 == 0, k % 128 == 0).
hipError_t launch_quantize_blocks(const uint16_t* w, int64_t n, int64_t k, int qtype, float qmax,
                                  uint8_t* q, float* scale, hipStream_t stream);

// Device E4M3FN encoder over n floats (n % 4 == 0).
hipError_t launch_e4m3fn_encode(const float* x, uint8_t* q, int64_t n, hipStream_t stream);

struct GemmArgs {
    const uint8_t* a;      // [m, k] codes (MXFP6: [k/128, m, 96])
    const uint8_t* b;      // [n, k] codes (MXFP6: [k/128, n, 96])
    const float* sa;       // [m] or [m, k/128]
    const float* sb;       // [n] or [n/128, k/128]
    const uint16_t* bias;  // [n] BF16 or null
    uint16_t* y;           // [m, n] BF16 or null
    int32_t* acc;          // [m, n] INT32 or null (INT8 only)
    int64_t m, n, k;
    int qtype;
    int scale_block;       // 0 or 128
    int epi;               // 0 none, 1 gelu-tanh
    const uint32_t* ea;    // MXFP8: E8M0 scale words [k/128, m] (sa, sb unused), else null
    const uint32_t* eb;    // MXFP8: E8M0 scale words [k/128, n], else null
    // grouped (MoE) FP8: b [groups, n, k], sb [groups, n], bias [groups, n];
    // rows group_offsets[g] .. group_offsets[g+1] (device int32) use group g
    const int32_t* group_offsets;
    int groups;            // 0 = not grouped
};

// A GEMM launch configuration: kernel 0 = 256x256 tiles, 1 = 256x128 tiles
// two per CU, 2 = 256x192 tiles (1 and 2: per-channel FP8 / INT8 only); band
// = tile rows per band of the tile order.  Every candidate configuration of a shape gives the same
// result bits.
struct GemmConfig {
    int kernel;
    int band;
};

GemmConfig default_config(const GemmArgs& g);
// the configurations the autotuner times for g (at most max_out)
int candidate_configs(const GemmArgs& g, GemmConfig* out, int max_out);
bool config_is_candidate(const GemmArgs& g, GemmConfig c);
hipError_t launch_scaled_gemm_with(const GemmArgs& g, GemmConfig c, hipStream_t stream);
// the library's GEMM launch: the autotuned configuration if autotuning is on
// (tune.cpp), else default_config
hipError_t launch_scaled_gemm(const GemmArgs& g, hipStream_t stream);

// The allocation-free fused Linear's scratch (noalloc.hip): a file-scope
// device array of kNoAllocScratchBytes per GPU; noalloc_scratch gives the
// current device's copy (hipGetSymbolAddress on first use per device).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void** out);
// the configuration launch_scaled_gemm would use, without ever tuning: the
// cached one if autotuning is on and the shape has been tuned, else the
// heuristic (no event creation, no synchronisation)
GemmConfig config_without_tuning(const GemmArgs& g);

// autotune mode (0 off, 1 on), cache lookup and reset (tune.cpp)
void set_autotune(int mode);
int autotune_mode();
bool autotune_lookup(int dev, const GemmArgs& g, GemmConfig* out);
// put c (a candidate of g) in the cache of device dev
void autotune_set(int dev, const GemmArgs& g, GemmConfig c);
void autotune_clear();

}  // namespace tfq
