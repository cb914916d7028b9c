/* A plain C11 client of include/tfq.h: compiled and run by
 * tests/test_c_client.py (no GPU needed).  Checks that the header is valid
 * C, that every declared entry point links against libtfq.so, and that host
 * validation answers through the C ABI: bad arguments come back as status
 * codes before any HIP call, with a message for each. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tfq.h"

static int fails = 0;
#define EXPECT(cond)                                                    \
    do {                                                                \
        if (!(cond)) {                                                  \
            printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);      \
            ++fails;                                                    \
        }                                                               \
    } while (0)

/* every entry point, taken by address so that a missing symbol fails the link */
typedef void (*fn_t)(void);
static const fn_t entry_points[] = {
    (fn_t)tfq_quantize_rows,           (fn_t)tfq_quantize_rows_gather,
    (fn_t)tfq_quantize_weight_per_channel, (fn_t)tfq_scaled_mm_fp8,
    (fn_t)tfq_scaled_mm_int8,          (fn_t)tfq_grouped_scaled_mm_fp8,
    (fn_t)tfq_quant_linear_workspace_bytes, (fn_t)tfq_quant_linear_fused,
    (fn_t)tfq_quantize_mx,             (fn_t)tfq_scaled_mm_mxfp8,
    (fn_t)tfq_quantize_mxfp4,          (fn_t)tfq_scaled_mm_mxfp4,
    (fn_t)tfq_quantize_mxfp6,          (fn_t)tfq_scaled_mm_mxfp6,
    (fn_t)tfq_kv_cache_store,          (fn_t)tfq_kv_cache_load,
    (fn_t)tfq_set_autotune,            (fn_t)tfq_autotune_lookup,
    (fn_t)tfq_autotune_clear,          (fn_t)tfq_autotune_set,
    (fn_t)tfq_quant_linear_fused_noalloc, (fn_t)tfq_e4m3fn_encode_f32,
    (fn_t)tfq_status_string,           (fn_t)tfq_last_hip_error,
    (fn_t)tfq_abi_version,
};

int main(void)
{
    for (size_t i = 0; i < sizeof entry_points / sizeof entry_points[0]; ++i)
        EXPECT(entry_points[i] != NULL);
    EXPECT(tfq_abi_version() == TFQ_ABI_VERSION);

    /* every status has a message */
    for (int s = TFQ_OK; s <= TFQ_ERR_HIP; ++s) {
        const char* msg = tfq_status_string((tfq_status)s);
        EXPECT(msg != NULL && strlen(msg) > 0);
    }

    /* host validation, before any HIP call (addresses never dereferenced) */
    static uint8_t host[1 << 17];
    uint8_t* p = (uint8_t*)(((uintptr_t)host + 255) & ~(uintptr_t)255);
    EXPECT(tfq_quantize_rows(NULL, 4, 128, 128, TFQ_QTYPE_E4M3FN, 448.0f, 0, p, (float*)(p + 4096), NULL) ==
           TFQ_ERR_NULL_POINTER);
    EXPECT(tfq_quantize_rows(p, 4, 100, 128, TFQ_QTYPE_E4M3FN, 448.0f, 0, p + 4096, (float*)(p + 8192), NULL) ==
           TFQ_ERR_BAD_SHAPE);                                        /* cols % 16 */
    EXPECT(tfq_quantize_rows(p, 4, 128, 128, TFQ_QTYPE_E4M3FN, 21.0f, 0, p + 4096, (float*)(p + 8192), NULL) ==
           TFQ_ERR_BAD_QMAX);                                         /* not on the E4M3FN grid */
    EXPECT(tfq_scaled_mm_int8((const int8_t*)p, (const float*)(p + 4096), (const int8_t*)(p + 8192),
                              (const float*)(p + 12288), 16, 16, 131072, NULL, TFQ_EPI_NONE,
                              p + 16384, NULL, NULL) == TFQ_ERR_BAD_SHAPE); /* INT32 overflow bound */
    EXPECT(tfq_scaled_mm_fp8(p, (const float*)(p + 4096), p + 8192, (const float*)(p + 12288), 16, 16, 128,
                             0, NULL, TFQ_EPI_GELU_TANH, p, NULL) == TFQ_ERR_ALIAS); /* y over a_q */
    EXPECT(tfq_quant_linear_workspace_bytes(1024, 4096, TFQ_QTYPE_E4M3FN, 0) >= (size_t)1024 * 4096);
    EXPECT(tfq_set_autotune(2) == TFQ_ERR_UNSUPPORTED);

    /* one error path of every other entry point */
    const float* f = (const float*)(p + 4096);
    EXPECT(tfq_quantize_rows_gather(p, 8, 128, 128, NULL, 4, TFQ_QTYPE_E4M3FN, 448.0f, 0, p + 4096,
                                    (float*)(p + 8192), NULL) == TFQ_ERR_NULL_POINTER);
    EXPECT(tfq_quantize_weight_per_channel(p, 100, 128, TFQ_QTYPE_E4M3FN, 448.0f, 128, p + 32768,
                                           (float*)(p + 49152), NULL) == TFQ_ERR_BAD_SHAPE); /* n % 128 */
    EXPECT(tfq_grouped_scaled_mm_fp8(p, f, p + 8192, f, (const int32_t*)(p + 12288), 0, 16, 16, 128,
                                     NULL, TFQ_EPI_NONE, p + 16384, NULL) != TFQ_OK);  /* no groups */
    EXPECT(tfq_quant_linear_fused(p, 16, 128, 128, p + 4096, f, 16, TFQ_QTYPE_E4M3FN, 448.0f, 0, NULL,
                                  TFQ_EPI_NONE, p + 8192, p + 16384, 16, NULL) ==
           TFQ_ERR_WORKSPACE_TOO_SMALL);
    /* 16384 x 5120 activation codes exceed the 64 MiB device scratch */
    EXPECT(tfq_quant_linear_fused_noalloc(p, 16384, 5120, 5120, p + 4096, f, 256, TFQ_QTYPE_E4M3FN,
                                          448.0f, 0, NULL, TFQ_EPI_NONE, p + 8192, NULL) ==
           TFQ_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(tfq_autotune_set(9, 64, 64, 64, TFQ_EPI_NONE, 0, 0, 4) == TFQ_ERR_UNSUPPORTED);
    EXPECT(tfq_quantize_mx(p, 4, 100, 128, p + 4096, (uint32_t*)(p + 8192), NULL) == TFQ_ERR_BAD_SHAPE);
    EXPECT(tfq_scaled_mm_mxfp8(p, (const uint32_t*)f, p + 8192, (const uint32_t*)f, 16, 16, 100, NULL,
                               TFQ_EPI_NONE, p + 16384, NULL) == TFQ_ERR_BAD_SHAPE);
    EXPECT(tfq_quantize_mxfp4(p + 2, 4, 128, 128, p + 4096, (uint32_t*)(p + 8192), NULL) ==
           TFQ_ERR_MISALIGNED);
    EXPECT(tfq_scaled_mm_mxfp4(p, (const uint32_t*)f, p + 8192, (const uint32_t*)f, 16, 16, 128, NULL,
                               7, p + 16384, NULL) == TFQ_ERR_UNSUPPORTED);        /* epilogue */
    EXPECT(tfq_quantize_mxfp6(p, 4, 128, 128, 5, p + 4096, (uint32_t*)(p + 8192), NULL) ==
           TFQ_ERR_UNSUPPORTED);                                             /* format */
    EXPECT(tfq_scaled_mm_mxfp6(p, (const uint32_t*)f, p + 8192, (const uint32_t*)f, 16, 16, 192, 0, NULL,
                               TFQ_EPI_NONE, p + 16384, NULL) == TFQ_ERR_BAD_SHAPE); /* k % 128 */
    EXPECT(tfq_kv_cache_store(p, 4, 2, 128, 256, NULL, 10, 448.0f, p + 4096, (float*)(p + 8192), NULL) ==
           TFQ_ERR_NULL_POINTER);
    EXPECT(tfq_kv_cache_load(p, f, 10, 2, 128, (const int32_t*)(p + 8192), 4, 9, p + 16384, NULL) ==
           TFQ_ERR_UNSUPPORTED);                                             /* output dtype */
    EXPECT(tfq_e4m3fn_encode_f32(f, p, 6, NULL) == TFQ_ERR_BAD_SHAPE);      /* n % 4 */
    int32_t kern = -1, band = -1;
    tfq_autotune_clear();
    EXPECT(tfq_autotune_lookup(0, 256, 256, 256, 0, 0, &kern, &band) == 0); /* nothing cached */
    EXPECT(tfq_last_hip_error() == 0);

    if (fails == 0) printf("c client ok: %zu entry points, ABI %d\n",
                           sizeof entry_points / sizeof entry_points[0], tfq_abi_version());
    return fails != 0;
}
