/* A plain C11 client of the library's C ABI (include/swiglu.h): host-only
 * calls and argument validation, which need no GPU.  Built and run by
 * tests/test_abi_cpu.py; prints "ok" and exits 0 when every check holds. */
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include "swiglu.h"

#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
            return 1;                                                      \
        }                                                                  \
    } while (0)

int main(void) {
    /* fake, 16-byte aligned, far apart device addresses: validation rejects
     * every call below before any of them could be dereferenced */
    const uint16_t *A = (const uint16_t *)(uintptr_t)0x100000000ull;
    const uint16_t *W = (const uint16_t *)(uintptr_t)0x200000000ull;
    uint16_t *Y = (uint16_t *)(uintptr_t)0x300000000ull;

    CHECK(strcmp(swiglu_status_string(SWIGLU_OK), "ok") == 0);
    CHECK(strcmp(swiglu_status_string(12345), "unknown status") == 0);
    CHECK(swiglu_select_variant(2048, 8960, 1536) == SWIGLU_VARIANT_I);
    CHECK(swiglu_select_variant(-1, 8, 8) == SWIGLU_ERR_SHAPE);
    CHECK(swiglu_fp8_scale_exp(448.0) == 0 && swiglu_fp8_scale_exp(5.0) == -6);

    CHECK(swiglu_fused_gemm(A, W, Y, 256, 256, 4, SWIGLU_AUTO, NULL, 0, NULL) == SWIGLU_ERR_SHAPE);
    CHECK(strlen(swiglu_last_error()) > 0);
    CHECK(swiglu_fused_gemm(A, W, NULL, 256, 256, 256, SWIGLU_VARIANT_I, NULL, 0, NULL) ==
          SWIGLU_ERR_NULL);
    CHECK(swiglu_fused_gemm(A, W, Y, 256, 256, 256, 7, NULL, 0, NULL) == SWIGLU_ERR_UNSUPPORTED);
    CHECK(swiglu_fused_gemm_strided(A, 248, W, Y, 256, 256, 256, 256, SWIGLU_VARIANT_I, NULL, 0,
                                    NULL) == SWIGLU_ERR_SHAPE);
    CHECK(swiglu_pack_weights(A, W, Y, 12, 8, NULL) == SWIGLU_ERR_SHAPE);
    CHECK(swiglu_pack_weights_nk(A, W, NULL, 8, 8, NULL) == SWIGLU_ERR_NULL);
    CHECK(swiglu_down_proj(A, W, Y, 256, 12, 256, NULL, 0, NULL) == SWIGLU_ERR_SHAPE);
    CHECK(swiglu_gated_mlp(A, W, W, Y, Y, 256, 256, 256, SWIGLU_VARIANT_I, NULL, 0, NULL) ==
          SWIGLU_ERR_ALIAS);
    CHECK(swiglu_quantize_fp8(A, (uint8_t *)Y, 24, 0, NULL) == SWIGLU_ERR_SHAPE);
    CHECK(swiglu_fused_gemm_fp8((const uint8_t *)A, (const uint8_t *)W, Y, 256, 256, 24, 0, 0,
                                SWIGLU_AUTO, NULL, 0, NULL) == SWIGLU_ERR_SHAPE);
    CHECK(swiglu_fused_gemm_fp8((const uint8_t *)A, (const uint8_t *)W, Y, 256, 256, 256, 0, 0, 9,
                                NULL, 0, NULL) == SWIGLU_ERR_UNSUPPORTED);
    CHECK(swiglu_silu_mul(A, A, Y, 12, NULL) == SWIGLU_ERR_SHAPE);
    /* empty problems succeed without touching anything */
    CHECK(swiglu_fused_gemm(NULL, NULL, NULL, 0, 256, 256, SWIGLU_AUTO, NULL, 0, NULL) == SWIGLU_OK);
    CHECK(swiglu_last_error()[0] == '\0');
    char buf[64];
    CHECK(swiglu_describe_launch(0, 256, 256, SWIGLU_AUTO, 0, buf, sizeof buf) == SWIGLU_OK);
    CHECK(strcmp(buf, "nothing (empty problem)") == 0);
    printf("ok\n");
    return 0;
}
