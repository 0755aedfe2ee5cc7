/* Host-side checks of the C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every argument-validation path of
 * include/cfp32.h, the workspace-size queries, the status strings and the
 * empty problems.  Built against api.hip alone, with launcher stubs that
 * abort if reached: none of these calls may get as far as a kernel launch.
 * Exit status 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/cfp32.h"

static int failures = 0;

#define CHECK(cond)                                                         \
    do {                                                                    \
        if (!(cond)) {                                                      \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

int main(int argc, char **argv)
{
    void *F = (void *)(uintptr_t)(1u << 20); /* never dereferenced */
    const float *fx = (const float *)F;
    const uint16_t *fw = (const uint16_t *)F;
    float *fy = (float *)F;
    uint16_t *fh = (uint16_t *)F;
    const cfp32_status E = CFP32_ERR_INVALID_VALUE;

    for (int s = 0; s <= 4; ++s) CHECK(strlen(cfp32_status_string(s)) > 0);
    CHECK(strcmp(cfp32_status_string(99), "unknown status") == 0);
    CHECK(strcmp(cfp32_status_string(-1), "unknown status") == 0);
    CHECK(cfp32_last_hip_error() == 0);

    /* negative sizes, null pointers, short leading dimensions */
    CHECK(cfp32_split(fx, 4, fh, fh, 4, -1, 4, NULL) == E);
    CHECK(cfp32_gemm(fw, fw, 4, fw, 4, fy, NULL, NULL, 4, 4, 4, -4, NULL) == E);
    CHECK(cfp32_split(NULL, 4, fh, fh, 4, 2, 4, NULL) == E);
    CHECK(cfp32_merge(fx, NULL, 4, fy, 4, 2, 4, NULL) == E);
    CHECK(cfp32_linear(fx, 8, NULL, 8, fy, 8, 2, 8, 8, NULL, 0, NULL) == E);
    CHECK(cfp32_split(fx, 3, fh, fh, 4, 2, 4, NULL) == E);
    CHECK(cfp32_gemm(fw, fw, 7, fw, 8, fy, NULL, NULL, 8, 4, 8, 8, NULL) == E);
    CHECK(cfp32_merge(fx, fx, 8, fy, 7, 2, 8, NULL) == E);
    /* separate-addition GEMM: unsupported depths, missing outputs */
    const int64_t bad_kpa[] = {-16, 8, 32, 128, 512};
    for (int i = 0; i < 5; ++i)
        CHECK(cfp32_gemm_separate_add(fw, fw, 8, fw, 8, fy, NULL, NULL, 8, 4, 8, 8, bad_kpa[i], NULL) == E);
    CHECK(cfp32_gemm_separate_add(fw, fw, 8, fw, 8, NULL, NULL, NULL, 8, 4, 8, 8, 16, NULL) == E);
    CHECK(cfp32_gemm_separate_add(fw, fw, 7, fw, 8, fy, NULL, NULL, 8, 4, 8, 8, 16, NULL) == E);
    /* gemm: no output, or only one of c_hi / c_lo */
    CHECK(cfp32_gemm(fw, fw, 8, fw, 8, NULL, NULL, NULL, 8, 4, 8, 8, NULL) == E);
    CHECK(cfp32_gemm(fw, fw, 8, fw, 8, NULL, fy, NULL, 8, 4, 8, 8, NULL) == E);
    /* linear: workspace missing or too small */
    const int64_t rows[] = {64, 1};
    for (int i = 0; i < 2; ++i) {
        size_t need = cfp32_linear_workspace_bytes(rows[i], 64, 64);
        CHECK(need > 0);
        CHECK(cfp32_linear(fx, 64, fw, 64, fy, 64, rows[i], 64, 64, NULL, 0, NULL) == E);
        CHECK(cfp32_linear(fx, 64, fw, 64, fy, 64, rows[i], 64, 64, F, need - 1, NULL) == E);
    }
    /* linear_noalloc: pointers, leading dimensions, sizes; scratch beyond 64 MiB */
    CHECK(cfp32_linear_noalloc(NULL, 8, fw, 8, fy, 8, 2, 8, 8, NULL) == E);
    CHECK(cfp32_linear_noalloc(fx, 7, fw, 8, fy, 8, 2, 8, 8, NULL) == E);
    CHECK(cfp32_linear_noalloc(fx, 8, fw, 8, fy, 7, 2, 8, 8, NULL) == E);
    CHECK(cfp32_linear_noalloc(fx, 8, fw, 8, fy, 8, -2, 8, 8, NULL) == E);
    CHECK(cfp32_linear_noalloc(fx, 1 << 20, fw, 8, fy, 8, 64, 8, 1 << 20, NULL) == CFP32_ERR_TOO_LARGE);
    /* linear_f32 */
    CHECK(cfp32_linear_f32(fx, 7, fw, 8, fy, 8, 2, 8, 8, NULL) == E);
    CHECK(cfp32_linear_f32(fx, 8, NULL, 8, fy, 8, 2, 8, 8, NULL) == E);
    CHECK(cfp32_linear_f32(fx, 8, fw, 8, fy, 8, 2, -8, 8, NULL) == E);
    /* linear_ex: unknown layout; [N, K] weights need ldw >= K */
    CHECK(cfp32_linear_ex(fx, 64, fw, 64, 2, NULL, fy, 64, 2, 64, 64, NULL, 0, NULL) == E);
    CHECK(cfp32_linear_ex(fx, 64, fw, 63, CFP32_W_NK, NULL, fy, 64, 2, 64, 64, NULL, 0, NULL) == E);
    CHECK(cfp32_linear_ex(fx, 64, fw, 32, CFP32_W_NK, NULL, fy, 64, 2, 16, 64, NULL, 0, NULL) == E);
    /* linear_geglu: w narrower than 2F, out narrower than F, small workspace */
    CHECK(cfp32_linear_geglu(fx, 64, fw, 63, NULL, fy, 32, 2, 32, 64, NULL, 0, NULL) == E);
    CHECK(cfp32_linear_geglu(fx, 64, fw, 64, NULL, fy, 31, 2, 32, 64, NULL, 0, NULL) == E);
    size_t gneed = cfp32_linear_geglu_workspace_bytes(2, 32, 64);
    CHECK(gneed > 0);
    CHECK(cfp32_linear_geglu(fx, 64, fw, 64, NULL, fy, 32, 2, 32, 64, F, gneed - 1, NULL) == E);
    /* qkv_rotary: odd D, non-positive theta, ldq below 3 H D, null input */
    CHECK(cfp32_qkv_rotary(fx, 96, NULL, 10000.0, fy, fy, fy, 4, 2, 15, NULL) == E);
    CHECK(cfp32_qkv_rotary(fx, 96, NULL, 0.0, fy, fy, fy, 4, 2, 16, NULL) == E);
    CHECK(cfp32_qkv_rotary(fx, 95, NULL, 10000.0, fy, fy, fy, 4, 2, 16, NULL) == E);
    CHECK(cfp32_qkv_rotary(NULL, 96, NULL, 10000.0, fy, fy, fy, 4, 2, 16, NULL) == E);
    /* extents of 2^48 elements or more, and products near the int64 limit */
    const int64_t big = (int64_t)1 << 40;
    CHECK(cfp32_split(fx, big, fh, fh, big, big, 4, NULL) == E);
    CHECK(cfp32_split(fx, (int64_t)1 << 48, fh, fh, (int64_t)1 << 48, 1, (int64_t)1 << 48, NULL) == E);
    CHECK(cfp32_gemm(fw, fw, (int64_t)1 << 47, fw, 8, fy, NULL, NULL, 8, 2, 8, 8, NULL) == E);
    CHECK(cfp32_gemm(fw, fw, 8, fw, 8, fy, NULL, NULL, 8, 2, 8, (int64_t)1 << 48, NULL) == E);
    CHECK(cfp32_linear(fx, ((int64_t)1 << 47) + 8, fw, 8, fy, 8, 2, 8, 8, F, 1 << 20, NULL) == E);
    CHECK(cfp32_merge(fx, fx, (int64_t)1 << 46, fy, 8, 4, 8, NULL) == E);
    CHECK(cfp32_qkv_rotary(fx, INT64_MAX, NULL, 1.0, fy, fy, fy, 2, INT64_MAX / 2, 2, NULL) == E);
    CHECK(cfp32_linear_geglu_workspace_bytes(2, INT64_MAX / 2, 8) == 0);
    CHECK(cfp32_linear_ex_workspace_bytes(INT64_MAX, INT64_MAX, INT64_MAX, CFP32_W_KN) == 0);

    /* workspace sizes */
    CHECK(cfp32_linear_workspace_bytes(1, 5, 1) == 0);
    CHECK(cfp32_linear_workspace_bytes(-1, 10, 10) == 0);
    CHECK(cfp32_linear_workspace_bytes(4096, 4096, 4096) == (size_t)2 * 4096 * 4096 * 2 + 256);
    CHECK(cfp32_linear_ex_workspace_bytes(1, 14336, 4096, CFP32_W_NK) == 0);
    CHECK(cfp32_linear_ex_workspace_bytes(9, 5, 1, 7) == 0);

    /* empty problems are no-ops */
    CHECK(cfp32_split(NULL, 0, NULL, NULL, 0, 0, 5, NULL) == CFP32_OK);
    CHECK(cfp32_gemm(NULL, NULL, 0, NULL, 0, NULL, NULL, NULL, 0, 0, 8, 8, NULL) == CFP32_OK);
    CHECK(cfp32_merge(NULL, NULL, 0, NULL, 0, 4, 0, NULL) == CFP32_OK);
    CHECK(cfp32_linear(NULL, 0, NULL, 0, NULL, 0, 0, 8, 8, NULL, 0, NULL) == CFP32_OK);
    CHECK(cfp32_linear_noalloc(NULL, 0, NULL, 0, NULL, 0, 5, 0, 8, NULL) == CFP32_OK);
    CHECK(cfp32_linear_f32(NULL, 0, NULL, 0, NULL, 0, 0, 8, 8, NULL) == CFP32_OK);
    CHECK(cfp32_qkv_rotary(NULL, 0, NULL, 10000.0, NULL, NULL, NULL, 0, 4, 8, NULL) == CFP32_OK);

    /* "no-device": a valid call on a machine without a gfx950 device must
     * refuse to run (there is no CPU fallback); the launcher stubs abort if
     * it went further */
    if (argc > 1 && strcmp(argv[1], "no-device") == 0) {
        CHECK(cfp32_split(fx, 4, fh, fh, 4, 1, 4, NULL) == CFP32_ERR_UNSUPPORTED_DEVICE);
        CHECK(cfp32_linear(fx, 8, fw, 8, fy, 8, 2, 8, 8, F, cfp32_linear_workspace_bytes(2, 8, 8), NULL) ==
              CFP32_ERR_UNSUPPORTED_DEVICE);
        CHECK(cfp32_linear_noalloc(fx, 8, fw, 8, fy, 8, 2, 8, 8, NULL) == CFP32_ERR_UNSUPPORTED_DEVICE);
    }
    fprintf(stderr, "abi_driver: %d failure(s)\n", failures);
    return failures == 0 ? 0 : 1;
}
