// Launcher stubs for the host-only sanitizer build of the C ABI: api.hip and
// plans.hip are built with AddressSanitizer and UndefinedBehaviorSanitizer
// and linked against these instead of the kernels.  The checks that run
// against that build never get as far as a launch (they fail validation, are
// empty, or find no gfx950 device), so every stub aborts: reaching one is a
// test failure.
#include <cstdio>
#include <cstdlib>

#include "../../compensated_fp32_projection_amd/csrc/launchers.h"

namespace cfp32 {

[[noreturn]] static void reached(const char *name)
{
    std::fprintf(stderr, "launcher stub reached: %s\n", name);
    std::abort();
}

hipError_t launch_split(const float *x, int64_t ldx, uint16_t *hi, uint16_t *lo, int64_t ldh, int64_t rows, int64_t cols, int64_t cols_out, hipStream_t stream)
{
    reached("launch_split");
}

hipError_t launch_merge(const float *c_hi, const float *c_lo, int64_t ldc, float *y, int64_t ldy, int64_t rows, int64_t cols, hipStream_t stream)
{
    reached("launch_merge");
}

hipError_t launch_pad_rows(const uint16_t *w, int64_t ldw, uint16_t *wp, int64_t ldp, int64_t rows, int64_t cols, int64_t cols_out, hipStream_t stream)
{
    reached("launch_pad_rows");
}

hipError_t launch_gemm(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w, int64_t ldw, float *y, int64_t ldy, float *c_hi, float *c_lo, int64_t ldc, int64_t M, int64_t N, int64_t K, bool a_zero_padded, hipStream_t stream, const float *bias, bool w_nk, bool geglu_rmw)
{
    reached("launch_gemm");
}

hipError_t launch_gemm_separate_add(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w, int64_t ldw, float *y, int64_t ldy, float *c_hi, float *c_lo, int64_t ldc, int64_t M, int64_t N, int64_t K, int k_steps_per_add, hipStream_t stream)
{
    reached("launch_gemm_separate_add");
}

hipError_t launch_gemm_dma(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w, int64_t ldw, float *y, int64_t ldy, float *c_hi, float *c_lo, int64_t ldc, int64_t M, int64_t N, int64_t K, bool a_zero_padded, hipStream_t stream, const float *bias, bool w_nk, int64_t kchunks, float *part, int64_t n_pad)
{
    reached("launch_gemm_dma");
}

hipError_t launch_gemm_chunked(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w, int64_t ldw, float *y, int64_t ldy, int64_t M, int64_t N, int64_t K, bool a_zero_padded, hipStream_t stream, const float *bias, bool w_nk, float *part, size_t part_bytes, bool geglu)
{
    reached("launch_gemm_chunked");
}

hipError_t launch_partial_merge(const float *part, int64_t n_pad, int64_t chunks, int64_t M, int64_t N, float *y, int64_t ldy, const float *bias, hipStream_t stream)
{
    reached("launch_partial_merge");
}

hipError_t launch_partial_geglu_merge(const float *part, int64_t n_pad, int64_t chunks, int64_t M, int64_t F, float *out, int64_t ldo, const float *bias, hipStream_t stream)
{
    reached("launch_partial_geglu_merge");
}

hipError_t launch_gemm_dma_split(const float *a, int64_t lda, const uint16_t *w, int64_t ldw, float *y, int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t stream, const float *bias, bool w_nk)
{
    reached("launch_gemm_dma_split");
}

hipError_t launch_gemm_dma_geglu(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w, int64_t ldw, float *out, int64_t ldo, int64_t M, int64_t F, int64_t K, bool a_zero_padded, hipStream_t stream, const float *bias)
{
    reached("launch_gemm_dma_geglu");
}

hipError_t launch_gemm_f32(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    reached("launch_gemm_f32");
}

hipError_t launch_qkv_rotary(const float *qkv, int64_t ldq, const int64_t *pos, double theta, float *q, float *k, float *v, int64_t T, int64_t H, int64_t D, hipStream_t stream)
{
    reached("launch_qkv_rotary");
}

hipError_t launch_gemv_nk(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t stream, const float *bias)
{
    reached("launch_gemv_nk");
}

hipError_t launch_gemv(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy, int64_t M, int64_t N, int64_t K, float *part, size_t part_bytes, hipStream_t stream, const float *bias, bool geglu_rmw)
{
    reached("launch_gemv");
}

hipError_t launch_gemv_geglu(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *out, int64_t ldo, int64_t M, int64_t F, int64_t K, float *part, size_t part_bytes, hipStream_t stream, const float *bias)
{
    reached("launch_gemv_geglu");
}


hipError_t launch_gemm_ksplit(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t stream, const float *bias, bool w_nk)
{
    reached("launch_gemm_ksplit");
}

hipError_t launch_gemm_xsplit(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t stream, const float *bias, bool w_nk)
{
    reached("launch_gemm_xsplit");
}

hipError_t launch_gemm_ksplit_geglu(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, int64_t up_off, float *out, int64_t ldo, int64_t M, int64_t F, int64_t K, hipStream_t stream, const float *bias)
{
    reached("launch_gemm_ksplit_geglu");
}

}  // namespace cfp32
