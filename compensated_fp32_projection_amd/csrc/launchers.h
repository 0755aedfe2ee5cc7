// Host-side launchers of the gfx950 kernels (internal to libcfp32).
// Arguments are already validated by api.hip; every launcher only enqueues
// kernels on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cfp32 {

hipError_t launch_split(const float *x, int64_t ldx, uint16_t *hi, uint16_t *lo, int64_t ldh,
                        int64_t rows, int64_t cols, hipStream_t stream);

hipError_t launch_merge(const float *c_hi, const float *c_lo, int64_t ldc, float *y, int64_t ldy,
                        int64_t rows, int64_t cols, hipStream_t stream);

// y (ldy) and/or c_hi, c_lo (ldc) outputs; any of them may be null.
hipError_t launch_gemm(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w,
                       int64_t ldw, float *y, int64_t ldy, float *c_hi, float *c_lo, int64_t ldc,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream);

// Fused split + both products + merge for 1 <= M <= 8.
hipError_t launch_gemv(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y,
                       int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t stream);

constexpr int64_t kGemvMaxRows = 8;

}  // namespace cfp32
