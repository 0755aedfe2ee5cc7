// True-FP32 projection: y = x W with the activations kept in FP32 (no FP16
// conversion) and FP32 products and sums on the matrix unit.
//
// The laya.cpp Vulkan guide's build-time extension adds true FP32 matrix
// kernels next to the compensated ones, so that FP32 operands are never
// converted to FP16 implicitly (true-FP32 paragraph); this is that kernel for
// gfx950, used as the in-run A/B partner of the compensated path (same
// operands: x FP32, W FP16 widened exactly to FP32).
//
//   * v_mfma_f32_16x16x4_f32: FP32 A and B fragments, FP32 accumulators.
//     Its peak is 256 FLOP per clock per CU (157.3 TFLOP/s on MI355X), an
//     eighth of the FP16 rate the compensated path's two products share.
//   * 256 threads (4 waves), a 128 x 128 output tile, each wave 64 x 64:
//     4 x 4 blocks of 16 x 16, 64 accumulators per lane.  K advances in
//     stages of 16 through two LDS buffers, loaded through registers (A as
//     FP32, W as FP16 widened to FP32 on the way into LDS).
//   * K order inside a stage: MFMA step j (0..3) of lane group q = lane / 16
//     multiplies physical k = 4 q + j.  A and B use the same mapping, so every
//     output still sums each product exactly once; in exchange a lane's four
//     A values of a stage (row r, k = 4q .. 4q + 3) and its four B values
//     (column c, the same k) are each one ds_read_b128: A sits in LDS row-major
//     and W column-major ([n][k]), rows padded to 20 floats so that the eight
//     lanes of one 128-byte read touch eight different bank groups.
//   * Out-of-range rows, columns and k read as zero and are not stored: any
//     M, N, K >= 0 works; 16-byte global loads where the pointers and leading
//     dimensions allow them, element loads otherwise.
#include "device_common.h"
#include "launchers.h"
#include "tile_order.h"

namespace cfp32 {

namespace {

constexpr int kF32Threads = 256;
constexpr int kF32BM = 128, kF32BN = 128, kF32BK = 16;
constexpr int kF32Ld = 20;  // LDS floats per row of 16 k (16 + 4 pad)

template <bool AV, bool WV>
__global__ __launch_bounds__(kF32Threads) void gemm_f32_kernel(const float *__restrict__ A, int64_t lda,
                                                               const uint16_t *__restrict__ W, int64_t ldw,
                                                               float *__restrict__ Y, int64_t ldy, int64_t M,
                                                               int64_t N, int64_t K)
{
    __shared__ float sA[2][kF32BM * kF32Ld];
    __shared__ float sW[2][kF32BN * kF32Ld];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int q = lane >> 4, r = lane & 15;

    const int64_t nbm = (M + kF32BM - 1) / kF32BM;
    const int64_t nbn = (N + kF32BN - 1) / kF32BN;
    int64_t tile_m, tile_n;
    tile_of_block(blockIdx.x, nbm, nbn, tile_m, tile_n);
    const int64_t m0 = tile_m * kF32BM, n0 = tile_n * kF32BN;

    // Loaders: A row t / 2, k 8 (t % 2) .. + 7; W k-row t / 16, columns
    // 8 (t % 16) .. + 7.
    const int a_row = tid >> 1, a_k = 8 * (tid & 1);
    const int w_k = tid >> 4, w_n = 8 * (tid & 15);
    float ra[8];
    float rw[8];

    auto load_stage = [&](int64_t k0) {
        const int64_t gm = m0 + a_row;
        const int64_t gk = k0 + a_k;
        if (AV && gm < M && gk + 8 <= K) {
            const floatx4_t v0 = *reinterpret_cast<const floatx4_t *>(A + gm * lda + gk);
            const floatx4_t v1 = *reinterpret_cast<const floatx4_t *>(A + gm * lda + gk + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) ra[e] = v0[e], ra[e + 4] = v1[e];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) ra[e] = (gm < M && gk + e < K) ? A[gm * lda + gk + e] : 0.0f;
        }
        const int64_t wk = k0 + w_k;
        const int64_t wcol = n0 + w_n;
        if (wk < K) {
            const uint4 v = load_row8<WV>(W + wk * ldw, wcol, N);
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) rw[e] = half_bits_to_float((d[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) rw[e] = 0.0f;
        }
    };
    auto store_stage = [&](int buf) {
        float *pa = &sA[buf][a_row * kF32Ld + a_k];
        *reinterpret_cast<floatx4_t *>(pa) = floatx4_t{ra[0], ra[1], ra[2], ra[3]};
        *reinterpret_cast<floatx4_t *>(pa + 4) = floatx4_t{ra[4], ra[5], ra[6], ra[7]};
#pragma unroll
        for (int e = 0; e < 8; ++e) sW[buf][(w_n + e) * kF32Ld + w_k] = rw[e];
    };

    floatx4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{};

    auto compute = [&](int buf) {
        floatx4_t a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = *reinterpret_cast<const floatx4_t *>(&sA[buf][(64 * wm + 16 * i + r) * kF32Ld + 4 * q]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            b[j] = *reinterpret_cast<const floatx4_t *>(&sW[buf][(64 * wn + 16 * j + r) * kF32Ld + 4 * q]);
#pragma unroll
        for (int step = 0; step < 4; ++step)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][step], b[j][step], acc[i][j], 0, 0, 0);
    };

    const int64_t nk = (K + kF32BK - 1) / kF32BK;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int64_t s = 0; s < nk; ++s) {
        const bool more = s + 1 < nk;
        if (more) load_stage((s + 1) * kF32BK);
        compute((int)(s & 1));
        if (more) store_stage((int)((s + 1) & 1));
        __syncthreads();
    }

    // 16 x 16 accumulator: lane holds column r, rows 4 q + e of its block.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + 64 * wn + 16 * j + r;
            if (col >= N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = m0 + 64 * wm + 16 * i + 4 * q + e;
                if (row < M) __builtin_nontemporal_store(acc[i][j][e], Y + row * ldy + col);
            }
        }
}

}  // namespace

hipError_t launch_gemm_f32(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    const int64_t blocks = ((M + kF32BM - 1) / kF32BM) * ((N + kF32BN - 1) / kF32BN);
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const bool av = (ldx % 4 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
    const bool wv = (ldw % 8 == 0) && ((reinterpret_cast<uintptr_t>(w) & 15) == 0);
    const dim3 grid((unsigned)blocks);
    if (av && wv)
        gemm_f32_kernel<true, true><<<grid, kF32Threads, 0, stream>>>(x, ldx, w, ldw, y, ldy, M, N, K);
    else if (av)
        gemm_f32_kernel<true, false><<<grid, kF32Threads, 0, stream>>>(x, ldx, w, ldw, y, ldy, M, N, K);
    else if (wv)
        gemm_f32_kernel<false, true><<<grid, kF32Threads, 0, stream>>>(x, ldx, w, ldw, y, ldy, M, N, K);
    else
        gemm_f32_kernel<false, false><<<grid, kF32Threads, 0, stream>>>(x, ldx, w, ldw, y, ldy, M, N, K);
    return hipGetLastError();
}

}  // namespace cfp32
