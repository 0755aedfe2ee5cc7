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
//     stages of 32 through two LDS buffers, loaded through registers (A as
//     FP32, W as FP16 widened to FP32 on the way into LDS); 72 KiB of LDS
//     and at most 256 registers give two blocks (two waves per SIMD) per CU.
//   * K order inside each 16-deep half of a stage: MFMA step j (0..3) of
//     lane group q = lane / 16 multiplies physical k = 4 q + j.  A and B use
//     the same mapping, so every output still sums each product exactly
//     once; in exchange a lane's four A values (row r, k = 4q .. 4q + 3) and
//     its four B values (column c, the same k) are each one ds_read_b128: A
//     sits in LDS row-major and W column-major ([n][k]), rows padded to 36
//     floats so that the eight lanes of one 128-byte read touch eight
//     different bank groups.  The order does not depend on the stage depth.
//   * Full stages of 16-byte-loadable operands are fetched with raw buffer
//     loads at per-lane offsets (rows past M and columns past N at an offset
//     no buffer reaches, which reads zero): no branch in the main loop, so
//     the compiler's wait for a stage's registers does not also wait for the
//     next stage's loads.  The ragged last stage, and operands that do not
//     allow 16-byte loads, take guarded element loads.  Any M, N, K >= 0
//     works.
#include "device_common.h"
#include "launchers.h"
#include "tile_order.h"

namespace cfp32 {

namespace {

constexpr int kF32Threads = 256;
constexpr int kF32BM = 128, kF32BN = 128, kF32BK = 32;
constexpr int kF32Ld = kF32BK + 4;            // LDS floats per row of a stage (+ 4 pad)
constexpr int kF32Chunks = kF32BK / 16;       // 8-element loads per thread per stage, for A and for W
constexpr int kF32NoOffset = 0x7FFFFFF0;      // a raw buffer load here reads zero
constexpr int kF32Word3 = 0x00020000;         // raw 32-bit buffer, gfx9 family

// BUF: x and W allow 16-byte loads and every byte offset the kernel forms
// stays below 2^31 (checked by the launcher).
template <bool AV, bool WV, bool BUF>
__global__ __launch_bounds__(kF32Threads) void gemm_f32_kernel(const float *__restrict__ A, int64_t lda,
                                                               const uint16_t *__restrict__ W, int64_t ldw,
                                                               float *__restrict__ Y, int64_t ldy, int64_t M,
                                                               int64_t N, int64_t K)
{
    static_assert(!BUF || (AV && WV), "buffer loads need 16-byte-loadable operands");
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

    // Loaders, chunk c = tid + 256 i: A row c / 4, k 8 (c % 4) .. + 7; W
    // k-row c / 16, columns 8 (c % 16) .. + 7.
    int a_row[kF32Chunks], a_k[kF32Chunks], w_k[kF32Chunks], w_n[kF32Chunks];
#pragma unroll
    for (int i = 0; i < kF32Chunks; ++i) {
        const int c = tid + kF32Threads * i;
        a_row[i] = c / (kF32BK / 8);
        a_k[i] = 8 * (c % (kF32BK / 8));
        w_k[i] = c / (kF32BN / 8);
        w_n[i] = 8 * (c % (kF32BN / 8));
    }
    float ra[kF32Chunks][8];
    uint4 rw[kF32Chunks];  // eight FP16 W values, widened when written to LDS

    const __amdgpu_buffer_rsrc_t rs_a =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(A), 0, BUF ? (int)(M * lda * 4) : 0, kF32Word3);
    const __amdgpu_buffer_rsrc_t rs_w =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(W), 0, BUF ? (int)(K * ldw * 2) : 0, kF32Word3);
    int voff_a[kF32Chunks], voff_w[kF32Chunks];
#pragma unroll
    for (int i = 0; i < kF32Chunks; ++i) {
        const int64_t gm = m0 + a_row[i], gn = n0 + w_n[i];
        voff_a[i] = BUF && gm < M ? (int)((gm * lda + a_k[i]) * 4) : kF32NoOffset;
        voff_w[i] = BUF && gn < N ? (int)((w_k[i] * ldw + gn) * 2) : kF32NoOffset;
    }

    // A full stage (k0 + 32 <= K), no branch; the stage's k offset travels
    // in the scalar offset (wave-uniform).
    auto load_stage_buf = [&](int64_t k0) __attribute__((always_inline)) {
        const int so_a = __builtin_amdgcn_readfirstlane((int)(k0 * 4));
        const int so_w = __builtin_amdgcn_readfirstlane((int)(k0 * ldw * 2));
#pragma unroll
        for (int i = 0; i < kF32Chunks; ++i) {
            const floatx4_t v0 = __builtin_bit_cast(floatx4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_a, voff_a[i], so_a, 0));
            const floatx4_t v1 =
                __builtin_bit_cast(floatx4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_a, voff_a[i] + 16, so_a, 0));
#pragma unroll
            for (int e = 0; e < 4; ++e) ra[i][e] = v0[e], ra[i][e + 4] = v1[e];
            rw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_w, voff_w[i], so_w, 0));
        }
    };
    // Any stage: rows past M, k past K and columns past N read as zero.
    auto load_stage = [&](int64_t k0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kF32Chunks; ++i) {
            const int64_t gm = m0 + a_row[i];
            const int64_t gk = k0 + a_k[i];
            if (AV && gm < M && gk + 8 <= K) {
                const floatx4_t v0 = *reinterpret_cast<const floatx4_t *>(A + gm * lda + gk);
                const floatx4_t v1 = *reinterpret_cast<const floatx4_t *>(A + gm * lda + gk + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) ra[i][e] = v0[e], ra[i][e + 4] = v1[e];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) ra[i][e] = (gm < M && gk + e < K) ? A[gm * lda + gk + e] : 0.0f;
            }
            const int64_t wk = k0 + w_k[i];
            rw[i] = wk < K ? load_row8<WV>(W + wk * ldw, n0 + w_n[i], N) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_stage = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kF32Chunks; ++i) {
            float *pa = &sA[buf][a_row[i] * kF32Ld + a_k[i]];
            *reinterpret_cast<floatx4_t *>(pa) = floatx4_t{ra[i][0], ra[i][1], ra[i][2], ra[i][3]};
            *reinterpret_cast<floatx4_t *>(pa + 4) = floatx4_t{ra[i][4], ra[i][5], ra[i][6], ra[i][7]};
            const uint32_t d[4] = {rw[i].x, rw[i].y, rw[i].z, rw[i].w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                sW[buf][(w_n[i] + e) * kF32Ld + w_k[i]] = half_bits_to_float((d[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        }
    };

    floatx4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{};

    auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < kF32BK / 16; ++h) {
            floatx4_t a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *reinterpret_cast<const floatx4_t *>(&sA[buf][(64 * wm + 16 * i + r) * kF32Ld + 16 * h + 4 * q]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = *reinterpret_cast<const floatx4_t *>(&sW[buf][(64 * wn + 16 * j + r) * kF32Ld + 16 * h + 4 * q]);
#pragma unroll
            for (int step = 0; step < 4; ++step)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][step], b[j][step], acc[i][j], 0, 0, 0);
        }
    };

    // Stage s is multiplied out of LDS buffer s & 1 while stage s + 1 is
    // fetched into registers; one barrier per stage.
    const int64_t nk = (K + kF32BK - 1) / kF32BK;
    const int64_t nk_full = BUF ? K / kF32BK : 0;
    if (nk > 0) {
        if (nk_full > 0)
            load_stage_buf(0);
        else
            load_stage(0);
        store_stage(0);
        __syncthreads();
        int64_t s = 0;
        for (; s + 1 < nk_full; ++s) {
            load_stage_buf((s + 1) * kF32BK);
            // Keep the loads ahead of the MFMAs: scheduled after them (to
            // reuse the fragment registers) they would not overlap compute.
            __builtin_amdgcn_sched_barrier(0);
            compute((int)(s & 1));
            store_stage((int)((s + 1) & 1));
            __syncthreads();
        }
        for (; s + 1 < nk; ++s) {
            load_stage((s + 1) * kF32BK);
            compute((int)(s & 1));
            store_stage((int)((s + 1) & 1));
            __syncthreads();
        }
        compute((int)(s & 1));
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
    // Buffer offsets are 32-bit: every byte offset a thread forms, including
    // a tile's overhang past M and N and a stage's past K, stays below this.
    constexpr int64_t kLim = kF32NoOffset - (1 << 20);
    const bool fits = (M + kF32BM) * ldx * 4 < kLim && (K + kF32BK) * ldw * 2 + (int64_t)kF32BN * 2 < kLim;
    const dim3 grid((unsigned)blocks);
    if (av && wv && fits)
        gemm_f32_kernel<true, true, true><<<grid, kF32Threads, 0, stream>>>(x, ldx, w, ldw, y, ldy, M, N, K);
    else if (av && wv)
        gemm_f32_kernel<true, true, false><<<grid, kF32Threads, 0, stream>>>(x, ldx, w, ldw, y, ldy, M, N, K);
    else if (av)
        gemm_f32_kernel<true, false, false><<<grid, kF32Threads, 0, stream>>>(x, ldx, w, ldw, y, ldy, M, N, K);
    else if (wv)
        gemm_f32_kernel<false, true, false><<<grid, kF32Threads, 0, stream>>>(x, ldx, w, ldw, y, ldy, M, N, K);
    else
        gemm_f32_kernel<false, false, false><<<grid, kF32Threads, 0, stream>>>(x, ldx, w, ldw, y, ldy, M, N, K);
    return hipGetLastError();
}

}  // namespace cfp32
