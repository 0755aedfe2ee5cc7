// Fused projection for 1 <= M <= 8 rows (decode-sized inputs).
//
// The laya.cpp Vulkan guide runs small projections at their real batch size,
// with no padding of the row count.  At M <= 8 the projection streams W once
// and does almost no arithmetic per byte, so it is bound by HBM bandwidth and
// by launch latency: one kernel does the split, both products and the merge.
//
// gfx950 design
//   * A block owns NB consecutive output columns and all of K.  Its threads
//     form CH = NB/8 column groups (8 FP16 columns = one 16-byte load) times
//     KL = THREADS/CH k-lanes; k-lane kl handles rows kl, kl+KL, kl+2KL, ...
//     A wave reads 64/CH rows x 16*CH contiguous bytes per load instruction.
//   * U loads per thread are issued before any of them is used, to keep
//     enough bytes in flight per CU to cover HBM latency.
//   * x is split in registers (same split as the standalone kernel); both
//     products accumulate in FP32 with fused multiply-adds (an FP16 x FP16
//     product is exact in FP32, so fusing does not change any rounding).
//   * The k-lane partial sums are reduced in a fixed order -- a butterfly
//     inside each wave, then the waves in index order through LDS -- so
//     results are identical from run to run; the merge follows, once per
//     output, after both reductions are complete.
#include "device_common.h"
#include "launchers.h"

namespace cfp32 {

namespace {

constexpr int kNoOffset = 0x7FFFFFF0;      // a raw buffer load here reads zero
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit buffer, gfx9 family
constexpr int kStreamAux = 2;             // cache policy "nt": W is read once, do not keep it in cache

// THREADS threads own NB output columns; U loads per thread in flight.
// BUF: W is 16-byte aligned with ldw % 8 == 0 and under 2^31 bytes, so W is
// read with raw buffer loads whose out-of-range lanes read zero (no branches,
// so all U loads of a thread are in flight together); otherwise W is read
// through the guarded element path.
template <int MR, bool BUF, int THREADS, int NB, int U>
__global__ __launch_bounds__(THREADS) void gemv_kernel(const float *__restrict__ x, int64_t ldx,
                                                       const uint16_t *__restrict__ w, int64_t ldw,
                                                       float *__restrict__ y, int64_t ldy, int64_t N, int64_t K)
{
    constexpr int CH = NB / 8;
    constexpr int KL = THREADS / CH;
    constexpr int WAVES = THREADS / 64;
    static_assert(CH <= 64 && (CH & (CH - 1)) == 0, "column groups are a power of two within a wave");

    __shared__ float red[WAVES][CH][MR][8][2];

    const int tid = threadIdx.x;
    const int c = tid % CH;
    const int kl = tid / CH;
    const int64_t n0 = (int64_t)blockIdx.x * NB;
    const int64_t n = n0 + 8 * c;

    const __amdgpu_buffer_rsrc_t rs_w =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(w), 0, BUF ? (int)(K * ldw * 2) : 0, kBufferWord3);

    float sh[MR][8], sl[MR][8];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) sh[m][e] = 0.0f, sl[m][e] = 0.0f;

    for (int64_t kb = kl; kb < K; kb += (int64_t)KL * U) {
        // x first, then W: the vector-memory counter drains in issue order, so
        // one wait for the last W load covers every x of the batch.
        float xv[U][MR];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = kb + (int64_t)u * KL;
#pragma unroll
            for (int m = 0; m < MR; ++m) xv[u][m] = (k < K) ? x[m * ldx + k] : 0.0f;
        }
        uint4 wv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = kb + (int64_t)u * KL;
            if constexpr (BUF) {
                const int off = (k < K && n < N) ? (int)((k * ldw + n) * 2) : kNoOffset;
                wv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_w, off, 0, kStreamAux));
            } else {
                wv[u] = (k < K) ? load_row8<false>(w + k * ldw, n, N) : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t d[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
            float wf[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) wf[e] = half_bits_to_float((d[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                _Float16 h16, l16;
                split_value(xv[u][m], h16, l16);
                const float h = (float)h16, l = (float)l16;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sh[m][e] = __builtin_fmaf(h, wf[e], sh[m][e]);
                    sl[m][e] = __builtin_fmaf(l, wf[e], sl[m][e]);
                }
            }
        }
    }

    // Butterfly over the k-lanes of this wave (lanes c, c+CH, c+2CH, ...).
#pragma unroll
    for (int sft = CH; sft < 64; sft <<= 1)
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sh[m][e] += __shfl_xor(sh[m][e], sft, 64);
                sl[m][e] += __shfl_xor(sl[m][e], sft, 64);
            }
    const int lane = tid & 63, wave = tid >> 6;
    if (lane < CH) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                red[wave][lane][m][e][0] = sh[m][e];
                red[wave][lane][m][e][1] = sl[m][e];
            }
    }
    __syncthreads();

    // Waves in index order, then the merge; one thread per output.
    for (int o = tid; o < MR * NB; o += THREADS) {
        const int m = o / NB, col = o % NB;
        const int64_t gn = n0 + col;
        if (gn >= N) continue;
        float th = 0.0f, tl = 0.0f;
#pragma unroll
        for (int wv = 0; wv < WAVES; ++wv) {
            th += red[wv][col >> 3][m][col & 7][0];
            tl += red[wv][col >> 3][m][col & 7][1];
        }
        y[m * ldy + gn] = merge_value(th, tl);
    }
}

template <int MR, int THREADS, int NB, int U>
hipError_t launch_cfg(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy,
                      int64_t N, int64_t K, hipStream_t stream)
{
    const int64_t blocks = (N + NB - 1) / NB;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks);
    const bool buf = (ldw % 8 == 0) && ((reinterpret_cast<uintptr_t>(w) & 15) == 0) &&
                     (K + 1) * ldw * 2 < kNoOffset - (1 << 20);
    if (buf)
        gemv_kernel<MR, true, THREADS, NB, U><<<grid, THREADS, 0, stream>>>(x, ldx, w, ldw, y, ldy, N, K);
    else
        gemv_kernel<MR, false, THREADS, NB, U><<<grid, THREADS, 0, stream>>>(x, ldx, w, ldw, y, ldy, N, K);
    return hipGetLastError();
}

// Launch shape per row count: 1024 threads keep more loads in flight while
// the accumulators are few; from three rows on, 512 threads leave each
// thread enough registers for 2 x 8 x M accumulators.
template <int MR>
hipError_t launch_rows(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy,
                       int64_t N, int64_t K, hipStream_t stream)
{
    if constexpr (MR <= 2)
        return launch_cfg<MR, 1024, 64, 8>(x, ldx, w, ldw, y, ldy, N, K, stream);
    else
        return launch_cfg<MR, 512, 64, 8>(x, ldx, w, ldw, y, ldy, N, K, stream);
}

}  // namespace

hipError_t launch_gemv(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    switch (M) {
    case 1: return launch_rows<1>(x, ldx, w, ldw, y, ldy, N, K, stream);
    case 2: return launch_rows<2>(x, ldx, w, ldw, y, ldy, N, K, stream);
    case 3: return launch_rows<3>(x, ldx, w, ldw, y, ldy, N, K, stream);
    case 4: return launch_rows<4>(x, ldx, w, ldw, y, ldy, N, K, stream);
    case 5: return launch_rows<5>(x, ldx, w, ldw, y, ldy, N, K, stream);
    case 6: return launch_rows<6>(x, ldx, w, ldw, y, ldy, N, K, stream);
    case 7: return launch_rows<7>(x, ldx, w, ldw, y, ldy, N, K, stream);
    case 8: return launch_rows<8>(x, ldx, w, ldw, y, ldy, N, K, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace cfp32
