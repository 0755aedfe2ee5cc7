// Small-grid projection in one launch: y = x W for shapes whose 128 x 256
// output tiles are too few to fill the GPU (laya.cpp Vulkan guide,
// compensated-FP32 paragraph: two FP16 products with FP32 accumulators,
// merged as C_hi + C_lo / 1024).
//
//   * A block (4 waves) owns a 32 x 64 output tile, and K is split inside
//     the block: wave w multiplies the 32-deep stages w, w + 4, w + 8, ...
//     of K for the whole tile (2 x 4 blocks of v_mfma_f32_16x16x32_f16 per
//     product, 64 accumulators per lane).  With a quarter of the stages each,
//     the chain of dependent memory round trips per block is a quarter as
//     long as in a K-sequential kernel.
//   * x arrives as FP32 straight into the A-fragment layout (lane l: row
//     l % 16, k = 8 (l / 16) .. + 7, two 16-byte loads per 16-row block) and
//     is split into hi and lo in registers, so no split dispatch runs first.
//   * W goes through a three-stage LDS ring private to each wave, filled by
//     LDS-DMA (four 1 KiB loads per stage: 32 k-rows x 128 bytes), and B
//     fragments are read with ds_read_b64_tr_b16 as in the large GEMM.  The
//     ring is the wave's own, so the loop needs no block barrier: a wave only
//     waits for its own loads (vector-memory count) and its own LDS reads.
//   * The four partial tiles are reduced in a fixed order through LDS,
//     ((w0 + w2) + (w1 + w3)) for C_hi and C_lo separately, then merged
//     (+ bias) and stored by wave 0.  Results repeat bit for bit; they are
//     not the bits of the K-sequential kernels (a different summation order),
//     and they meet the same tolerance.
//   * Needs K % 8 == 0, x and W 16-byte aligned with ldx % 4 == 0 and
//     ldw % 8 == 0, and byte offsets below 2^31; the launcher returns
//     hipErrorNotSupported (nothing enqueued) otherwise.
#include "device_common.h"
#include "launchers.h"

#define CFP32_LDS __attribute__((address_space(3)))

namespace cfp32 {

namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));

constexpr int kKsWaves = 4;
constexpr int kKsThreads = 64 * kKsWaves;
constexpr int kKsBM = kKsplitTileM, kKsBN = kKsplitTileN, kKsBK = 32;
constexpr int kKsTM = kKsBM / 16, kKsTN = kKsBN / 16;  // 16x16 blocks per product: 2 x 4
constexpr int kKsRing = 3;                               // stages in flight per wave
constexpr int kKsSlots = kKsBK * kKsBN / 8;              // W granules per wave and stage (256 = 4 KiB)
constexpr int kKsLoads = 2 * kKsTM + kKsSlots / 64;      // loads per wave and stage: 4 x, 4 W
constexpr int kKsNoOffset = 0x7FFFFFF0;
constexpr int kKsWord3 = 0x00020000;

// One LDS object per ring buffer (each holds the four waves' buffers), so
// the compiler can tell which buffer an LDS-DMA load fills.  After the loop
// the three objects hold the partial tiles of the reduction (16 KiB each).
__shared__ uint4 g_ks0[kKsWaves * kKsSlots];
__shared__ uint4 g_ks1[kKsWaves * kKsSlots];
__shared__ uint4 g_ks2[kKsWaves * kKsSlots];

template <int B>
__device__ __forceinline__ uint4 *ks_buf()
{
    if constexpr (B == 0) return g_ks0;
    else if constexpr (B == 1) return g_ks1;
    else return g_ks2;
}

// Granule of W stage row k (0..31) holding columns 8 ng .. 8 ng + 7 sits at
// slot 8 k + (ng ^ ks_swz(k)).  A transposed read touches 16 k-rows (k and
// k + 8, 16, 24 of four consecutive k) and two granules of each; rows are
// 128 bytes, so two rows share a 256-byte bank window, and XOR-ing granule
// bits 1-2 with k bits 3-4 spreads the 32 granules read over all 16 slots of
// the window twice: two passes, the minimum for 512 bytes.
__device__ __forceinline__ int ks_swz(int k) { return ((k >> 3) & 3) << 1; }

__device__ __forceinline__ void ks_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt immediates (gfx9 encoding): vector-memory count n and LDS
// count 0, or vector-memory count n alone.
constexpr int ks_wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (0 << 8); }
constexpr int ks_wait_lgkm0() { return 15 | (3 << 14) | (7 << 4) | (0 << 8); }

// WNK: W given as [N, K] (ldw >= K): each wave's stage holds 64 columns x 4
// k-granules of 16 bytes, granule kg of column n at slot 4 n + (kg ^ ((n >> 2)
// & 3)), and a B fragment is one ds_read_b128 (no transpose).  Same
// products in the same order: the bits of the [K, N] form.
//
// GEGLU ([K, N] W with N = 2F, gate columns then up columns; the feed-
// forward GEGLU of the laya.cpp Vulkan guide's graph paragraph): a block
// owns 32 output columns, its 64 W columns being their gate columns (tile
// columns 0-31) and up columns (32-63), so lane l holds the gate and the up
// of the same output in column blocks j and j + 2 and writes
// gelu(gate + b_gate) * (up + b_up).  Every gate and up sum is the one the
// plain kernel forms for that column of the [K, 2F] projection.  The up
// columns start at W column up_off (F, or F rounded up to 8 in a padded
// copy of W), which must keep them 16-byte aligned.
template <bool WNK, bool GEGLU = false>
__global__ __launch_bounds__(kKsThreads) void gemm_ksplit_kernel(const float *__restrict__ x, int64_t ldx,
                                                                 const uint16_t *__restrict__ w, int64_t ldw,
                                                                 float *__restrict__ y, int64_t ldy,
                                                                 const float *__restrict__ bias, int M, int N,
                                                                 int K, int up_off = 0)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    static_assert(!(WNK && GEGLU), "GEGLU takes [K, 2F] weights");
    const int F = N / 2;  // GEGLU: output columns; their up columns start at W column up_off
    // Tiles row by row in block order.  Blocks go to the 8 XCDs round-robin,
    // so with 8 | tiles per row each XCD reads an eighth of W's columns for
    // every row of tiles (256 x 4096 x 4096: 47 us; regrouped so that each
    // XCD ran whole rows of tiles, and so all of W: 55 us).
    const int nbn = GEGLU ? (F + kKsBN / 2 - 1) / (kKsBN / 2) : (N + kKsBN - 1) / kKsBN;
    const int m0 = ((int)blockIdx.x / nbn) * kKsBM;
    const int n0 = ((int)blockIdx.x % nbn) * (GEGLU ? kKsBN / 2 : kKsBN);  // GEGLU: first output column
    const int nst = (K + kKsBK - 1) / kKsBK;
    const int iters = (nst + kKsWaves - 1) / kKsWaves;  // stages per wave (the last ones may lie past K)

    const __amdgpu_buffer_rsrc_t rs_x =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(x), 0, (int)((int64_t)M * ldx * 4), kKsWord3);
    const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(w), 0, (int)((int64_t)(WNK ? N : K) * ldw * 2), kKsWord3);

    // x: lane's rows m0 + 16 i + l % 16 at k = 8 (l / 16) of each stage.
    const int kq = lane >> 4;
    int x_off[kKsTM];
#pragma unroll
    for (int i = 0; i < kKsTM; ++i) {
        const int row = m0 + 16 * i + (lane & 15);
        x_off[i] = row < M ? (int)(((int64_t)row * ldx + 8 * kq) * 4) : -1;
    }
    // W: load d (0..3) of a stage fills slots 64 d + l.  [K, N]: stage rows
    // 8 d + l / 8, slot l % 8 of each, with the granule that belongs there.
    // [N, K]: columns 16 d + l / 4, slot l % 4 of each.  w_row: the k offset
    // of the load's granule within the stage.
    int w_off[kKsSlots / 64];
    int w_row[kKsSlots / 64];
#pragma unroll
    for (int d = 0; d < kKsSlots / 64; ++d) {
        if constexpr (WNK) {
            const int c = 16 * d + (lane >> 2);
            const int kg = (lane & 3) ^ ((c >> 2) & 3);
            w_row[d] = 8 * kg;
            w_off[d] = n0 + c < N ? (int)(((int64_t)(n0 + c) * ldw + 8 * kg) * 2) : -1;
        } else {
            const int r = 8 * d + (lane >> 3);
            const int g = (lane & 7) ^ ks_swz(r);  // tile columns 8 g .. 8 g + 7
            int col = n0 + 8 * g;
            bool in = col < N;
            if constexpr (GEGLU) {  // granules 0-3: gate columns, 4-7: the same outputs' up columns
                const int oc = n0 + 8 * (g & 3);
                in = oc < F;
                col = oc + (g >= 4 ? up_off : 0);
            }
            w_row[d] = r;
            w_off[d] = in ? (int)(((int64_t)r * ldw + col) * 2) : -1;
        }
    }

    floatx4_t xr[kKsRing][kKsTM][2];  // raw FP32 x of the stages in flight
    auto issue = [&](auto buf_tag, int t) __attribute__((always_inline)) {
        constexpr int B = decltype(buf_tag)::value;
        const int k0 = kKsBK * (wave + kKsWaves * t);  // >= K: every load a zero load
#pragma unroll
        for (int i = 0; i < kKsTM; ++i) {
            const bool ok = (x_off[i] >= 0) & (k0 + 8 * kq < K);
            const int o = ok ? x_off[i] + 4 * k0 : kKsNoOffset;  // below 2^31 when ok (launcher)
            const int o2 = ok ? o + 16 : kKsNoOffset;
            xr[B][i][0] = __builtin_bit_cast(floatx4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_x, o, 0, 0));
            xr[B][i][1] = __builtin_bit_cast(floatx4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_x, o2, 0, 0));
        }
        uint4 *dst = ks_buf<B>() + wave * kKsSlots;
#pragma unroll
        for (int d = 0; d < kKsSlots / 64; ++d) {
            const bool ok = (w_off[d] >= 0) & (k0 + w_row[d] < K);
            const int64_t o64 = (int64_t)w_off[d] + (WNK ? (int64_t)k0 * 2 : (int64_t)k0 * ldw * 2);
            const int o = ok ? (int)o64 : kKsNoOffset;  // o64 < 2^31 when ok (launcher)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_w, (CFP32_LDS void *)(dst + 64 * d), 16, o, 0, 0, 0);
        }
    };

    floatx4_t acc_hi[kKsTM][kKsTN], acc_lo[kKsTM][kKsTN];
#pragma unroll
    for (int i = 0; i < kKsTM; ++i)
#pragma unroll
        for (int j = 0; j < kKsTN; ++j) acc_hi[i][j] = floatx4_t{}, acc_lo[i][j] = floatx4_t{};

    // B fragment of column block j: lane l reads stage rows 8 (l / 16) +
    // (l % 16) / 4 + 4 h at columns 16 j + 4 (l % 4) .. + 3.
    const int b_k0 = 8 * kq + ((lane & 15) >> 2);
    const int b_c0 = 4 * (lane & 3);
    auto compute = [&](auto buf_tag) __attribute__((always_inline)) {
        constexpr int B = decltype(buf_tag)::value;
        const uint4 *src = ks_buf<B>() + wave * kKsSlots;
        half8_t bw[kKsTN];
#pragma unroll
        for (int j = 0; j < kKsTN; ++j) {
            if constexpr (WNK) {
                const int n = 16 * j + (lane & 15);
                bw[j] = __builtin_bit_cast(half8_t, src[4 * n + (kq ^ ((n >> 2) & 3))]);
                continue;
            }
            const int c = 16 * j + b_c0;
            short4_t t[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = b_k0 + 4 * h;
                const int byte = (8 * k + ((c >> 3) ^ ks_swz(k))) * 16 + (c & 7) * 2;
                t[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CFP32_LDS short4_t *)((CFP32_LDS char *)src + byte));
            }
            const short8_t v = {t[0][0], t[0][1], t[0][2], t[0][3], t[1][0], t[1][1], t[1][2], t[1][3]};
            bw[j] = __builtin_bit_cast(half8_t, v);
        }
#pragma unroll
        for (int i = 0; i < kKsTM; ++i) {
            half8_t ah, al;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                _Float16 hh, ll;
                split_value(xr[B][i][e >> 2][e & 3], hh, ll);
                ah[e] = hh;
                al[e] = ll;
            }
#pragma unroll
            for (int j = 0; j < kKsTN; ++j) {
                acc_hi[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bw[j], acc_hi[i][j], 0, 0, 0);
                acc_lo[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bw[j], acc_lo[i][j], 0, 0, 0);
            }
        }
    };

    // Stage t of this wave: its loads landed once at most the loads of the
    // two stages after it are pending (the counter completes in order); after
    // the fragment reads of buffer t % 3 are done it is refilled with t + 3.
    auto step = [&](auto buf_tag, int t) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(ks_wait_vm_lgkm0((kKsRing - 1) * kKsLoads));
        compute(buf_tag);
        __builtin_amdgcn_s_waitcnt(ks_wait_lgkm0());
        issue(buf_tag, t + kKsRing);
    };

    issue(std::integral_constant<int, 0>{}, 0);
    issue(std::integral_constant<int, 1>{}, 1);
    issue(std::integral_constant<int, 2>{}, 2);
    int t = 0;
    for (; t + kKsRing <= iters; t += kKsRing) {
        step(std::integral_constant<int, 0>{}, t);
        step(std::integral_constant<int, 1>{}, t + 1);
        step(std::integral_constant<int, 2>{}, t + 2);
    }
    if (t < iters) step(std::integral_constant<int, 0>{}, t);
    if (t + 1 < iters) step(std::integral_constant<int, 1>{}, t + 1);
    __builtin_amdgcn_s_waitcnt(ks_wait_vm_lgkm0(0));  // the trailing zero loads land before LDS is reused
    // The wait counts above count the x register loads of every stage; those
    // of the stages past the end have no reader, and a load whose value is
    // unused may be deleted, which would shift the counts.  Reading the
    // registers here keeps every one of them issued.
#pragma unroll
    for (int b = 0; b < kKsRing; ++b)
#pragma unroll
        for (int i = 0; i < kKsTM; ++i) asm volatile("" ::"v"(xr[b][i][0]), "v"(xr[b][i][1]));

    // Reduction: partial tile element e of lane l at float e * 64 + l of a
    // 16 KiB region (C_hi in e < 32, C_lo above).
    auto put = [&](float *region) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kKsTM; ++i)
#pragma unroll
            for (int j = 0; j < kKsTN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int q = (i * kKsTN + j) * 4 + e;
                    region[q * 64 + lane] = acc_hi[i][j][e];
                    region[(q + 32) * 64 + lane] = acc_lo[i][j][e];
                }
    };
    auto add = [&](const float *region) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kKsTM; ++i)
#pragma unroll
            for (int j = 0; j < kKsTN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int q = (i * kKsTN + j) * 4 + e;
                    acc_hi[i][j][e] = acc_hi[i][j][e] + region[q * 64 + lane];
                    acc_lo[i][j][e] = acc_lo[i][j][e] + region[(q + 32) * 64 + lane];
                }
    };
    float *r0 = reinterpret_cast<float *>(g_ks0);
    float *r1 = reinterpret_cast<float *>(g_ks1);
    float *r2 = reinterpret_cast<float *>(g_ks2);
    ks_barrier();  // every wave's ring reads are done: the buffers become the reduction's regions
    if (wave == 2) put(r0);
    if (wave == 3) put(r1);
    __builtin_amdgcn_s_waitcnt(ks_wait_lgkm0());
    ks_barrier();
    if (wave == 0) add(r0);
    if (wave == 1) add(r1);
    if (wave == 1) put(r2);
    __builtin_amdgcn_s_waitcnt(ks_wait_lgkm0());
    ks_barrier();
    if (wave != 0) return;
    add(r2);

    // 16x16 accumulator: lane l holds column l % 16, rows 4 (l / 16) + e.
    if constexpr (GEGLU) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + 16 * j + (lane & 15);
            if (col >= F) continue;
            const float bg = bias ? bias[col] : 0.0f;
            const float bu = bias ? bias[F + col] : 0.0f;
#pragma unroll
            for (int i = 0; i < kKsTM; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = m0 + 16 * i + 4 * kq + e;
                    if (row >= M) continue;
                    float gate = merge_value(acc_hi[i][j][e], acc_lo[i][j][e]);
                    float up = merge_value(acc_hi[i][j + 2][e], acc_lo[i][j + 2][e]);
                    if (bias) {
                        gate = gate + bg;
                        up = up + bu;
                    }
                    __builtin_nontemporal_store(gelu_value(gate) * up, y + (int64_t)row * ldy + col);
                }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < kKsTN; ++j) {
        const int col = n0 + 16 * j + (lane & 15);
        if (col >= N) continue;
        const float b = bias ? bias[col] : 0.0f;
#pragma unroll
        for (int i = 0; i < kKsTM; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + 16 * i + 4 * kq + e;
                if (row >= M) continue;
                float v = merge_value(acc_hi[i][j][e], acc_lo[i][j][e]);
                if (bias) v = v + b;
                __builtin_nontemporal_store(v, y + (int64_t)row * ldy + col);
            }
    }
}

}  // namespace

hipError_t launch_gemm_ksplit(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy,
                              int64_t M, int64_t N, int64_t K, hipStream_t stream, const float *bias, bool w_nk)
{
    if (!ksplit_supported(x, ldx, w, ldw, M, N, K, w_nk)) return hipErrorNotSupported;
    const int64_t blocks = ksplit_blocks(M, N);
    if (blocks > 0x7FFFFFFF) return hipErrorNotSupported;
    if (w_nk)
        gemm_ksplit_kernel<true><<<dim3((unsigned)blocks), kKsThreads, 0, stream>>>(x, ldx, w, ldw, y, ldy, bias,
                                                                                    (int)M, (int)N, (int)K);
    else
        gemm_ksplit_kernel<false><<<dim3((unsigned)blocks), kKsThreads, 0, stream>>>(x, ldx, w, ldw, y, ldy, bias,
                                                                                     (int)M, (int)N, (int)K);
    return hipGetLastError();
}

hipError_t launch_gemm_ksplit_geglu(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, int64_t up_off,
                                    float *out, int64_t ldo, int64_t M, int64_t F, int64_t K, hipStream_t stream,
                                    const float *bias)
{
    if (F <= 0 || up_off % 8 || up_off < F || up_off + F > ldw || up_off >= ((int64_t)1 << 30) ||
        !ksplit_supported(x, ldx, w, ldw, M, up_off + F, K, false))
        return hipErrorNotSupported;
    const int64_t blocks = ((M + kKsBM - 1) / kKsBM) * ((F + kKsBN / 2 - 1) / (kKsBN / 2));
    if (blocks > 0x7FFFFFFF) return hipErrorNotSupported;
    gemm_ksplit_kernel<false, true><<<dim3((unsigned)blocks), kKsThreads, 0, stream>>>(
        x, ldx, w, ldw, out, ldo, bias, (int)M, (int)(2 * F), (int)K, (int)up_off);
    return hipGetLastError();
}

}  // namespace cfp32
