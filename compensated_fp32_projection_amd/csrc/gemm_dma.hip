// Dual-product MFMA GEMM, main variant: operands go from HBM straight into
// LDS (buffer_load ... lds), through a four-stage ring.
//
// Same arithmetic as the generic kernel in gemm.hip (C_hi = A_hi W and
// C_lo = A_lo W with FP32 accumulators, y = C_hi + C_lo / 1024 merged once in
// the epilogue; laya.cpp Vulkan guide, compensated-FP32 paragraph), organised
// for gfx950:
//   * 256 threads, a 128 x 256 output tile (256 x 256 with the hi and lo rows),
//     each wave 64 x 128 of both products: 256 FP32 accumulators per lane.
//   * K in stages of 32.  Each stage (A_hi, A_lo: 128 x 32 FP16; W: 32 x 256
//     FP16; 32 KiB) is fetched by 32 wave-wide 1 KiB LDS-DMA loads that need
//     no registers, so three stages are in flight while a fourth is used.
//     A wave waits for its own loads of the next stage (vmcnt), then a bare
//     s_barrier publishes every wave's loads; the ring buffers are separate
//     LDS objects so the compiler can tell the DMA targets from the reads.
//   * A sits in LDS as 16-byte k-granules, row-major, the granule order of
//     each row XOR-ed with bits of the row index; an MFMA A fragment is one
//     conflict-free ds_read_b128.  W sits N-contiguous (as in memory), the
//     granule order of each k-row XOR-ed with the row's low bits; an MFMA B
//     fragment (8 consecutive k of one column) is two ds_read_b64_tr_b16,
//     the gfx950 LDS transpose read: in each 16-lane group, lane j's element
//     e comes from element j%4 of the 8 bytes addressed by lane j/4 + 4e.
//   * Loads outside the matrices get an offset no buffer reaches and read as
//     zero, so partial tiles need no branches.
#include <type_traits>

#include "device_common.h"
#include "launchers.h"
#include "tile_order.h"

#define CFP32_LDS __attribute__((address_space(3)))

namespace cfp32 {

namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));

constexpr int kT = 256;
constexpr int BM = 128, BN = 256, BK = 32, NST = 4;
constexpr int KG = BK / 8;                          // k-granules per A row per stage
constexpr int A_SLOTS = BM * KG;                    // granules per A plane per stage
constexpr int WG = BN / 8;                          // granules per W row
constexpr int W_SLOTS = BK * WG;                    // granules of W per stage
constexpr int STAGE_SLOTS = 2 * A_SLOTS + W_SLOTS;  // 2048 granules = 32 KiB
constexpr int kNoOffset = 0x7FFFFFF0;
constexpr int kBufferWord3 = 0x00020000;

static_assert(A_SLOTS % (64 * 4) == 0 && W_SLOTS % (64 * 4) == 0, "DMA loads split evenly over 4 waves");

__shared__ uint4 g_stage0[STAGE_SLOTS];
__shared__ uint4 g_stage1[STAGE_SLOTS];
__shared__ uint4 g_stage2[STAGE_SLOTS];
__shared__ uint4 g_stage3[STAGE_SLOTS];

template <int S>
__device__ __forceinline__ uint4 *stage_buf()
{
    if constexpr (S == 0) return g_stage0;
    else if constexpr (S == 1) return g_stage1;
    else if constexpr (S == 2) return g_stage2;
    else return g_stage3;
}

__device__ __forceinline__ int a_slot(int plane, int row, int kg)
{
    return plane * A_SLOTS + row * KG + (kg ^ ((row >> 2) & 3));
}

__device__ __forceinline__ int w_slot(int k, int ng)
{
    return 2 * A_SLOTS + k * WG + (ng ^ ((k & 3) << 2));
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void block_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

struct DmaArgs {
    const uint16_t *a_hi;
    const uint16_t *a_lo;
    int64_t lda;
    const uint16_t *w;
    int64_t ldw;
    float *y;
    int64_t ldy;
    float *c_hi;
    float *c_lo;
    int64_t ldc;
    int64_t M, N, K;
    int64_t Ka;  // columns of A that may be read: K, or K rounded up to 8 when A is zero-padded
};

__global__ __launch_bounds__(kT) void gemm_dma_kernel(DmaArgs g)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;

    const int64_t nbm = (g.M + BM - 1) / BM;
    const int64_t nbn = (g.N + BN - 1) / BN;
    int64_t tile_m, tile_n;
    tile_of_block(blockIdx.x, nbm, nbn, tile_m, tile_n);
    const int64_t m0 = tile_m * BM;
    const int64_t n0 = tile_n * BN;

    const __amdgpu_buffer_rsrc_t rs_hi =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(g.a_hi), 0, (int)(g.M * g.lda * 2), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rs_lo =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(g.a_lo), 0, (int)(g.M * g.lda * 2), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rs_w =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(g.w), 0, (int)(g.K * g.ldw * 2), kBufferWord3);

    // Which granule this lane fetches in each of its DMA loads.  Load j of a
    // plane fills slots 64j .. 64j+63; lane i fills slot 64j + i.  The byte
    // offsets of stage 0 are formed once; a stage adds 2*k0 (A) or
    // 2*k0*ldw (W).  Granules outside the operands use kNoOffset.
    int a_off[2], a_kend[2], w_off[4], w_kend[4];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int slot = 64 * (2 * wave + jj) + lane;
        const int row = slot / KG;
        const int kg = (slot % KG) ^ ((row >> 2) & 3);
        const bool ok = m0 + row < g.M;
        a_off[jj] = ok ? (int)(((m0 + row) * g.lda + 8 * kg) * 2) : kNoOffset;
        a_kend[jj] = ok ? (int)(g.Ka - 8 * kg) : 0;  // stage k0 reads this granule while k0 < a_kend
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int slot = 64 * (4 * wave + jj) + lane;
        const int k = slot / WG;
        const int ng = (slot % WG) ^ ((k & 3) << 2);
        const bool ok = n0 + 8 * ng < g.N;
        w_off[jj] = ok ? (int)((k * g.ldw + n0 + 8 * ng) * 2) : kNoOffset;
        w_kend[jj] = ok ? (int)(g.K - k) : 0;
    }

    auto issue = [&](auto stage_tag, int64_t k0_64) {
        constexpr int S = decltype(stage_tag)::value;
        uint4 *s = stage_buf<S>();
        const int k0 = (int)k0_64;
        const int wstep = (int)(k0_64 * g.ldw * 2);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int j = 2 * wave + jj;
            const int off = k0 < a_kend[jj] ? a_off[jj] + 2 * k0 : kNoOffset;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_hi, (CFP32_LDS void *)(s + 64 * j), 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_lo, (CFP32_LDS void *)(s + A_SLOTS + 64 * j), 16, off, 0, 0, 0);
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int j = 4 * wave + jj;
            const int off = k0 < w_kend[jj] ? w_off[jj] + wstep : kNoOffset;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_w, (CFP32_LDS void *)(s + 2 * A_SLOTS + 64 * j), 16, off, 0, 0, 0);
        }
    };

    floatx16_t acc_hi[2][4], acc_lo[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc_hi[i][j] = floatx16_t{}, acc_lo[i][j] = floatx16_t{};

    struct Frags {
        half8_t ah[2], al[2], bw[4];
    };
    // Per-lane parts of the fragment addresses.
    const int a_row0 = wm * 64 + (lane & 31);
    const int b_kl = 8 * (lane >> 5) + ((lane & 15) >> 2);                 // + 16 ks + 4 h
    const int b_n0 = wn * 128 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // + 32 tn

    auto read_frags = [&](const uint4 *s, int ks, Frags &f) {
        const int kg = 2 * ks + (lane >> 5);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = a_row0 + 32 * i;
            f.ah[i] = __builtin_bit_cast(half8_t, s[a_slot(0, row, kg)]);
            f.al[i] = __builtin_bit_cast(half8_t, s[a_slot(1, row, kg)]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = b_n0 + 32 * j;
            short4_t t[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = 16 * ks + 4 * h + b_kl;
                const int byte = w_slot(k, n >> 3) * 16 + (n & 7) * 2;
                t[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (CFP32_LDS short4_t *)((CFP32_LDS char *)s + byte));
            }
            typedef short short8_t __attribute__((ext_vector_type(8)));
            const short8_t v = {t[0][0], t[0][1], t[0][2], t[0][3], t[1][0], t[1][1], t[1][2], t[1][3]};
            f.bw[j] = __builtin_bit_cast(half8_t, v);
        }
    };
    auto mfmas = [&](const Frags &f) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc_hi[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.ah[i], f.bw[j], acc_hi[i][j], 0, 0, 0);
                acc_lo[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.al[i], f.bw[j], acc_lo[i][j], 0, 0, 0);
            }
    };

    const int64_t nk = (g.Ka + BK - 1) / BK;

    // Software pipeline over K stages (ring of NST = 4 LDS buffers).
    // Invariant at the top of step s: the fragments of stage s are in
    // registers (set F), the loads of stages s+1, s+2, s+3 are in flight
    // (8 per wave each), and buffer s&3 is free once every wave's reads of
    // it have completed.  Step s:
    //   1. wait until this wave's reads are done (lgkmcnt 0) and 16 loads
    //      remain (stage s+1 landed), then a barrier: stage s+1 is complete
    //      for every wave and nobody reads buffer s&3 any more;
    //   2. refill buffer s&3 with stage s+4;
    //   3. read stage s+1's fragments into the other register set;
    //   4. run stage s's 32 MFMAs, which overlap step 3's LDS reads.
    // Stages past the end are issued too: all their offsets fall outside the
    // operands, so they read zeros into a buffer nobody reads, and the wait
    // count stays one constant.
    auto read_stage = [&](const uint4 *buf, Frags (&f)[2]) {
        read_frags(buf, 0, f[0]);
        read_frags(buf, 1, f[1]);
    };
    auto step = [&](auto stage_tag, int64_t s, Frags (&cur)[2], Frags (&nxt)[2]) {
        constexpr int S = decltype(stage_tag)::value;
        __builtin_amdgcn_s_waitcnt((16 & 15) | (1 << 14) | (7 << 4) | (0 << 8));  // vmcnt(16) lgkmcnt(0)
        block_barrier();
        issue(std::integral_constant<int, S>{}, (s + 4) * BK);
        read_stage(stage_buf<(S + 1) & 3>(), nxt);
        mfmas(cur[0]);
        mfmas(cur[1]);
        // Instruction order for the scheduler: the 8 DMA loads and 24 LDS
        // reads of this step are threaded between the first 16 of its 32
        // MFMAs (MFMA, load, 2 reads; then MFMA, read), so the matrix pipe is
        // fed while they issue instead of idling behind a block of them.
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read (the DMA)
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    };

    Frags fa[2], fb[2];
    issue(std::integral_constant<int, 0>{}, 0);
    issue(std::integral_constant<int, 1>{}, BK);
    issue(std::integral_constant<int, 2>{}, 2 * BK);
    issue(std::integral_constant<int, 3>{}, 3 * BK);
    wait_vmcnt<24>();
    block_barrier();
    read_stage(stage_buf<0>(), fa);
    const int64_t nk4 = nk / NST * NST;
    for (int64_t s0 = 0; s0 < nk4; s0 += NST) {
        step(std::integral_constant<int, 0>{}, s0, fa, fb);
        step(std::integral_constant<int, 1>{}, s0 + 1, fb, fa);
        step(std::integral_constant<int, 2>{}, s0 + 2, fa, fb);
        step(std::integral_constant<int, 3>{}, s0 + 3, fb, fa);
    }
    if (nk4 < nk) step(std::integral_constant<int, 0>{}, nk4, fa, fb);
    if (nk4 + 1 < nk) step(std::integral_constant<int, 1>{}, nk4 + 1, fb, fa);
    if (nk4 + 2 < nk) step(std::integral_constant<int, 2>{}, nk4 + 2, fa, fb);
    wait_vmcnt<0>();  // drain the trailing zero loads before the block exits

    // Epilogue.  32x32 accumulator layout: lane holds column (lane & 31);
    // element e holds row 8*(e/4) + 4*(lane/32) + (e%4) of the block.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + wn * 128 + j * 32 + (lane & 31);
            if (col >= g.N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (row >= g.M) continue;
                const float h = acc_hi[i][j][e], l = acc_lo[i][j][e];
                // Outputs are written once: non-temporal stores keep them from
                // evicting the A and W panels other tiles still read from L2.
                if (g.y) __builtin_nontemporal_store(merge_value(h, l), g.y + row * g.ldy + col);
                if (g.c_hi) {
                    __builtin_nontemporal_store(h, g.c_hi + row * g.ldc + col);
                    __builtin_nontemporal_store(l, g.c_lo + row * g.ldc + col);
                }
            }
        }
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

// Runs the LDS-DMA kernel when the operands allow it; returns
// hipErrorNotSupported (and enqueues nothing) otherwise.  a_zero_padded: the
// columns of A from K up to the next multiple of 8 hold +0 and may be read.
hipError_t launch_gemm_dma(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w,
                           int64_t ldw, float *y, int64_t ldy, float *c_hi, float *c_lo, int64_t ldc,
                           int64_t M, int64_t N, int64_t K, bool a_zero_padded, hipStream_t stream)
{
    if (K <= 0 || lda % 8 || ldw % 8 || !aligned16(a_hi) || !aligned16(a_lo) || !aligned16(w))
        return hipErrorNotSupported;
    const int64_t Ka = (K % 8 == 0) ? K : (a_zero_padded ? (K + 7) / 8 * 8 : -1);
    if (Ka < 0 || Ka > lda) return hipErrorNotSupported;
    // Every byte offset a lane forms (including a tile's overhang) stays below kNoOffset.
    constexpr int64_t kLim = kNoOffset - (1 << 20);
    if ((M + BM) * lda * 2 >= kLim || (K + BK) * ldw * 2 + (int64_t)BN * 2 >= kLim) return hipErrorNotSupported;
    const int64_t blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    if (blocks > 0x7FFFFFFF) return hipErrorNotSupported;
    DmaArgs g{a_hi, a_lo, lda, w, ldw, y, ldy, c_hi, c_lo, ldc, M, N, K, Ka};
    gemm_dma_kernel<<<dim3((unsigned)blocks), kT, 0, stream>>>(g);
    return hipGetLastError();
}

}  // namespace cfp32
