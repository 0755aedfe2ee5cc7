// Dual-product MFMA GEMM, main variant: operands go from HBM straight into
// LDS (buffer_load ... lds) through a four-stage ring, and two waves per SIMD
// take turns on the matrix unit ("ping-pong").
//
// Same arithmetic as the generic kernel in gemm.hip (C_hi = A_hi W and
// C_lo = A_lo W with FP32 accumulators, y = C_hi + C_lo / 1024 merged once in
// the epilogue; laya.cpp Vulkan guide, compensated-FP32 paragraph), organised
// for gfx950:
//   * 512 threads (8 waves, 2 per SIMD), a 128 x 256 output tile (256 x 256
//     with the hi and lo rows).  Each wave owns 64 rows x 64 columns of both
//     products: 4 x 4 blocks of v_mfma_f32_16x16x32_f16 per product, 128
//     FP32 accumulators per lane.  Every W fragment feeds four hi and four
//     lo MFMAs.  The 16x16x32 form was measured against 32x32x16 blocks of
//     the same wave tile (same LDS traffic, same results bit for bit): on
//     normal-distributed data the chip runs at its power limit, and the
//     16x16 form, with a quarter of the accumulator registers per
//     instruction, draws less per product (8192 x 4096 x 14336: 1640 ->
//     1530 us).
//   * K in stages of 32.  Each stage (A_hi, A_lo: 128 x 32 FP16; W: 32 x 256
//     FP16; 32 KiB) is fetched by 32 wave-wide 1 KiB LDS-DMA loads (4 per
//     wave) that need no registers; three stages are in flight.
//   * Waves 0-3 and waves 4-7 form two groups, one wave of each per SIMD.  A
//     wave alternates a memory phase (read its fragments of stage s from LDS,
//     issue its loads of stage s+3, wait for them) and a compute phase (the
//     32 MFMAs of stage s at raised priority), with a block barrier after
//     each.  The second group starts one barrier late, so while one group
//     multiplies the other loads: each SIMD's matrix unit is fed by one wave
//     while its partner waits on memory.
//   * Synchronisation: at the end of its memory phase a wave waits until its
//     fragment reads have landed and only its loads of the two newest stages
//     are pending (vmcnt 8).  The barrier that follows therefore publishes
//     stage s+1 to the group about to read it, and every wave's reads of a
//     ring buffer complete before the barrier after which it is refilled.
//     The ring buffers are separate LDS objects, so the compiler can tell the
//     DMA targets from the reads and inserts no waits of its own.
//   * A sits in LDS as 16-byte k-granules, row-major, the granule order of
//     each row XOR-ed with bits of the row index; an MFMA A fragment is one
//     conflict-free ds_read_b128 (lane l: row l % 16, k-granule l / 16).  W
//     sits N-contiguous (as in memory), the granule order of each k-row
//     XOR-ed with bits 0, 1 and 3 of k, so that the 8 k-rows one B read
//     touches (k and k + 8 of 4 consecutive k) land in distinct banks; an
//     MFMA B fragment (8 consecutive k of one column) is two
//     ds_read_b64_tr_b16, the gfx950 LDS transpose read: in each 16-lane
//     group, lane j's element e comes from element j%4 of the 8 bytes
//     addressed by lane j/4 + 4e.
//   * Loads outside the matrices get an offset no buffer reaches and read as
//     zero, so partial tiles need no branches; stages past the end are loaded
//     the same way, which keeps every wait count constant.
//   * W given as [N, K] (a torch.nn.Linear weight) sits in LDS like A, as
//     k-granules of each column, and a B fragment is one ds_read_b128.  Its
//     W ring holds three 64-deep stages (whole 128-byte lines of every W
//     row; 32-deep stages fetch 64-byte halves) beside a ring of four
//     32-deep A stages, 160 KiB in all; the k order, and so every bit of the
//     result, is the [K, N] kernel's.
#include <type_traits>

#include "device_common.h"
#include "launchers.h"
#include "tile_order.h"

#define CFP32_LDS __attribute__((address_space(3)))

namespace cfp32 {

namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));

constexpr int kT = 512;                             // 8 waves
constexpr int BM = 128, BN = 256, BK = 32, NST = 4;
constexpr int WTM = 64, WTN = 64;                   // wave tile (rows per product x columns)
constexpr int TM = WTM / 16, TN = WTN / 16;         // 16x16 MFMA blocks per wave and product
constexpr int WAVES_N = BN / WTN;                   // 4 waves across N, 2 across M
constexpr int KG = BK / 8;                          // k-granules per A row per stage
constexpr int A_SLOTS = BM * KG;                    // granules per A plane per stage (512)
constexpr int WG = BN / 8;                          // granules per W row (32)
constexpr int W_SLOTS = BK * WG;                    // granules of W per stage (1024)
constexpr int STAGE_SLOTS = 2 * A_SLOTS + W_SLOTS;  // 2048 granules = 32 KiB
constexpr int LOADS_PER_WAVE = 4;                   // 1 per A plane + 2 for W
constexpr int kNoOffset = 0x7FFFFFF0;
constexpr int kBufferWord3 = 0x00020000;

static_assert(A_SLOTS == 64 * (kT / 64) && W_SLOTS == 2 * 64 * (kT / 64), "each wave loads 1 A granule row per plane and 2 of W");
static_assert((BM / WTM) * WAVES_N == kT / 64, "wave tiles cover the block tile");

__shared__ uint4 g_stage0[STAGE_SLOTS];
__shared__ uint4 g_stage1[STAGE_SLOTS];
__shared__ uint4 g_stage2[STAGE_SLOTS];
__shared__ uint4 g_stage3[STAGE_SLOTS];

// SPLIT variant: the hi and lo planes of A for the stage being multiplied,
// converted from the FP32 ring once per stage (two buffers, by stage parity;
// the same layout as the A planes of a ring stage).
__shared__ uint4 g_conv0[2 * A_SLOTS];
__shared__ uint4 g_conv1[2 * A_SLOTS];

// W64 variant ([N, K] W): an A ring of four 32-deep stages (both planes,
// 16 KiB each) and a W ring of three 64-deep stages (256 columns x 8
// k-granules, 32 KiB each: whole 128-byte lines of every W row).
constexpr int W64_KG = 8;
constexpr int W64_SLOTS = BN * W64_KG;
__shared__ uint4 g_a64_0[2 * A_SLOTS];
__shared__ uint4 g_a64_1[2 * A_SLOTS];
__shared__ uint4 g_a64_2[2 * A_SLOTS];
__shared__ uint4 g_a64_3[2 * A_SLOTS];
__shared__ uint4 g_w64_0[W64_SLOTS];
__shared__ uint4 g_w64_1[W64_SLOTS];
__shared__ uint4 g_w64_2[W64_SLOTS];
template <int S>
__device__ __forceinline__ uint4 *a64_buf()
{
    if constexpr (S == 0) return g_a64_0;
    else if constexpr (S == 1) return g_a64_1;
    else if constexpr (S == 2) return g_a64_2;
    else return g_a64_3;
}
template <int T>
__device__ __forceinline__ uint4 *w64_buf()
{
    if constexpr (T == 0) return g_w64_0;
    else if constexpr (T == 1) return g_w64_1;
    else return g_w64_2;
}
// Column n's k-granule g: 16 consecutive columns of one granule fall in 16
// different 16-byte bank groups (columns are 128 bytes apart).
__device__ __forceinline__ int w64_slot(int n, int g) { return n * W64_KG + (g ^ ((n >> 1) & 7)); }

template <int P>
__device__ __forceinline__ uint4 *conv_buf()
{
    if constexpr (P == 0) return g_conv0;
    else return g_conv1;
}

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

// Granule swizzle of W k-row k: bits 0-1 of k select one of four 64-byte
// quarters of a 256-byte bank window, bit 3 one of two 32-byte halves.
__device__ __forceinline__ int w_swz(int k) { return ((k & 3) << 2) ^ (((k >> 3) & 1) << 1); }
__device__ __forceinline__ int w_slot(int k, int ng)
{
    return 2 * A_SLOTS + k * WG + (ng ^ w_swz(k));
}

// WNK variant (W given as [N, K], K-contiguous): W sits in LDS like A, as
// 16-byte k-granules of each of the 256 columns, the granule order XOR-ed with
// bits of the column index; an MFMA B fragment is one ds_read_b128.
__device__ __forceinline__ int w_slot_nk(int n, int kg) { return 2 * A_SLOTS + n * KG + (kg ^ ((n >> 2) & 3)); }

// s_waitcnt immediates (gfx9 encoding): vector-memory count N, LDS count 0 or any.
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (0 << 8); }
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ void block_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

struct DmaArgs {
    const uint16_t *a_hi;
    const uint16_t *a_lo;
    const float *a32;  // SPLIT variant: FP32 A, split in LDS once per stage
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
    const float *bias;  // FP32 [N] added to y after the merge, or null
    int64_t F;          // GEGLU variant: output columns; W, bias are [.., 2F] (gate | up)
    // Split K (plain variants): K is cut into 64-deep units, dealt in order to
    // `kchunks` chunks as evenly as possible (the generic kernel cuts at the
    // same places, so both give the same partial sums); block b computes tile
    // b % tiles over chunk b / tiles and writes its unmerged C_hi, C_lo to
    // part[chunk][row][2][n_pad] (C_hi, then C_lo at + n_pad); a merge
    // dispatch sums the chunks in order.  kchunks == 1: no split, no part.
    int64_t kchunks;
    float *part;
    int64_t n_pad;
};

// FP32 A in LDS (SPLIT variant): each 128-byte row of 32 floats is 8
// granules, granule g stored at position g ^ (row % 8); eight consecutive
// lanes reading one granule column then touch eight different 16-byte bank
// groups.
__device__ __forceinline__ int a32_slot(int row, int g) { return row * 8 + (g ^ (row & 7)); }

// SPLIT = false: A arrives as the FP16 planes A_hi, A_lo.  SPLIT = true: A
// arrives as FP32 (same bytes per stage: 128 x 32 x 4 B).  While a wave's
// MFMAs of stage s run, the wave splits its share of stage s + 1 (the 64 rows
// its group multiplies, 8 values per lane) with the same split as the
// standalone split kernel and writes hi and lo to a conversion buffer laid
// out like the ring's A planes, so both variants multiply identical operands
// and the split costs each value one conversion per block.  Group g's rows
// are loaded and converted by group g's own waves only, so the barriers that
// already separate the two groups' phases order every conversion.
// WNK = true: W is [N, K] (ldw >= K, K % 8 == 0), else [K, N].
//
// GEGLU = true (with [K, N] W, N = 2F): the feed-forward GEGLU of the laya.cpp
// Vulkan guide's graph paragraph fused into the epilogue, out = gelu(gate) *
// up with gate = x W[:, :F] and up = x W[:, F:].  A block computes 128
// output columns: wave column wn owns output columns 32 wn .. 32 wn + 31 and
// multiplies their gate columns in its first 32x32 block and their up
// columns in its second, so one lane holds the gate and up of the same
// output and applies the activation there.  Products, k order and merge are
// those of the plain GEMM.
//
// STACK = true (split K with M <= 64 only): the block's 128 rows hold the hi
// rows of x (rows 0-63, wave row 0) and its lo rows (rows 64-127, wave row
// 1), and each wave runs one product, C = [A_hi; A_lo] W, instead of two
// products over mostly empty rows.  Every accumulator sums the same
// products in the same k order as in the two-product form, so the partial
// sums are the same bits; wave row 0 writes them as C_hi, wave row 1 as C_lo.
template <bool SPLIT, bool WNK, bool GEGLU = false, bool STACK = false, bool W64 = false>
__global__ __launch_bounds__(kT) void gemm_dma_kernel(DmaArgs g)
{
    static_assert(!W64 || (WNK && !SPLIT && !GEGLU && !STACK), "W64: plain [N, K] variant");
    static_assert(!STACK || (!SPLIT && !GEGLU && WTM == 64 && BM == 2 * WTM), "STACK: two wave rows, hi then lo");
    constexpr int LPW = STACK ? LOADS_PER_WAVE - 1 : LOADS_PER_WAVE;  // STACK: one A load per wave
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: barriers branch on it
    const int group = wave >> 2;                                 // waves 0-3 and 4-7; one of each per SIMD
    const int wm = wave / WAVES_N;
    const int wn = wave % WAVES_N;

    const int64_t nbm = (g.M + BM - 1) / BM;
    static_assert(!GEGLU || (TN == 4 && !WNK && !SPLIT), "GEGLU: four 16-column blocks per wave, [K, N] W");
    constexpr int TW = GEGLU ? BN / 2 : BN;  // output columns per block
    const int64_t ncols = GEGLU ? g.F : g.N;
    const int64_t nbn = (ncols + TW - 1) / TW;
    int64_t tile_m, tile_n;
    const int64_t tiles = nbm * nbn;
    const int64_t chunk = (int64_t)blockIdx.x / tiles;  // 0 unless K is split
    tile_of_block((int64_t)blockIdx.x % tiles, nbm, nbn, tile_m, tile_n);
    // This block's K stages and the first k its loads may not reach.
    const int64_t nk_all = (g.Ka + BK - 1) / BK;
    const int64_t units = (g.Ka + 63) / 64;
    const int64_t u_base = units / g.kchunks, u_extra = units % g.kchunks;
    const int64_t u_begin = chunk * u_base + (chunk < u_extra ? chunk : u_extra);
    const int64_t u_end = u_begin + u_base + (chunk < u_extra ? 1 : 0);
    const int64_t s_begin = 2 * u_begin;
    const int64_t nk = (2 * u_end < nk_all ? 2 * u_end : nk_all) - s_begin;
    const int64_t k_end = 64 * u_end;
    const int64_t ka_stop = k_end < g.Ka ? k_end : g.Ka;  // A (zero-padded to Ka)
    const int64_t kw_stop = k_end < g.K ? k_end : g.K;    // W, and A in the SPLIT variant
    const int64_t m0 = tile_m * BM;
    const int64_t n0 = tile_n * TW;

    // SPLIT: both A resources cover the FP32 matrix (rs_lo is unused).
    const __amdgpu_buffer_rsrc_t rs_hi =
        SPLIT ? __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(g.a32), 0, (int)(g.M * g.lda * 4), kBufferWord3)
              : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(g.a_hi), 0, (int)(g.M * g.lda * 2),
                                                  kBufferWord3);
    const __amdgpu_buffer_rsrc_t rs_lo =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(SPLIT ? nullptr : g.a_lo), 0,
                                          (int)(SPLIT ? 0 : g.M * g.lda * 2), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rs_w =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(g.w), 0, (int)((WNK ? g.N : g.K) * g.ldw * 2),
                                          kBufferWord3);

    // This wave's loads of a stage: granules 64*wave + lane of each A plane
    // and 64*(2*wave + jj) + lane of W (lane i fills slot base + i).  Byte
    // offsets of stage 0 are formed once; a stage adds 2*k0 (A) or 2*k0*ldw
    // (W).  Granules outside the operands use kNoOffset.
    // SPLIT: the wave's two A loads are FP32 granules 64*(2*wave + jj) + lane
    // (8 per row: 4 floats each), a_off[jj] / a_kend[jj].
    int a_off[2], a_kend[2], w_off[2], w_kend[2];
    if constexpr (SPLIT) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int slot = 64 * (2 * wave + jj) + lane;
            const int row = slot / 8;
            const int gr = (slot % 8) ^ (row & 7);
            const bool ok = m0 + row < g.M;
            a_off[jj] = ok ? (int)(((m0 + row) * g.lda + 4 * gr) * 4) : kNoOffset;
            a_kend[jj] = ok ? (int)(kw_stop - 4 * gr) : 0;  // K % 4 == 0: a granule is all in or all out
        }
    } else {
        const int slot = 64 * wave + lane;
        const int row = slot / KG;
        const int kg = (slot % KG) ^ ((row >> 2) & 3);
        // STACK (one tile row, m0 = 0): block row r holds x row r % 64 of the
        // hi plane (waves 0-3) or the lo plane (waves 4-7).
        const int64_t xrow = STACK ? (int64_t)(row & 63) : m0 + row;
        const bool ok = xrow < g.M;
        a_off[0] = ok ? (int)((xrow * g.lda + 8 * kg) * 2) : kNoOffset;
        a_kend[0] = ok ? (int)(ka_stop - 8 * kg) : 0;  // stage k0 reads this granule while k0 < a_kend
        a_off[1] = a_off[0];
        a_kend[1] = a_kend[0];
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int slot = 64 * (2 * wave + jj) + lane;
        if constexpr (WNK) {
            const int n = slot / KG;
            const int kg = (slot % KG) ^ ((n >> 2) & 3);
            const bool ok = n0 + n < g.N;
            w_off[jj] = ok ? (int)(((n0 + n) * g.ldw + 8 * kg) * 2) : kNoOffset;
            w_kend[jj] = ok ? (int)(kw_stop - 8 * kg) : 0;  // K % 8 == 0: a granule is all in or all out
        } else {
            const int k = slot / WG;
            const int ng = (slot % WG) ^ w_swz(k);
            int64_t gcol;  // W column of this granule's first of 8 columns
            bool ok;
            if constexpr (GEGLU) {
                const int c = 8 * ng;  // tile column: wave column c / 64, block (c / 32) % 2
                const int64_t out_col = n0 + 32 * (c >> 6) + (c & 31);
                ok = out_col < g.F;
                gcol = out_col + (((c >> 5) & 1) ? g.F : 0);
            } else {
                gcol = n0 + 8 * ng;
                ok = gcol < g.N;
            }
            w_off[jj] = ok ? (int)((k * g.ldw + gcol) * 2) : kNoOffset;
            w_kend[jj] = ok ? (int)(kw_stop - k) : 0;
        }
    }

    // W64: the wave's four 1 KiB loads of a 64-deep W stage: load q covers
    // columns 8 (4 wave + q) .. + 7, lane l column + l / 8 and the granule
    // that belongs at slot l % 8 of that column.
    int w64_off[4], w64_kend[4];
    if constexpr (W64) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = 8 * (4 * wave + q) + (lane >> 3);
            const int gr = (lane & 7) ^ ((c >> 1) & 7);
            const bool ok = n0 + c < g.N;
            w64_off[q] = ok ? (int)(((n0 + c) * g.ldw + 8 * gr) * 2) : kNoOffset;
            w64_kend[q] = ok ? (int)(kw_stop - 8 * gr) : 0;
        }
    }
    auto issue_a64 = [&](auto buf_tag, int64_t k0_64) __attribute__((always_inline)) {
        constexpr int B = decltype(buf_tag)::value;
        uint4 *s = a64_buf<B>();
        const int k0 = (int)k0_64;
        const int a = k0 < a_kend[0] ? a_off[0] + 2 * k0 : kNoOffset;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_hi, (CFP32_LDS void *)(s + 64 * wave), 16, a, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_lo, (CFP32_LDS void *)(s + A_SLOTS + 64 * wave), 16, a, 0, 0, 0);
    };
    auto issue_w64 = [&](auto buf_tag, int64_t k0_64) __attribute__((always_inline)) {
        constexpr int T = decltype(buf_tag)::value;
        uint4 *s = w64_buf<T>();
        const int k0 = (int)k0_64;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int o = k0 < w64_kend[q] ? w64_off[q] + 2 * k0 : kNoOffset;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_w, (CFP32_LDS void *)(s + 64 * (4 * wave + q)), 16, o, 0, 0, 0);
        }
    };

    auto issue = [&](auto stage_tag, int64_t k0_64) {
        constexpr int S = decltype(stage_tag)::value;
        uint4 *s = stage_buf<S>();
        const int k0 = (int)k0_64;
        if constexpr (SPLIT) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int a = k0 < a_kend[jj] ? a_off[jj] + 4 * k0 : kNoOffset;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_hi, (CFP32_LDS void *)(s + 64 * (2 * wave + jj)), 16, a,
                                                         0, 0, 0);
            }
        } else {
            const int a = k0 < a_kend[0] ? a_off[0] + 2 * k0 : kNoOffset;
            if constexpr (STACK) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(group == 0 ? rs_hi : rs_lo, (CFP32_LDS void *)(s + 64 * wave),
                                                         16, a, 0, 0, 0);
            } else {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_hi, (CFP32_LDS void *)(s + 64 * wave), 16, a, 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_lo, (CFP32_LDS void *)(s + A_SLOTS + 64 * wave), 16, a, 0,
                                                         0, 0);
            }
        }
        const int wstep = WNK ? 2 * k0 : (int)(k0_64 * g.ldw * 2);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int o = k0 < w_kend[jj] ? w_off[jj] + wstep : kNoOffset;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_w, (CFP32_LDS void *)(s + 2 * A_SLOTS + 64 * (2 * wave + jj)),
                                                     16, o, 0, 0, 0);
        }
    };

    floatx4_t acc_hi[TM][TN], acc_lo[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc_hi[i][j] = floatx4_t{}, acc_lo[i][j] = floatx4_t{};

    struct Frags {
        half8_t ah[TM], al[TM], bw[TN];
    };
    // Per-lane parts of the fragment addresses (16x16x32 operand layout: lane
    // l holds row / column l % 16 and k = 8 (l / 16) .. 8 (l / 16) + 7).
    const int a_row0 = wm * WTM + (lane & 15);                       // + 16 i
    const int a_kg = lane >> 4;
    const int b_k0 = 8 * (lane >> 4) + ((lane & 15) >> 2);           // + 4 h
    const int b_n0 = wn * WTN + 4 * (lane & 3);                      // + 16 j
    const int b_col0 = wn * WTN + (lane & 15);                       // WNK: + 16 j

    // Fragment reads of a stage.  [K, N] W: the transposed B reads first (the
    // slower kind, about 80 bytes per clock per CU against 240 for
    // ds_read_b128), then A (8192 x 4096 x 14336: 1415 -> 1395 us).
    auto read_a = [&](const uint4 *sa, Frags &f) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = a_row0 + 16 * i;
            f.ah[i] = __builtin_bit_cast(half8_t, sa[a_slot(0, row, a_kg)]);
            if constexpr (!STACK) f.al[i] = __builtin_bit_cast(half8_t, sa[a_slot(1, row, a_kg)]);
        }
    };
    auto read_frags = [&](const uint4 *s, const uint4 *sa, Frags &f) {
        if constexpr (WNK) {
            read_a(sa, f);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                f.bw[j] = __builtin_bit_cast(half8_t, s[w_slot_nk(b_col0 + 16 * j, a_kg)]);
            return;
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = b_n0 + 16 * j;
            short4_t t[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = b_k0 + 4 * h;
                const int byte = w_slot(k, n >> 3) * 16 + (n & 7) * 2;
                t[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CFP32_LDS short4_t *)((CFP32_LDS char *)s + byte));
            }
            const short8_t v = {t[0][0], t[0][1], t[0][2], t[0][3], t[1][0], t[1][1], t[1][2], t[1][3]};
            f.bw[j] = __builtin_bit_cast(half8_t, v);
        }
        __builtin_amdgcn_sched_barrier(0);
        read_a(sa, f);
    };
    // The hi and lo MFMAs of one block back to back, sharing their B
    // fragment (8192 x 4096 x 14336: about 1% faster than all four hi
    // blocks of a row before its lo blocks; same bits, each accumulator's k
    // order is unchanged).
    auto mfmas = [&](const Frags &f) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                acc_hi[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.ah[i], f.bw[j], acc_hi[i][j], 0, 0, 0);
                if constexpr (!STACK)
                    acc_lo[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.al[i], f.bw[j], acc_lo[i][j], 0, 0, 0);
            }
    };

    // SPLIT: lane's conversion unit: row 64*group + u/4, k-granule u%4.
    auto convert = [&](const uint4 *src, uint4 *dst) {
        const int u = 64 * (wave & 3) + lane;
        const int row = 64 * group + (u >> 2);
        const int kg = u & 3;
        const floatx4_t v0 = __builtin_bit_cast(floatx4_t, src[a32_slot(row, 2 * kg)]);
        const floatx4_t v1 = __builtin_bit_cast(floatx4_t, src[a32_slot(row, 2 * kg + 1)]);
        half8_t h, l;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            _Float16 hh, ll;
            split_value(e < 4 ? v0[e] : v1[e - 4], hh, ll);
            h[e] = hh;
            l[e] = ll;
        }
        dst[a_slot(0, row, kg)] = __builtin_bit_cast(uint4, h);
        dst[a_slot(1, row, kg)] = __builtin_bit_cast(uint4, l);
    };

    Frags f0;
    // One stage for this wave: memory phase, barrier, compute phase, barrier.
    auto stage = [&](auto stage_tag, int64_t s) {
        constexpr int S = decltype(stage_tag)::value;
        const uint4 *buf = stage_buf<S>();
        const uint4 *abuf = SPLIT ? conv_buf<S & 1>() : buf;
        // Fragment reads first: the LDS-DMA loads of a group queue behind one
        // another at issue (about 160 cycles for four per wave), and reads
        // issued after them would wait too (8192 x 4096 x 14336: 1470 ->
        // 1420 us).  The two touch different ring buffers.
        read_frags(buf, abuf, f0);
        __builtin_amdgcn_sched_barrier(0);
        issue(std::integral_constant<int, (S + 3) & 3>{}, (s + 3) * BK);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * LPW));
        block_barrier();
        __builtin_amdgcn_s_setprio(1);
        mfmas(f0);
        if constexpr (SPLIT) {
            // Stage s + 1 landed (this group's loads) before the barrier above.
            convert(stage_buf<(S + 1) & 3>(), conv_buf<(S + 1) & 1>());
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * LPW));  // the conversion's LDS writes are done
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        block_barrier();
    };

    if constexpr (W64) {
        // Stage S of a 12-stage round (relative stage index r, r % 12 == S):
        // A from buffer S % 4, W from buffer (S / 2) % 3 at k-granules
        // 4 (S % 2) ..; the memory phase refills A buffer (S + 3) % 4 with
        // stage r + 3 and, at even S, W buffer (S / 2 + 2) % 3 with the W
        // stage that starts at r + 4.  Even stages issue 6 loads, odd ones
        // 2, so at the end of any stage the wait for "all but the newest 8"
        // covers the A stage r + 1 and the W stage it needs.
        auto stage64 = [&](auto stage_tag, int64_t s) __attribute__((always_inline)) {
            constexpr int S = decltype(stage_tag)::value;
            const uint4 *abuf = a64_buf<S & 3>();
            const uint4 *wbuf = w64_buf<(S >> 1) % 3>();
#pragma unroll
            for (int j = 0; j < TN; ++j)
                f0.bw[j] = __builtin_bit_cast(half8_t, wbuf[w64_slot(b_col0 + 16 * j, 4 * (S & 1) + a_kg)]);
            __builtin_amdgcn_sched_barrier(0);
            read_a(abuf, f0);
            __builtin_amdgcn_sched_barrier(0);
            issue_a64(std::integral_constant<int, (S + 3) & 3>{}, (s + 3) * BK);
            if constexpr ((S & 1) == 0) issue_w64(std::integral_constant<int, ((S >> 1) + 2) % 3>{}, (s + 4) * BK);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(8));
            block_barrier();
            __builtin_amdgcn_s_setprio(1);
            mfmas(f0);
            __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
            block_barrier();
        };
        issue_w64(std::integral_constant<int, 0>{}, s_begin * BK);
        issue_a64(std::integral_constant<int, 0>{}, s_begin * BK);
        issue_w64(std::integral_constant<int, 1>{}, (s_begin + 2) * BK);
        issue_a64(std::integral_constant<int, 1>{}, (s_begin + 1) * BK);
        issue_a64(std::integral_constant<int, 2>{}, (s_begin + 2) * BK);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));  // W stage 0 and A stage 0 landed for this wave
        block_barrier();
        if (group == 1) block_barrier();
        const int64_t nkr = nk / 12 * 12;
        for (int64_t s0 = 0; s0 < nkr; s0 += 12) {
            stage64(std::integral_constant<int, 0>{}, s_begin + s0);
            stage64(std::integral_constant<int, 1>{}, s_begin + s0 + 1);
            stage64(std::integral_constant<int, 2>{}, s_begin + s0 + 2);
            stage64(std::integral_constant<int, 3>{}, s_begin + s0 + 3);
            stage64(std::integral_constant<int, 4>{}, s_begin + s0 + 4);
            stage64(std::integral_constant<int, 5>{}, s_begin + s0 + 5);
            stage64(std::integral_constant<int, 6>{}, s_begin + s0 + 6);
            stage64(std::integral_constant<int, 7>{}, s_begin + s0 + 7);
            stage64(std::integral_constant<int, 8>{}, s_begin + s0 + 8);
            stage64(std::integral_constant<int, 9>{}, s_begin + s0 + 9);
            stage64(std::integral_constant<int, 10>{}, s_begin + s0 + 10);
            stage64(std::integral_constant<int, 11>{}, s_begin + s0 + 11);
        }
        if (nkr < nk) stage64(std::integral_constant<int, 0>{}, s_begin + nkr);
        if (nkr + 1 < nk) stage64(std::integral_constant<int, 1>{}, s_begin + nkr + 1);
        if (nkr + 2 < nk) stage64(std::integral_constant<int, 2>{}, s_begin + nkr + 2);
        if (nkr + 3 < nk) stage64(std::integral_constant<int, 3>{}, s_begin + nkr + 3);
        if (nkr + 4 < nk) stage64(std::integral_constant<int, 4>{}, s_begin + nkr + 4);
        if (nkr + 5 < nk) stage64(std::integral_constant<int, 5>{}, s_begin + nkr + 5);
        if (nkr + 6 < nk) stage64(std::integral_constant<int, 6>{}, s_begin + nkr + 6);
        if (nkr + 7 < nk) stage64(std::integral_constant<int, 7>{}, s_begin + nkr + 7);
        if (nkr + 8 < nk) stage64(std::integral_constant<int, 8>{}, s_begin + nkr + 8);
        if (nkr + 9 < nk) stage64(std::integral_constant<int, 9>{}, s_begin + nkr + 9);
        if (nkr + 10 < nk) stage64(std::integral_constant<int, 10>{}, s_begin + nkr + 10);
    } else {
    issue(std::integral_constant<int, 0>{}, s_begin * BK);
    issue(std::integral_constant<int, 1>{}, (s_begin + 1) * BK);
    issue(std::integral_constant<int, 2>{}, (s_begin + 2) * BK);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LPW));  // stage 0 landed for this wave
    block_barrier();
    if constexpr (SPLIT) {
        convert(stage_buf<0>(), conv_buf<0>());
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * LPW));
        block_barrier();
    }
    if (group == 1) block_barrier();  // the second group runs one phase behind
    const int64_t nk4 = nk / NST * NST;
    for (int64_t s0 = 0; s0 < nk4; s0 += NST) {
        stage(std::integral_constant<int, 0>{}, s_begin + s0);
        stage(std::integral_constant<int, 1>{}, s_begin + s0 + 1);
        stage(std::integral_constant<int, 2>{}, s_begin + s0 + 2);
        stage(std::integral_constant<int, 3>{}, s_begin + s0 + 3);
    }
    if (nk4 < nk) stage(std::integral_constant<int, 0>{}, s_begin + nk4);
    if (nk4 + 1 < nk) stage(std::integral_constant<int, 1>{}, s_begin + nk4 + 1);
    if (nk4 + 2 < nk) stage(std::integral_constant<int, 2>{}, s_begin + nk4 + 2);
    }
    if (group == 0) block_barrier();  // both groups pass the same number of barriers
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // drain the trailing zero loads before the block exits

    // Epilogue.  16x16 accumulator layout: lane holds column (lane & 15);
    // element e holds row 4*(lane/16) + e of the block.
    if constexpr (GEGLU) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
        const int64_t col = n0 + 32 * wn + 16 * jj + (lane & 15);
        if (col >= g.F) continue;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = m0 + wm * WTM + i * 16 + 4 * (lane >> 4) + e;
                if (row >= g.M) continue;
                float gate = merge_value(acc_hi[i][jj][e], acc_lo[i][jj][e]);
                float up = merge_value(acc_hi[i][jj + 2][e], acc_lo[i][jj + 2][e]);
                if (g.bias) {
                    gate = gate + g.bias[col];
                    up = up + g.bias[g.F + col];
                }
                __builtin_nontemporal_store(gelu_value(gate) * up, g.y + row * g.ldy + col);
            }
        }
        return;
    }
    if constexpr (STACK) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int64_t col = n0 + wn * WTN + j * 16 + (lane & 15);
                if (col >= g.N) continue;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t xrow = i * 16 + 4 * (lane >> 4) + e;
                    if (xrow >= g.M) continue;
                    // wave row 0: C_hi, wave row 1: C_lo (at + n_pad)
                    __builtin_nontemporal_store(acc_hi[i][j][e],
                                                g.part + ((chunk * g.M + xrow) * 2 + wm) * g.n_pad + col);
                }
            }
        return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t col = n0 + wn * WTN + j * 16 + (lane & 15);
            if (col >= g.N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = m0 + wm * WTM + i * 16 + 4 * (lane >> 4) + e;
                if (row >= g.M) continue;
                const float h = acc_hi[i][j][e], l = acc_lo[i][j][e];
                // Outputs are written once: non-temporal stores keep them from
                // evicting the A and W panels other tiles still read from L2.
                if (g.kchunks > 1) {
                    float *p = g.part + ((chunk * g.M + row) * 2) * g.n_pad + col;
                    __builtin_nontemporal_store(h, p);
                    __builtin_nontemporal_store(l, p + g.n_pad);
                    continue;
                }
                if (g.y) {
                    float v = merge_value(h, l);
                    if (g.bias) v = v + g.bias[col];
                    __builtin_nontemporal_store(v, g.y + row * g.ldy + col);
                }
                if (g.c_hi) {
                    __builtin_nontemporal_store(h, g.c_hi + row * g.ldc + col);
                    __builtin_nontemporal_store(l, g.c_lo + row * g.ldc + col);
                }
            }
        }
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Every byte offset a lane forms into W (including a tile's overhang past K
// or N) stays below kNoOffset.
inline bool w_fits(int64_t ldw, int64_t N, int64_t K, bool w_nk)
{
    constexpr int64_t kLim = kNoOffset - (1 << 20);
    return w_nk ? (N + BN) * ldw * 2 + (int64_t)BK * 8 < kLim : (K + BK) * ldw * 2 + (int64_t)BN * 2 < kLim;
}

}  // namespace

// Runs the LDS-DMA kernel when the operands allow it; returns
// hipErrorNotSupported (and enqueues nothing) otherwise.  a_zero_padded: the
// columns of A from K up to the next multiple of 8 hold +0 and may be read.
hipError_t launch_gemm_dma(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w,
                           int64_t ldw, float *y, int64_t ldy, float *c_hi, float *c_lo, int64_t ldc,
                           int64_t M, int64_t N, int64_t K, bool a_zero_padded, hipStream_t stream,
                           const float *bias, bool w_nk, int64_t kchunks, float *part, int64_t n_pad)
{
    if (kchunks < 1 || (kchunks > 1 && (!part || n_pad < N))) return hipErrorNotSupported;
    if (K <= 0 || lda % 8 || ldw % 8 || !aligned16(a_hi) || !aligned16(a_lo) || !aligned16(w))
        return hipErrorNotSupported;
    if (w_nk && K % 8) return hipErrorNotSupported;
    const int64_t Ka = (K % 8 == 0) ? K : (a_zero_padded ? (K + 7) / 8 * 8 : -1);
    if (Ka < 0 || Ka > lda) return hipErrorNotSupported;
    // Every byte offset a lane forms (including a tile's overhang) stays below kNoOffset.
    constexpr int64_t kLim = kNoOffset - (1 << 20);
    if ((M + BM) * lda * 2 >= kLim || !w_fits(ldw, N, K, w_nk)) return hipErrorNotSupported;
    const int64_t blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN) * kchunks;
    if (blocks > 0x7FFFFFFF) return hipErrorNotSupported;
    DmaArgs g{a_hi, a_lo, nullptr, lda, w, ldw, y, ldy, c_hi, c_lo, ldc, M, N, K, Ka, bias, 0, kchunks, part, n_pad};
    // Split K over at most 64 rows: the hi and lo rows stacked into one tile
    // (8 x 4096 x 14336 .. 64 x 4096 x 14336: half the matrix-unit work).
    const bool stack = kchunks > 1 && 2 * M <= BM;
    // [N, K] W (unless stacked): 64-deep W stages, whole 128-byte lines of
    // every W row per stage (8192 x 4096 x 14336: 1490 -> 1405 us against
    // 32-deep stages, bit-identical; the [K, N] kernel takes 1415 us).
    if (w_nk && stack)
        gemm_dma_kernel<false, true, false, true><<<dim3((unsigned)blocks), kT, 0, stream>>>(g);
    else if (w_nk)
        gemm_dma_kernel<false, true, false, false, true><<<dim3((unsigned)blocks), kT, 0, stream>>>(g);
    else if (stack)
        gemm_dma_kernel<false, false, false, true><<<dim3((unsigned)blocks), kT, 0, stream>>>(g);
    else
        gemm_dma_kernel<false, false><<<dim3((unsigned)blocks), kT, 0, stream>>>(g);
    return hipGetLastError();
}

// The same GEMM reading FP32 A and splitting it while the A fragments are
// formed (no hi/lo planes in memory, one launch for the whole projection).
// Needs 16-byte granules of A that lie wholly inside or wholly outside K
// (K % 4 == 0, lda % 4 == 0, A 16-byte aligned); hipErrorNotSupported
// otherwise, with nothing enqueued.
hipError_t launch_gemm_dma_split(const float *a, int64_t lda, const uint16_t *w, int64_t ldw, float *y,
                                 int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t stream,
                                 const float *bias, bool w_nk)
{
    if (K <= 0 || K % 4 || lda % 4 || ldw % 8 || !aligned16(a) || !aligned16(w)) return hipErrorNotSupported;
    if (w_nk && K % 8) return hipErrorNotSupported;
    constexpr int64_t kLim = kNoOffset - (1 << 20);
    if ((M + BM) * lda * 4 >= kLim || !w_fits(ldw, N, K, w_nk)) return hipErrorNotSupported;
    const int64_t blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    if (blocks > 0x7FFFFFFF) return hipErrorNotSupported;
    DmaArgs g{nullptr, nullptr, a, lda, w, ldw, y, ldy, nullptr, nullptr, ldy, M, N, K, K, bias, 0, 1, nullptr, 0};
    if (w_nk)
        gemm_dma_kernel<true, true><<<dim3((unsigned)blocks), kT, 0, stream>>>(g);
    else
        gemm_dma_kernel<true, false><<<dim3((unsigned)blocks), kT, 0, stream>>>(g);
    return hipGetLastError();
}

// GEGLU-fused GEMM on the split planes: out [M, F] = gelu(x W[:, :F] + b[:F])
// * (x W[:, F:] + b[F:]), W [K, 2F] (ldw >= 2F), bias [2F] or null.  Same
// operand conditions as launch_gemm_dma; hipErrorNotSupported otherwise.
hipError_t launch_gemm_dma_geglu(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w,
                                 int64_t ldw, float *out, int64_t ldo, int64_t M, int64_t F, int64_t K,
                                 bool a_zero_padded, hipStream_t stream, const float *bias)
{
    if (K <= 0 || lda % 8 || ldw % 8 || !aligned16(a_hi) || !aligned16(a_lo) || !aligned16(w))
        return hipErrorNotSupported;
    const int64_t Ka = (K % 8 == 0) ? K : (a_zero_padded ? (K + 7) / 8 * 8 : -1);
    if (Ka < 0 || Ka > lda) return hipErrorNotSupported;
    constexpr int64_t kLim = kNoOffset - (1 << 20);
    if ((M + BM) * lda * 2 >= kLim || !w_fits(ldw, 2 * F, K, false)) return hipErrorNotSupported;
    const int64_t blocks = ((M + BM - 1) / BM) * ((F + BN / 2 - 1) / (BN / 2));
    if (blocks > 0x7FFFFFFF) return hipErrorNotSupported;
    DmaArgs g{a_hi, a_lo, nullptr, lda, w, ldw, out, ldo, nullptr, nullptr, ldo, M, 2 * F, K, Ka, bias, F, 1, nullptr, 0};
    gemm_dma_kernel<false, false, true><<<dim3((unsigned)blocks), kT, 0, stream>>>(g);
    return hipGetLastError();
}

}  // namespace cfp32
