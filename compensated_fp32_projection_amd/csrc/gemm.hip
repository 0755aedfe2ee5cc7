// Dual-product MFMA GEMM with the merge fused into its epilogue.
//
// Computes C_hi = A_hi W and C_lo = A_lo W with FP32 accumulators and
// y = C_hi + C_lo / 1024 (laya.cpp Vulkan guide, compensated-FP32 paragraph:
// both products use FP32 accumulators and are combined in FP32).
//
// gfx950 design
//   * A block of 256 threads (4 waves of 64) owns a BM x BN tile of the
//     output and therefore 2*BM rows of "effective" A (BM hi rows, BM lo
//     rows).  Each wave owns a (BM/WM) x (BN/WN) sub-tile of both products.
//   * The inner operation is v_mfma_f32_32x32x16_f16: a 32x16 FP16 A
//     fragment times a 16x32 FP16 W fragment into 32x32 FP32 accumulators.
//     FP16 x FP16 products are exact in FP32, so the instruction only rounds
//     in its FP32 accumulation.  Every W fragment read from LDS feeds two
//     MFMAs, one for the hi rows and one for the lo rows.
//   * K advances in stages of 64.  A stage of A_hi, A_lo and W is loaded from
//     global memory into registers while the previous stage is multiplied out
//     of LDS, then written to the other half of a double-buffered LDS area:
//     one barrier per stage.  The 32 x 128 tile, which runs the smallest
//     grids, keeps two register sets and so loads two stages ahead, and can
//     take FP32 x and split it in registers (one launch for the projection).
//   * LDS holds 16-byte "k-granules" (8 consecutive k of one row or one
//     column), which is the per-lane operand shape of the MFMA, so every
//     fragment read is one 16-byte LDS read.  W arrives N-contiguous from
//     memory; each thread loads an 8k x 8n block and transposes it in
//     registers into eight k-granules before writing them.  Granule slots
//     are XOR-swizzled (by k-group for A, by the column's 8-group for W) so
//     that both the writes and the fragment reads spread over all LDS banks.
//   * Blocks are renumbered so that the tiles one XCD (one L2) works on are
//     contiguous and grouped GROUP_M tile-rows high, which keeps the A panels
//     and W panels those tiles share resident in that XCD's L2.
//   * Out-of-range rows, columns and k read as zero and are not stored, so
//     any M, N, K >= 1 works.  16-byte global loads are used when the base
//     pointer and leading dimension allow it, element loads otherwise.
#include <type_traits>

#include "device_common.h"
#include "launchers.h"
#include "tile_order.h"

namespace cfp32 {

namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kBK = 64;        // k per stage
constexpr int kKG = kBK / 8;   // k-granules per stage

template <int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
    static constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 MFMA blocks per wave, per product
    static constexpr int A_CHUNKS = BM * kKG / kThreads;  // 16-byte A loads per thread per plane
    static constexpr int W_BLOCKS = kKG * (BN / 8);       // 8x8 W blocks per stage
    static constexpr int W_ITERS = (W_BLOCKS + kThreads - 1) / kThreads;
    static constexpr int LDS_A = 2 * kKG * BM;  // granules (16 B) of A per stage, both planes
    static constexpr int LDS_W = kKG * BN;      // granules of W per stage
    static constexpr int LDS_STAGE = LDS_A + LDS_W;
    static_assert(WM * WN == kThreads / 64, "four waves per block");
    static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile is whole MFMA blocks");
    static_assert((BM * kKG) % kThreads == 0, "A stage splits evenly over the threads");
    static_assert(W_BLOCKS % 64 == 0, "W loaders are whole waves");
    static constexpr int W_NK_CHUNKS = kKG * BN / kThreads;  // [N, K] W: 16-byte loads per thread per stage
    static_assert(W_NK_CHUNKS <= 8 * W_ITERS && (kKG * BN) % kThreads == 0, "[N, K] granules fit the W registers");
    static_assert(2 * LDS_STAGE * 16 <= 160 * 1024, "double-buffered stage fits in LDS");
};

using TileLarge = TileCfg<128, 256, 2, 2>;   // wave: 64 M-rows (128 hi+lo rows) x 128 cols
using TileMedium = TileCfg<64, 128, 2, 2>;   // wave: 32 x 64
using TileSmall = TileCfg<32, 128, 1, 4>;    // wave: 32 x 32

struct GemmArgs {
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
    const float *bias;  // FP32 [N] added to y after the merge, or null
    int geglu_rmw;      // y holds a GEGLU gate on entry: y = gelu(y) * (merged value + bias)
    // Split K: K is cut into 64-deep units (one stage each), dealt in order to
    // `kchunks` chunks as evenly as possible, the cuts the LDS-DMA kernel
    // makes; block b computes tile b % tiles over chunk b / tiles and writes
    // its unmerged C_hi, C_lo to part[chunk][row][2][n_pad].  kchunks == 1:
    // no split (the only case with SEP > 0 or geglu_rmw).
    int64_t kchunks;
    float *part;
    int64_t n_pad;
};

// Slot of A granule (k-group kg, tile row `row`) of plane p inside a stage.
template <class T>
__device__ __forceinline__ int a_slot(int p, int kg, int row)
{
    return p * (kKG * T::BM) + kg * T::BM + (row ^ kg);
}

// Slot of W granule (k-group kg, tile column n) inside a stage.
template <class T>
__device__ __forceinline__ int w_slot(int kg, int n)
{
    return T::LDS_A + kg * T::BN + (n ^ ((n >> 3) & 7));
}

// The same for W given as [N, K]: the 8 granules of a column are stored
// together (the 8 lanes that load a column's 128 bytes write one 128-byte
// LDS row; in the layout above they all hit the same banks), their order
// XOR-ed with bits 1-3 of n, so that the 16 consecutive columns a B
// fragment read takes at one k-group fall in 16 different bank groups.
template <class T>
__device__ __forceinline__ int w_slot_nk(int kg, int n)
{
    return T::LDS_A + n * kKG + (kg ^ ((n >> 1) & 7));
}

// [K, N] W in the 128-column tiles: the stage's 64 rows as loaded (row k,
// granule ng of 8 columns), the granule order XOR-ed with 4 (k % 4).  A
// store instruction writes whole 256-byte rows; a transposed B read (rows
// k .. k + 3 and k + 8 .. k + 11 at four granules) meets every bank group
// twice, the least for its 512 bytes.
template <class T>
__device__ __forceinline__ int w_slot_kn(int k, int ng)
{
    return T::LDS_A + k * (T::BN / 8) + (ng ^ (4 * (k & 3)));
}

// Offset that no buffer reaches: a raw buffer load at it returns zero and
// touches no memory, whether or not the scalar offset enters the range check.
constexpr int kNoOffset = 0x7FFFFFF0;
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit buffer, gfx9 family

// BUF: every operand is 16-byte aligned and smaller than 2^31 bytes, so full
// K stages are fetched with raw buffer loads (no per-load branches; rows past
// M and columns past N read as zero).  The ragged last stage, and every stage
// of the generic variant, use guarded loads.
//
// SEP > 0 selects the separate-addition accumulation of the laya.cpp Vulkan
// guide's AMD path (compensated-FP32 paragraph: tile results added with
// separate FP32 additions, against drift in long multiply-add chains): the
// matrix unit accumulates SEP consecutive 16-deep k-steps (SEP = 1: each
// MFMA starts from zero), and each such partial result is added to a running
// FP32 sum with an ordinary vector addition.  SEP is 1, 4 (one stage) or a
// multiple of 4.
//
// WNK: W is given as [N, K] (ldw >= K); its 16-byte k-granules are loaded and
// stored exactly like those of A, no transpose needed.
//
// XF: A is the FP32 input x itself (a_hi holds x, lda its row stride in
// elements; a_lo unused), and the split happens in registers (split_value,
// the conversion of the split dispatch): the eight values of a k-group
// arrive as two 16-byte loads into the two staging slots that otherwise hold
// the hi and lo granules, and are written to LDS as those granules.  The
// planes are the split dispatch's, so every bit of the result is that of
// split + GEMM.  Only the 32 x 128 tile with 16-byte loads takes it.
template <class T, bool AL_A, bool AL_W, bool BUF, int SEP = 0, bool WNK = false, bool XF = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(T::BM <= 32 && SEP == 0 ? 2 : 1))) void gemm_kernel(GemmArgs g)
{
    static_assert(SEP == 0 || SEP == 1 || SEP % 4 == 0, "separate additions per MFMA or per whole stages");
    __shared__ uint4 lds[2 * T::LDS_STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / T::WN;
    const int wn = wave % T::WN;

    // --- tile scheduling: XCD-contiguous renumbering, then grouped order ---
    const int64_t nbm = (g.M + T::BM - 1) / T::BM;
    const int64_t nbn = (g.N + T::BN - 1) / T::BN;
    const int64_t total = nbm * nbn;
    const int64_t chunk = (int64_t)blockIdx.x / total;  // 0 unless K is split
    int64_t tile_m, tile_n;
    tile_of_block((int64_t)blockIdx.x % total, nbm, nbn, tile_m, tile_n);
    const int64_t m0 = tile_m * T::BM;
    const int64_t n0 = tile_n * T::BN;

    // This block's 64-deep K stages [u_begin, u_end) and the first k its loads
    // may not reach.
    const int64_t units = (g.K + kBK - 1) / kBK;
    const int64_t u_base = units / g.kchunks, u_extra = units % g.kchunks;
    const int64_t u_begin = chunk * u_base + (chunk < u_extra ? chunk : u_extra);
    const int64_t u_end = u_begin + u_base + (chunk < u_extra ? 1 : 0);
    const int64_t k_begin = kBK * u_begin;
    const int64_t klim = kBK * u_end < g.K ? kBK * u_end : g.K;

    floatx16_t acc_hi[T::TM][T::TN];
    floatx16_t acc_lo[T::TM][T::TN];
    floatx16_t sum_hi[T::TM][T::TN];  // SEP > 0: the running FP32 sums
    floatx16_t sum_lo[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            acc_hi[i][j] = floatx16_t{};
            acc_lo[i][j] = floatx16_t{};
            sum_hi[i][j] = floatx16_t{};
            sum_lo[i][j] = floatx16_t{};
        }
    // Add the matrix unit's partial sums to the running sums and restart them
    // from zero (after every k-step for SEP == 1, every SEP k-steps above).
    auto flush = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    sum_hi[i][j][e] += acc_hi[i][j][e];
                    sum_lo[i][j][e] += acc_lo[i][j][e];
                }
                acc_hi[i][j] = floatx16_t{};
                acc_lo[i][j] = floatx16_t{};
            }
    };

    // [K, N] W in 128-column tiles: stored as loaded, B fragments by the
    // gfx950 transposed LDS read (no register transpose).
    constexpr bool kTR = !WNK && T::BN == 128;
    // Staging registers.  The 32 x 128 tile (plain accumulation, 16-byte
    // loads) keeps two sets, so that a stage's loads land in one set while
    // the previous stage's set is written to LDS; the others use set 0 only.
    constexpr bool kTwoSets = BUF && T::BM <= 32 && SEP == 0;
    static_assert(!XF || kTwoSets, "the FP32-input form is the 32 x 128 tile's");
    const float *xf = reinterpret_cast<const float *>(g.a_hi);  // XF: x
    uint4 ra_set[2][2][T::A_CHUNKS];
    uint4 rw_set[2][T::W_ITERS][8];

    // Buffer-load state (used only when BUF): wave-uniform descriptors and
    // per-thread byte offsets that do not change from stage to stage; the
    // stage's k offset travels in the scalar offset.
    constexpr int kAElem = XF ? 4 : 2;  // bytes per A element in memory
    const __amdgpu_buffer_rsrc_t rs_hi = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(g.a_hi), 0, (int)(g.M * g.lda * kAElem), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rs_lo = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(XF ? g.a_hi : g.a_lo), 0, (int)(g.M * g.lda * kAElem), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rs_w =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(g.w), 0, (int)((WNK ? g.N : g.K) * g.ldw * 2),
                                          kBufferWord3);
    int voff_a[T::A_CHUNKS];
    int voff_w[T::W_ITERS];
    int voff_wn[T::W_NK_CHUNKS];  // WNK: like voff_a, granule q of column (c >> 3)
    if constexpr (BUF && WNK) {
#pragma unroll
        for (int q = 0; q < T::W_NK_CHUNKS; ++q) {
            const int c = tid + kThreads * q;
            const int64_t gn = n0 + (c >> 3);
            voff_wn[q] = gn < g.N ? (int)((gn * g.ldw + 8 * (c & 7)) * 2) : kNoOffset;
        }
    }
    // kTR: granule q of every thread is stage row c / (BN / 8), 8 columns
    // at (c % (BN / 8)) * 8, c = tid + kThreads q (whole 256-byte rows per
    // 16 lanes); the stage adds its k0 rows as a scalar offset.
    if constexpr (BUF && kTR) {
#pragma unroll
        for (int q = 0; q < T::W_NK_CHUNKS; ++q) {
            const int c = tid + kThreads * q;
            const int64_t gn = n0 + 8 * (c % (T::BN / 8));
            voff_wn[q] = gn < g.N ? (int)(((int64_t)(c / (T::BN / 8)) * g.ldw + gn) * 2) : kNoOffset;
        }
    }
    if constexpr (BUF) {
#pragma unroll
        for (int i = 0; i < T::A_CHUNKS; ++i) {
            const int c = tid + kThreads * i;
            const int64_t gm = m0 + (c >> 3);
            voff_a[i] = gm < g.M ? (int)((gm * g.lda + 8 * (c & 7)) * kAElem) : kNoOffset;
        }
#pragma unroll
        for (int j = 0; j < T::W_ITERS; ++j) {
            const int b = tid + kThreads * j;
            const int kgw = b / (T::BN / 8), nc = b % (T::BN / 8);
            const int64_t gn = n0 + 8 * nc;
            voff_w[j] = gn < g.N && b < T::W_BLOCKS ? (int)((8 * kgw * g.ldw + gn) * 2) : kNoOffset;
        }
    }

    // The scalar offsets are wave-uniform; readfirstlane states so, which
    // keeps the compiler from wrapping each load in a loop over the distinct
    // values of an offset it could not prove uniform.
    auto load_stage_buf = [&](auto set_tag, int64_t k0) {
        auto &ra = ra_set[decltype(set_tag)::value];
        auto &rw = rw_set[decltype(set_tag)::value];
        const int so_k = __builtin_amdgcn_readfirstlane((int)(k0 * 2));
#pragma unroll
        for (int i = 0; i < T::A_CHUNKS; ++i) {
            if constexpr (XF) {  // x[k .. k + 3] and x[k + 4 .. k + 7]
                const int so_x = __builtin_amdgcn_readfirstlane((int)(k0 * 4));
                ra[0][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_hi, voff_a[i], so_x, 0));
                ra[1][i] =
                    __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_hi, voff_a[i] + 16, so_x, 0));
                continue;
            }
            ra[0][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_hi, voff_a[i], so_k, 0));
            ra[1][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_lo, voff_a[i], so_k, 0));
        }
        if constexpr (WNK) {
#pragma unroll
            for (int q = 0; q < T::W_NK_CHUNKS; ++q)
                rw[q >> 3][q & 7] =
                    __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_w, voff_wn[q], so_k, 0));
            return;
        }
        if constexpr (kTR) {
            const int so_r = __builtin_amdgcn_readfirstlane((int)(k0 * g.ldw * 2));
#pragma unroll
            for (int q = 0; q < T::W_NK_CHUNKS; ++q)
                rw[q >> 3][q & 7] =
                    __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_w, voff_wn[q], so_r, 0));
            return;
        }
#pragma unroll
        for (int j = 0; j < T::W_ITERS; ++j) {
            // With two register sets, threads past the stage's W blocks load
            // too (offsets no buffer reaches, values never stored), so every
            // wave issues the same loads and the compiler's wait counts
            // between the sets stay exact; otherwise they skip the loads.
            if (!kTwoSets && tid + kThreads * j >= T::W_BLOCKS) continue;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int so_w = __builtin_amdgcn_readfirstlane((int)((k0 + r) * g.ldw * 2));
                rw[j][r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_w, voff_w[j], so_w, 0));
            }
        }
    };

    auto load_stage = [&](auto set_tag, int64_t k0) {
        auto &ra = ra_set[decltype(set_tag)::value];
        auto &rw = rw_set[decltype(set_tag)::value];
#pragma unroll
        for (int i = 0; i < T::A_CHUNKS; ++i) {
            const int c = tid + kThreads * i;
            const int kg = c & 7, row = c >> 3;
            const int64_t gm = m0 + row, gk = k0 + 8 * kg;
            if constexpr (XF) {  // ragged stage: values past klim (or rows past M) read as +0
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = gm < g.M && gk + e < klim ? xf[gm * g.lda + gk + e] : 0.0f;
                ra[0][i] = make_uint4(__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                                      __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3]));
                ra[1][i] = make_uint4(__builtin_bit_cast(uint32_t, v[4]), __builtin_bit_cast(uint32_t, v[5]),
                                      __builtin_bit_cast(uint32_t, v[6]), __builtin_bit_cast(uint32_t, v[7]));
                continue;
            }
            if (gm < g.M) {
                ra[0][i] = load_row8<AL_A>(g.a_hi + gm * g.lda, gk, klim);
                ra[1][i] = load_row8<AL_A>(g.a_lo + gm * g.lda, gk, klim);
            } else {
                ra[0][i] = make_uint4(0, 0, 0, 0);
                ra[1][i] = make_uint4(0, 0, 0, 0);
            }
        }
        if constexpr (WNK) {
#pragma unroll
            for (int q = 0; q < T::W_NK_CHUNKS; ++q) {
                const int c = tid + kThreads * q;
                const int64_t gn = n0 + (c >> 3), gk = k0 + 8 * (c & 7);
                rw[q >> 3][q & 7] = gn < g.N ? load_row8<AL_W>(g.w + gn * g.ldw, gk, klim) : make_uint4(0, 0, 0, 0);
            }
            return;
        }
        if constexpr (kTR) {
#pragma unroll
            for (int q = 0; q < T::W_NK_CHUNKS; ++q) {
                const int c = tid + kThreads * q;
                const int64_t gk = k0 + c / (T::BN / 8), gn = n0 + 8 * (c % (T::BN / 8));
                rw[q >> 3][q & 7] = gk < klim ? load_row8<AL_W>(g.w + gk * g.ldw, gn, g.N) : make_uint4(0, 0, 0, 0);
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < T::W_ITERS; ++j) {
            const int b = tid + kThreads * j;
            if (b < T::W_BLOCKS) {
                const int kgw = b / (T::BN / 8), nc = b % (T::BN / 8);
                const int64_t gn = n0 + 8 * nc;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int64_t gk = k0 + 8 * kgw + r;
                    rw[j][r] = gk < klim ? load_row8<AL_W>(g.w + gk * g.ldw, gn, g.N) : make_uint4(0, 0, 0, 0);
                }
            }
        }
    };

    auto store_stage = [&](auto set_tag, int st) {
        auto &ra = ra_set[decltype(set_tag)::value];
        auto &rw = rw_set[decltype(set_tag)::value];
        uint4 *s = lds + st * T::LDS_STAGE;
#pragma unroll
        for (int i = 0; i < T::A_CHUNKS; ++i) {
            const int c = tid + kThreads * i;
            const int kg = c & 7, row = c >> 3;
            if constexpr (XF) {  // eight FP32 values -> the hi and lo granules
                const floatx4_t x0 = __builtin_bit_cast(floatx4_t, ra[0][i]);
                const floatx4_t x1 = __builtin_bit_cast(floatx4_t, ra[1][i]);
                half8_t h, l;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    _Float16 hh, ll;
                    split_value(e < 4 ? x0[e] : x1[e - 4], hh, ll);
                    h[e] = hh;
                    l[e] = ll;
                }
                s[a_slot<T>(0, kg, row)] = __builtin_bit_cast(uint4, h);
                s[a_slot<T>(1, kg, row)] = __builtin_bit_cast(uint4, l);
                continue;
            }
            s[a_slot<T>(0, kg, row)] = ra[0][i];
            s[a_slot<T>(1, kg, row)] = ra[1][i];
        }
        if constexpr (WNK) {
#pragma unroll
            for (int q = 0; q < T::W_NK_CHUNKS; ++q) {
                const int c = tid + kThreads * q;
                s[w_slot_nk<T>(c & 7, c >> 3)] = rw[q >> 3][q & 7];
            }
            return;
        }
        if constexpr (kTR) {
#pragma unroll
            for (int q = 0; q < T::W_NK_CHUNKS; ++q) {
                const int c = tid + kThreads * q;
                s[w_slot_kn<T>(c / (T::BN / 8), c % (T::BN / 8))] = rw[q >> 3][q & 7];
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < T::W_ITERS; ++j) {
            const int b = tid + kThreads * j;
            if (b < T::W_BLOCKS) {
                const int kgw = b / (T::BN / 8), nc = b % (T::BN / 8);
                // rw[j][r] holds W[k = 8*kgw + r][n = 8*nc .. 8*nc + 7]; gather
                // column e into one granule of eight k values.  Each dword of
                // the granule is one byte permute: the e-th halves of rows 2p
                // (low half) and 2p + 1 (high half).
                const uint32_t *v = reinterpret_cast<const uint32_t *>(rw[j]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int q = e >> 1;
                    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                    uint32_t d[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        d[p] = __builtin_amdgcn_perm(v[(2 * p + 1) * 4 + q], v[(2 * p) * 4 + q], sel);
                    s[w_slot<T>(kgw, 8 * nc + e)] = make_uint4(d[0], d[1], d[2], d[3]);
                }
            }
        }
    };

    // Fragments of one 16-deep k-step: A hi/lo rows and W columns.
    struct Frags {
        half8_t ah[T::TM], al[T::TM], bw[T::TN];
    };
    auto read_frags = [&](const uint4 *s, int ks, Frags &f) __attribute__((always_inline)) {
        const int kg = 2 * ks + (lane >> 5);
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            const int row = wm * T::WTM + i * 32 + (lane & 31);
            f.ah[i] = __builtin_bit_cast(half8_t, s[a_slot<T>(0, kg, row)]);
            f.al[i] = __builtin_bit_cast(half8_t, s[a_slot<T>(1, kg, row)]);
        }
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            if constexpr (kTR) {
                // Lanes in groups of 16: group G takes columns 16 (G % 2) ..
                // + 15 at k = 16 ks + 8 (G / 2) .. + 7; lane i of a group
                // addresses row (i / 4) + 4 h at columns 4 (i % 4) .. + 3, and
                // the transposed read hands it column i at those four rows.
                const int grp = lane >> 4, li = lane & 15;
                const int c = wn * T::WTN + j * 32 + 16 * (grp & 1) + 4 * (li & 3);
                short4_t t[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int k = 16 * ks + 8 * (grp >> 1) + (li >> 2) + 4 * h;
                    const int byte = w_slot_kn<T>(k, c >> 3) * 16 + (c & 7) * 2;
                    t[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) short4_t *)((__attribute__((address_space(3))) char *)s + byte));
                }
                const short8_t v = {t[0][0], t[0][1], t[0][2], t[0][3], t[1][0], t[1][1], t[1][2], t[1][3]};
                f.bw[j] = __builtin_bit_cast(half8_t, v);
                continue;
            }
            const int n = wn * T::WTN + j * 32 + (lane & 31);
            f.bw[j] = __builtin_bit_cast(half8_t, s[WNK ? w_slot_nk<T>(kg, n) : w_slot<T>(kg, n)]);
        }
    };
    auto mfmas = [&](const Frags &f) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                acc_hi[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.ah[i], f.bw[j], acc_hi[i][j], 0, 0, 0);
                acc_lo[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.al[i], f.bw[j], acc_lo[i][j], 0, 0, 0);
            }
        // SEP == 1: every MFMA started from zero; add its result now.
        if constexpr (SEP == 1) flush();
    };
    // The fragments of k-step ks+1 are read while the MFMAs of ks run.
    // Stage kt covers k-steps 4 kt .. 4 kt + 3; with SEP >= 4 the running sums
    // take the partial sums after every SEP k-steps.
    auto compute_stage = [&](int st, int64_t kt) __attribute__((always_inline)) {
        const uint4 *s = lds + st * T::LDS_STAGE;
        Frags f[2];
        read_frags(s, 0, f[0]);
#pragma unroll
        for (int ks = 0; ks < kKG / 2; ++ks) {
            if (ks + 1 < kKG / 2) read_frags(s, ks + 1, f[(ks + 1) & 1]);
            mfmas(f[ks & 1]);
        }
        if constexpr (SEP >= 4) {
            if (((kt + 1) * (kKG / 2)) % SEP == 0) flush();
        }
    };

    // K loop.  Stage kt is multiplied out of LDS buffer kt & 1; its
    // successors travel in the two register sets.  Full stages use the
    // buffer loads, so the main loops have no branch; the ragged last stage
    // (if K is not a multiple of 64) uses guarded loads.  (Chunk boundaries
    // are multiples of 64, so only the chunk that ends at K can have a
    // ragged last stage.)
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    const int64_t nk = u_end - u_begin;
    const int64_t nk_full = BUF ? (klim - k_begin) / kBK : 0;
    if (nk == 0) {
        // K == 0: nothing to accumulate; the epilogue writes +0.
    } else if (kTwoSets && nk_full >= 4) {
        // Two stages ahead: while stage kt is multiplied, stage kt + 1 waits
        // in one register set to be written to LDS and stage kt + 2 loads
        // into the other, so two memory round trips overlap each stage's
        // MFMAs.  Invariant at the top of a pair (kt even): LDS buffer 0
        // holds stage kt, set 1 holds (or is loading) stage kt + 1.
        load_stage_buf(S0{}, k_begin);
        load_stage_buf(S1{}, k_begin + kBK);
        store_stage(S0{}, 0);
        __syncthreads();
        int64_t kt = 0;
        for (; kt + 3 < nk_full; kt += 2) {
            load_stage_buf(S0{}, k_begin + (kt + 2) * kBK);
            compute_stage(0, kt);
            store_stage(S1{}, 1);
            __syncthreads();
            load_stage_buf(S1{}, k_begin + (kt + 3) * kBK);
            compute_stage(1, kt + 1);
            store_stage(S0{}, 0);
            __syncthreads();
        }
        // 2 to 4 stages remain (kt + 1 < nk_full, kt + 3 >= nk_full >= nk - 1):
        // the same steps with guarded loads, which also cover a ragged last
        // stage.
        for (; kt + 1 < nk; ++kt) {
            const bool more = kt + 2 < nk;
            if ((kt & 1) == 0) {
                if (more) load_stage(S0{}, k_begin + (kt + 2) * kBK);
                compute_stage(0, kt);
                store_stage(S1{}, 1);
            } else {
                if (more) load_stage(S1{}, k_begin + (kt + 2) * kBK);
                compute_stage(1, kt);
                store_stage(S0{}, 0);
            }
            __syncthreads();
        }
        compute_stage((int)(kt & 1), kt);
    } else {
        // Short or unaligned K: one stage ahead.
        if (nk_full > 0)
            load_stage_buf(S0{}, k_begin);
        else
            load_stage(S0{}, k_begin);
        store_stage(S0{}, 0);
        __syncthreads();
        int64_t kt = 0;
        for (; kt + 1 < nk_full; ++kt) {
            load_stage_buf(S0{}, k_begin + (kt + 1) * kBK);
            compute_stage((int)(kt & 1), kt);
            store_stage(S0{}, (int)((kt + 1) & 1));
            __syncthreads();
        }
        for (; kt + 1 < nk; ++kt) {
            load_stage(S0{}, k_begin + (kt + 1) * kBK);
            compute_stage((int)(kt & 1), kt);
            store_stage(S0{}, (int)((kt + 1) & 1));
            __syncthreads();
        }
        compute_stage((int)(kt & 1), kt);
    }
    if constexpr (SEP >= 4) flush();  // the last, possibly short, group of k-steps

    // --- epilogue: 32x32 accumulator layout of v_mfma_f32_32x32x16_f16:
    // lane holds column (lane & 31); element e holds row
    // 8*(e/4) + 4*(lane/32) + (e%4) of the 32x32 block.
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const int64_t col = n0 + wn * T::WTN + j * 32 + (lane & 31);
            if (col >= g.N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + wm * T::WTM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (row >= g.M) continue;
                const float h = SEP ? sum_hi[i][j][e] : acc_hi[i][j][e];
                const float l = SEP ? sum_lo[i][j][e] : acc_lo[i][j][e];
                if (g.kchunks > 1) {
                    float *p = g.part + ((chunk * g.M + row) * 2) * g.n_pad + col;
                    p[0] = h;
                    p[g.n_pad] = l;
                    continue;
                }
                if (g.y) {
                    float v = merge_value(h, l);
                    if (g.bias) v = v + g.bias[col];
                    if (g.geglu_rmw) v = gelu_value(g.y[row * g.ldy + col]) * v;
                    g.y[row * g.ldy + col] = v;
                }
                if (g.c_hi) {
                    g.c_hi[row * g.ldc + col] = h;
                    g.c_lo[row * g.ldc + col] = l;
                }
            }
        }
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <class T, int SEP = 0, bool WNK = false>
hipError_t launch_tile(const GemmArgs &g, hipStream_t stream)
{
    const int64_t blocks = ((g.M + T::BM - 1) / T::BM) * ((g.N + T::BN - 1) / T::BN) * g.kchunks;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const bool al_a = (g.lda % 8 == 0) && aligned16(g.a_hi) && aligned16(g.a_lo);
    const bool al_w = (g.ldw % 8 == 0) && aligned16(g.w);
    // Buffer offsets are 32-bit: every byte offset a thread forms, including a
    // tile's overhang past M and N, must stay below kNoOffset.
    constexpr int64_t kLim = kNoOffset - (1 << 20);
    const bool fits = (g.M + T::BM) * g.lda * 2 < kLim &&
                      (WNK ? (g.N + T::BN) * g.ldw * 2 + (int64_t)kBK * 2 < kLim
                           : (g.K + kBK) * g.ldw * 2 + (int64_t)T::BN * 2 < kLim);
    const dim3 grid((unsigned)blocks);
    if (al_a && al_w && fits)
        gemm_kernel<T, true, true, true, SEP, WNK><<<grid, kThreads, 0, stream>>>(g);
    else if (al_a && al_w)
        gemm_kernel<T, true, true, false, SEP, WNK><<<grid, kThreads, 0, stream>>>(g);
    else if (al_a)
        gemm_kernel<T, true, false, false, SEP, WNK><<<grid, kThreads, 0, stream>>>(g);
    else if (al_w)
        gemm_kernel<T, false, true, false, SEP, WNK><<<grid, kThreads, 0, stream>>>(g);
    else
        gemm_kernel<T, false, false, false, SEP, WNK><<<grid, kThreads, 0, stream>>>(g);
    return hipGetLastError();
}

template <class T>
int64_t tiles_of(int64_t M, int64_t N)
{
    return ((M + T::BM - 1) / T::BM) * ((N + T::BN - 1) / T::BN);
}

constexpr int64_t kCus = 256;

// Below the LDS-DMA kernel's grids, the 64 x 128 tile only where the
// 32 x 128 tile would deal more than three tiles to each CU (2048 x 4096 x
// 1792, 896 small tiles: 107 against 123 us); with its two register sets,
// loads two stages ahead and the split in registers, the 32 x 128 tile won
// up to there (1024 x 4096 x 2048: 85 -> 60 us, 2048 x 8192 x 1024: 168 ->
// 110 us, 4096 x 2048 x 512: 60 -> 34 us, 3000 x 3000 x 1000 [N, K]: 85 ->
// 77 us).
bool medium_tile(int64_t M, int64_t N)
{
    return tiles_of<TileMedium>(M, N) >= kCus && tiles_of<TileSmall>(M, N) > 3 * kCus;
}

// The generic kernel's tile for an M x N output when the LDS-DMA kernel does
// not run: 0 = 128 x 256, 1 = 64 x 128, 2 = 32 x 128 (see launch_gemm).
int generic_tile(int64_t M, int64_t N)
{
    if (tiles_of<TileLarge>(M, N) >= kCus / 2) return 0;
    return medium_tile(M, N) ? 1 : 2;
}

}  // namespace

// Tile choice: the LDS-DMA kernel (128 x 256 tiles) from half a block per
// CU (128 tiles) up, below that the generic kernel's 32 x 128 tile, or its
// 64 x 128 tile on the largest of those grids (medium_tile).  Even with CUs left
// idle the LDS-DMA kernel wins there: 512 x 4096 x 14336 (224 tiles) 123
// against 174 us for the whole projection with the generic 64 x 128 tile;
// 300 x 4096 x 14336 (168 tiles) 102 against 158 us, 1024 x 4096 x 4096
// (128 tiles) 95 against 112 us ([N, K] weights: 96 against 140 us); the
// same bits.
hipError_t launch_gemm(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w,
                       int64_t ldw, float *y, int64_t ldy, float *c_hi, float *c_lo, int64_t ldc,
                       int64_t M, int64_t N, int64_t K, bool a_zero_padded, hipStream_t stream,
                       const float *bias, bool w_nk, bool geglu_rmw)
{
    GemmArgs g{a_hi, a_lo, lda, w, ldw, y, ldy, c_hi, c_lo, ldc, M, N, K, bias, geglu_rmw ? 1 : 0, 1, nullptr, 0};
    if (tiles_of<TileLarge>(M, N) >= kCus / 2 && !geglu_rmw) {
        const hipError_t e = launch_gemm_dma(a_hi, a_lo, lda, w, ldw, y, ldy, c_hi, c_lo, ldc, M, N, K,
                                             a_zero_padded, stream, bias, w_nk);
        if (e != hipErrorNotSupported) return e;
        return w_nk ? launch_tile<TileLarge, 0, true>(g, stream) : launch_tile<TileLarge>(g, stream);
    }
    if (medium_tile(M, N))
        return w_nk ? launch_tile<TileMedium, 0, true>(g, stream) : launch_tile<TileMedium>(g, stream);
    return w_nk ? launch_tile<TileSmall, 0, true>(g, stream) : launch_tile<TileSmall>(g, stream);
}

// The projection in one launch on the grids that take the 32 x 128 tile:
// x split in registers as its stages are loaded (the split dispatch and the
// planes drop out; the bits are those of split + launch_gemm).
hipError_t launch_gemm_xsplit(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy,
                              int64_t M, int64_t N, int64_t K, hipStream_t stream, const float *bias, bool w_nk)
{
    if (M <= 0 || N <= 0 || K <= 0 || generic_tile(M, N) != 2) return hipErrorNotSupported;
    if (ldx % 4 || !aligned16(x) || ldw % 8 || !aligned16(w)) return hipErrorNotSupported;
    constexpr int64_t kLim = kNoOffset - (1 << 20);
    const bool fits = (M + TileSmall::BM) * ldx * 4 < kLim &&
                      (w_nk ? (N + TileSmall::BN) * ldw * 2 + (int64_t)kBK * 2 < kLim
                            : (K + kBK) * ldw * 2 + (int64_t)TileSmall::BN * 2 < kLim);
    if (!fits) return hipErrorNotSupported;
    GemmArgs g{reinterpret_cast<const uint16_t *>(x), nullptr, ldx, w, ldw, y, ldy, nullptr, nullptr, 0, M, N, K,
               bias, 0, 1, nullptr, 0};
    const dim3 grid((unsigned)tiles_of<TileSmall>(M, N));
    if (w_nk)
        gemm_kernel<TileSmall, true, true, true, 0, true, true><<<grid, kThreads, 0, stream>>>(g);
    else
        gemm_kernel<TileSmall, true, true, true, 0, false, true><<<grid, kThreads, 0, stream>>>(g);
    return hipGetLastError();
}


hipError_t launch_gemm_chunked(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w,
                               int64_t ldw, float *y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                               bool a_zero_padded, hipStream_t stream, const float *bias, bool w_nk, float *part,
                               size_t part_bytes, bool geglu)
{
    const GemmSplitPlan p = gemm_split_plan(M, N, K);
    if (p.chunks < 2 || !part || part_bytes < p.workspace_bytes || (geglu && (w_nk || N % 2)))
        return hipErrorNotSupported;
    hipError_t e = launch_gemm_dma(a_hi, a_lo, lda, w, ldw, nullptr, 0, nullptr, nullptr, 0, M, N, K, a_zero_padded,
                                   stream, nullptr, w_nk, p.chunks, part, p.n_pad);
    if (e == hipErrorNotSupported) {
        GemmArgs g{a_hi, a_lo, lda, w, ldw, nullptr, 0, nullptr, nullptr, 0, M, N, K, nullptr, 0, p.chunks, part,
                   p.n_pad};
        e = w_nk ? launch_tile<TileSmall, 0, true>(g, stream) : launch_tile<TileSmall>(g, stream);
    }
    if (e != hipSuccess) return e;
    if (geglu) return launch_partial_geglu_merge(part, p.n_pad, p.chunks, M, N / 2, y, ldy, bias, stream);
    return launch_partial_merge(part, p.n_pad, p.chunks, M, N, y, ldy, bias, stream);
}

// Separate-addition accumulation (see gemm_kernel): one tile configuration,
// 32 x 128 (a wave holds 32 running sums next to its 32 accumulators).
// k_steps_per_add: 0 (plain accumulation in the same configuration, for
// comparison), 1, 4 or 16 sixteen-deep k-steps per separate addition.
hipError_t launch_gemm_separate_add(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w,
                                    int64_t ldw, float *y, int64_t ldy, float *c_hi, float *c_lo, int64_t ldc,
                                    int64_t M, int64_t N, int64_t K, int k_steps_per_add, hipStream_t stream)
{
    GemmArgs g{a_hi, a_lo, lda, w, ldw, y, ldy, c_hi, c_lo, ldc, M, N, K, nullptr, 0, 1, nullptr, 0};
    // The 32 x 128 configuration: its running sums and accumulators fit two
    // waves per SIMD (the 64 x 128 one needs more than 256 registers once the
    // running sums are added and ran 12-45% slower; same bits).
    switch (k_steps_per_add) {
    case 0: return launch_tile<TileSmall, 0>(g, stream);
    case 1: return launch_tile<TileSmall, 1>(g, stream);
    case 4: return launch_tile<TileSmall, 4>(g, stream);
    case 16: return launch_tile<TileSmall, 16>(g, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace cfp32
