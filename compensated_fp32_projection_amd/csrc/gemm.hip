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
//     one barrier per stage.
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
#include "device_common.h"
#include "launchers.h"

namespace cfp32 {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;        // k per stage
constexpr int kKG = kBK / 8;   // k-granules per stage
constexpr int kGroupM = 4;     // tile-rows per scheduling group
constexpr int kXcds = 8;       // XCDs on MI355X; blocks are dealt to them round-robin

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

template <class T, bool AL_A, bool AL_W>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g)
{
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
    int64_t bid = blockIdx.x;
    {
        const int64_t q = total / kXcds, r = total % kXcds;
        const int64_t xcd = bid % kXcds, local = bid / kXcds;
        bid = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
    }
    const int64_t group_span = (int64_t)kGroupM * nbn;
    const int64_t first_m = (bid / group_span) * kGroupM;
    const int64_t gsize = (nbm - first_m) < kGroupM ? (nbm - first_m) : kGroupM;
    const int64_t tile_m = first_m + (bid % group_span) % gsize;
    const int64_t tile_n = (bid % group_span) / gsize;
    const int64_t m0 = tile_m * T::BM;
    const int64_t n0 = tile_n * T::BN;

    floatx16_t acc_hi[T::TM][T::TN];
    floatx16_t acc_lo[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            acc_hi[i][j] = floatx16_t{};
            acc_lo[i][j] = floatx16_t{};
        }

    uint4 ra[2][T::A_CHUNKS];
    uint4 rw[T::W_ITERS][8];

    auto load_stage = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < T::A_CHUNKS; ++i) {
            const int c = tid + kThreads * i;
            const int kg = c & 7, row = c >> 3;
            const int64_t gm = m0 + row, gk = k0 + 8 * kg;
            if (gm < g.M) {
                ra[0][i] = load_row8<AL_A>(g.a_hi + gm * g.lda, gk, g.K);
                ra[1][i] = load_row8<AL_A>(g.a_lo + gm * g.lda, gk, g.K);
            } else {
                ra[0][i] = make_uint4(0, 0, 0, 0);
                ra[1][i] = make_uint4(0, 0, 0, 0);
            }
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
                    rw[j][r] = gk < g.K ? load_row8<AL_W>(g.w + gk * g.ldw, gn, g.N) : make_uint4(0, 0, 0, 0);
                }
            }
        }
    };

    auto store_stage = [&](int st) {
        uint4 *s = lds + st * T::LDS_STAGE;
#pragma unroll
        for (int i = 0; i < T::A_CHUNKS; ++i) {
            const int c = tid + kThreads * i;
            const int kg = c & 7, row = c >> 3;
            s[a_slot<T>(0, kg, row)] = ra[0][i];
            s[a_slot<T>(1, kg, row)] = ra[1][i];
        }
#pragma unroll
        for (int j = 0; j < T::W_ITERS; ++j) {
            const int b = tid + kThreads * j;
            if (b < T::W_BLOCKS) {
                const int kgw = b / (T::BN / 8), nc = b % (T::BN / 8);
                // rw[j][r] holds W[k = 8*kgw + r][n = 8*nc .. 8*nc + 7]; gather
                // column e into one granule of eight k values.
                const uint32_t *v = reinterpret_cast<const uint32_t *>(rw[j]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int q = e >> 1, sh = 16 * (e & 1);
                    uint32_t d[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const uint32_t lo16 = (v[(2 * p) * 4 + q] >> sh) & 0xFFFFu;
                        const uint32_t hi16 = (v[(2 * p + 1) * 4 + q] >> sh) & 0xFFFFu;
                        d[p] = lo16 | (hi16 << 16);
                    }
                    s[w_slot<T>(kgw, 8 * nc + e)] = make_uint4(d[0], d[1], d[2], d[3]);
                }
            }
        }
    };

    auto compute_stage = [&](int st) {
        const uint4 *s = lds + st * T::LDS_STAGE;
#pragma unroll
        for (int ks = 0; ks < kKG / 2; ++ks) {
            const int kg = 2 * ks + (lane >> 5);
            half8_t ah[T::TM], al[T::TM], bw[T::TN];
#pragma unroll
            for (int i = 0; i < T::TM; ++i) {
                const int row = wm * T::WTM + i * 32 + (lane & 31);
                ah[i] = __builtin_bit_cast(half8_t, s[a_slot<T>(0, kg, row)]);
                al[i] = __builtin_bit_cast(half8_t, s[a_slot<T>(1, kg, row)]);
            }
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                const int n = wn * T::WTN + j * 32 + (lane & 31);
                bw[j] = __builtin_bit_cast(half8_t, s[w_slot<T>(kg, n)]);
            }
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int j = 0; j < T::TN; ++j) {
                    acc_hi[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i], bw[j], acc_hi[i][j], 0, 0, 0);
                    acc_lo[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[i], bw[j], acc_lo[i][j], 0, 0, 0);
                }
        }
    };

    const int64_t nk = (g.K + kBK - 1) / kBK;
    if (nk > 0) {
        load_stage(0);
        store_stage(0);
    }
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = (int)(kt & 1);
        if (kt + 1 < nk) load_stage((kt + 1) * kBK);
        compute_stage(cur);
        if (kt + 1 < nk) store_stage(cur ^ 1);
        __syncthreads();
    }

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
                const float h = acc_hi[i][j][e], l = acc_lo[i][j][e];
                if (g.y) g.y[row * g.ldy + col] = merge_value(h, l);
                if (g.c_hi) {
                    g.c_hi[row * g.ldc + col] = h;
                    g.c_lo[row * g.ldc + col] = l;
                }
            }
        }
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <class T>
hipError_t launch_tile(const GemmArgs &g, hipStream_t stream)
{
    const int64_t blocks = ((g.M + T::BM - 1) / T::BM) * ((g.N + T::BN - 1) / T::BN);
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const bool al_a = (g.lda % 8 == 0) && aligned16(g.a_hi) && aligned16(g.a_lo);
    const bool al_w = (g.ldw % 8 == 0) && aligned16(g.w);
    const dim3 grid((unsigned)blocks);
    if (al_a && al_w)
        gemm_kernel<T, true, true><<<grid, kThreads, 0, stream>>>(g);
    else if (al_a)
        gemm_kernel<T, true, false><<<grid, kThreads, 0, stream>>>(g);
    else if (al_w)
        gemm_kernel<T, false, true><<<grid, kThreads, 0, stream>>>(g);
    else
        gemm_kernel<T, false, false><<<grid, kThreads, 0, stream>>>(g);
    return hipGetLastError();
}

template <class T>
int64_t tiles_of(int64_t M, int64_t N)
{
    return ((M + T::BM - 1) / T::BM) * ((N + T::BN - 1) / T::BN);
}

}  // namespace

// Tile choice: the largest tile that still gives at least one block per CU
// (256 CUs); below that, the smallest tile, which has the most blocks.
hipError_t launch_gemm(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w,
                       int64_t ldw, float *y, int64_t ldy, float *c_hi, float *c_lo, int64_t ldc,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    GemmArgs g{a_hi, a_lo, lda, w, ldw, y, ldy, c_hi, c_lo, ldc, M, N, K};
    constexpr int64_t kCus = 256;
    if (tiles_of<TileLarge>(M, N) >= kCus) return launch_tile<TileLarge>(g, stream);
    if (tiles_of<TileMedium>(M, N) >= kCus) return launch_tile<TileMedium>(g, stream);
    return launch_tile<TileSmall>(g, stream);
}

}  // namespace cfp32
