// Host-side planning of the K-split small-M and small-grid paths (no device
// code): how many chunks K is cut into, and the workspace the partial sums
// take.  Kept apart from the kernels so that the host logic -- argument
// validation in api.hip and these plans -- can be built on its own, for
// instance with the host sanitizers, without compiling any kernel.
#include "launchers.h"

namespace cfp32 {

namespace {

int64_t gemv_tiles(int64_t N) { return (N + kGemvTileN - 1) / kGemvTileN; }

}  // namespace

GemvPlan gemv_plan(int64_t M, int64_t N, int64_t K)
{
    GemvPlan p{};
    if (M <= 0 || M > kGemvMaxRowsKN || N <= 0 || K <= 0) return p;
    const int64_t ntiles = gemv_tiles(N);
    if (ntiles > ((int64_t)1 << 40)) return p;  // keeps the byte count below in range
    p.stages = (K + kGemvStageRows - 1) / kGemvStageRows;
    // At most one block per CU; among those counts, the largest that deals the
    // same number of blocks to each of the 8 XCDs (measured at 1 x 4096 x
    // 14336: 8 chunks, 224 blocks, 0.4 us faster than 9 chunks, 252 blocks).
    int64_t chunks = kGemvTargetBlocks / ntiles;
    for (int64_t c = chunks; c >= 1 && c > chunks - 8; --c)
        if ((c * ntiles) % 8 == 0) {
            chunks = c;
            break;
        }
    if (chunks > p.stages) chunks = p.stages;
    // Above 8 rows the partial sums (8 M N bytes per chunk, written and read
    // back) are kept within a quarter of W's 2 K N bytes.
    if (M > kGemvMaxRows && chunks > K / (16 * M)) chunks = K / (16 * M);
    if (chunks < 1) chunks = 1;
    p.chunks = chunks;
    p.n_pad = ntiles * kGemvTileN;
    p.workspace_bytes = chunks == 1 ? 0 : (size_t)chunks * (size_t)M * 2u * (size_t)p.n_pad * sizeof(float);
    return p;
}

// The GEGLU merge dispatch always follows the product dispatch, so the
// partial sums are kept even for a single chunk.
GemvPlan gemv_geglu_plan(int64_t M, int64_t F, int64_t K)
{
    GemvPlan p = gemv_plan(M, 2 * F, K);
    if (p.chunks > 0) p.workspace_bytes = (size_t)p.chunks * (size_t)M * 2u * (size_t)p.n_pad * sizeof(float);
    return p;
}

GemmSplitPlan gemm_split_plan(int64_t M, int64_t N, int64_t K)
{
    GemmSplitPlan p{1, 0, 0};
    // M <= 64: at 1 x 4096 x 14336 split K cuts M = 9..64 from 72-74 us to
    // 35-52 us.  Above 64 rows too the grid must stay below 128 tiles of
    // 128 x 256 (where the LDS-DMA kernel takes over), the chunks must bring
    // it to at least 128 blocks (192 where the small-grid kernel could run
    // it instead), and the partial sums may take up to W's bytes and 56 MiB.
    // Against the generic 32 x 128 tile (one launch, transposed W reads):
    // 65 / 96 / 192 / 256 x 4096 x 14336 56.0 / 58.1 / 94-98 / 100-105 us
    // unsplit, 48.1 / 55.1 / 74.2 / 87-90 us split; 128 x 8192 x 14336 119
    // -> 94 us, 448 x 4096 x 5120 81 -> 64 us, 300 x 4096 x 4096 49 -> 45
    // us; 128 x 4096 x 14336 and 512 x 4096 x 4096 are within 1-4 us either
    // way.  Where K per chunk is short (2048 x 1024 x 2048: 39 -> 55 us;
    // 1024^3: 20 -> 33 us) it lost, which the conditions keep out.
    constexpr int64_t kTileRows = 128, kTileCols = 256, kUnit = 64, kMinUnits = 4, kSmallRows = 64;
    constexpr int64_t kMinBlocksWide = 128, kMinBlocksKsplit = 192;
    constexpr int64_t kMaxPartBytesWide = (int64_t)56 << 20;
    if (M <= kGemvMaxRows || N <= 0 || K <= 0 || K % 8) return p;
    if (M > ((int64_t)1 << 40) || N > ((int64_t)1 << 40)) return p;
    const int64_t tiles = ((M + kTileRows - 1) / kTileRows) * ((N + kTileCols - 1) / kTileCols);
    if (tiles >= 128) return p;
    int64_t c = 256 / tiles;
    for (int64_t cc = c; cc >= 1 && cc > c - 8; --cc)
        if ((cc * tiles) % 8 == 0) {
            c = cc;
            break;
        }
    const int64_t units = (K + kUnit - 1) / kUnit;
    if (c > units / kMinUnits) c = units / kMinUnits;
    const int64_t n_pad = (N + 63) / 64 * 64;
    if (M <= kSmallRows) {
        // From 17 rows, no split where the generic kernel's 32 x 128 tiles
        // make 192 to 256 blocks (one per CU at most) and K <= 4096: that
        // one-launch form walks all of K without partial sums (64 / 48 x
        // 4096 x 14336: 45.1 / 42.0 -> 40.6 / 39.2 us; [N, K] 64 rows 45.4 ->
        // 41.6 us; 64 x 2048 x 14336 27.5 -> 20.7 us; [N, K] 64 x 4096 x
        // 12288 41.7 -> 39.4 us).  On smaller grids, with two blocks per CU
        // or with longer K, split K stays ahead (64 x 4096 x 4096: 26 us
        // either way; 64 x 14336 x 4096: 52 against 94 us; 40 / 64 x 4096 x
        // 28672: 60.6 / 70.0 against 67.3 / 75.0 us; 64 x 8192 x 14336: 69.8
        // against 76.3 us; GEGLU at 40 x 4096 x 2 * 14336: 67 against 91 us).
        const int64_t tiles32 = ((M + 31) / 32) * ((N + 127) / 128);
        if (M > 16 && tiles32 >= 192 && tiles32 <= 256 && K <= 4096) return p;
        // The partial sums (8 M N bytes per chunk, written and read back)
        // stay within a quarter of W's 2 K N bytes.
        if (c > K / (16 * M)) c = K / (16 * M);
    } else {
        // Within W's bytes and 56 MiB, and enough blocks to fill the GPU.
        if (c > K / (4 * M)) c = K / (4 * M);
        const int64_t cap = kMaxPartBytesWide / (M * 2 * n_pad * (int64_t)sizeof(float));
        if (c > cap) c = cap;
        // Where the small-grid kernel takes the grid (at most
        // kKsplitMaxBlocks tiles of 32 x 64) it wins below 192 blocks (96 x
        // 4096 x 4096: 28 us there, 39 us split in 160 blocks).
        const int64_t min_blocks = ksplit_blocks(M, N) <= kKsplitMaxBlocks ? kMinBlocksKsplit : kMinBlocksWide;
        if (c * tiles < min_blocks) return p;
    }
    if (c < 2) return p;
    p.chunks = c;
    p.n_pad = n_pad;
    p.workspace_bytes = (size_t)c * (size_t)M * 2u * (size_t)p.n_pad * sizeof(float);
    return p;
}

int64_t ksplit_blocks(int64_t M, int64_t N)
{
    return ((M + kKsplitTileM - 1) / kKsplitTileM) * ((N + kKsplitTileN - 1) / kKsplitTileN);
}

bool ksplit_supported(const void *x, int64_t ldx, const void *w, int64_t ldw, int64_t M, int64_t N, int64_t K,
                      bool w_nk)
{
    // Byte offsets the kernel forms (buffer loads: 31 bits, with room for
    // the stages it loads past K and a tile's overhang) stay below this.
    constexpr int64_t kLimit = 0x7FFFFFF0 - (1 << 20);
    if (M <= 0 || N <= 0 || K <= 0 || K % 8 || ldx % 4 || ldw % 8) return false;
    if (((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w)) & 15) != 0) return false;
    if (M > kLimit || N > kLimit || K > kLimit) return false;
    if ((M + kKsplitTileM) * ldx * 4 + (K + 1024) * 4 >= kLimit) return false;
    const int64_t w_bytes = w_nk ? (N + kKsplitTileN) * ldw * 2 + (K + 1024) * 2 : (K + 1024) * ldw * 2;
    return w_bytes < kLimit && N + kKsplitTileN < ((int64_t)1 << 31);
}

}  // namespace cfp32
