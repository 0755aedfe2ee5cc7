// Small-M projection (decode-sized inputs: up to 8 rows of x, and up to 16
// with [K, N] weights that allow 16-byte loads).
//
// The laya.cpp Vulkan guide runs small projections at their real batch size,
// with no padding of the row count.  With few rows the projection streams W
// once and does little arithmetic per byte, so it is bound by HBM bandwidth;
// W is read in whole 1 KiB row segments (512 columns), the access pattern
// that streams fastest, and K is cut into row chunks so that there are
// enough blocks to keep every CU loading.
//
// Two dispatches, as in the guide's description of the method (the products,
// then the merge as one dispatch):
//
//  1. gemv_mfma_kernel<G> -- split + both products.  A block (4 waves) owns
//     one 512-column tile of one row chunk and walks it in stages of 32 rows
//     through a four-buffer LDS ring filled by LDS-DMA loads (W: one 1 KiB
//     row per wave instruction, streaming cache policy; x: the chunk's 32
//     columns of every row, 4 bytes per lane, so x needs no alignment).
//     The matrix unit does the products: the hi and lo halves of each group
//     of 8 rows are interleaved into the 16 rows of one
//     v_mfma_f32_16x16x32_f16 A operand (row 2m = hi of x row m, row 2m + 1
//     = lo), so one MFMA chain forms C_hi and C_lo together with FP32
//     accumulators, and the split of x happens in registers as the A
//     fragment is built; G = 2 groups share every B fragment.  Each wave
//     owns 128 columns (8 MFMA tiles); no reduction across waves is needed.
//     The block writes its chunk's C_hi and C_lo partial sums to the
//     workspace, or, when K is a single chunk, merges and writes y itself
//     (no second dispatch).  For M <= 2, gemv_valu_kernel runs the same
//     chunks with FP32 FMAs on the vector unit and deeper load queues.
//  2. gemv_merge4_kernel (four outputs per thread), or gemv_merge_kernel
//     (one: for small outputs, in 64-thread blocks, and where 16-byte loads
//     of the partial sums are not possible) -- for every output, sums the
//     chunk partials of C_hi and of C_lo in chunk order, then merges
//     y = C_hi + C_lo / 1024.  The split-K GEMM path uses them too.
//
// Every summation order is fixed, so results are identical from run to run.
// W that is not 16-byte aligned with ldw % 8 == 0 (or too large for 32-bit
// buffer offsets) goes through gemv_generic_kernel instead: one launch, a
// block per 64 columns and all of K, W rows read at any 2-byte offset
// (batched dword loads and funnel shifts), FP32 FMAs on the vector unit (an
// FP16 x FP16 product is exact in FP32, so fusing it into the accumulation
// rounds once, as the matrix unit does).
#include <climits>
#include <type_traits>

#include "device_common.h"
#include "launchers.h"

#define CFP32_LDS __attribute__((address_space(3)))

namespace cfp32 {

namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));

constexpr int kNoOffset = 0x7FFFFFF0;      // a raw buffer load here reads zero
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit buffer, gfx9 family
constexpr int kStreamAux = 2;             // cache policy "nt": W is read once, do not keep it in cache
constexpr int kTileN = kGemvTileN;        // columns per tile: 1 KiB of an FP16 row
constexpr int kTargetBlocks = kGemvTargetBlocks;  // one block per CU
constexpr int kT = 256;                   // 4 waves, 128 columns each
constexpr int kBK = kGemvStageRows;       // rows of W per stage (the MFMA's k)
constexpr int kRowSlots = kTileN / 8;     // 16-byte granules per W row in LDS
constexpr int kWSlots = kBK * kRowSlots;  // 2048 granules: 32 KiB of W per stage
constexpr int kMaxGroups = 2;             // matrix-unit kernel: up to 2 groups of 8 rows of x
constexpr int kXSlots = 64 * kMaxGroups;  // x[8 G rows][32 columns] FP32 per stage (G KiB)
// Loads per wave per stage: 8 W rows + one x load per group of 8 rows.
template <int G>
constexpr int loads_per_stage() { return kBK / (kT / 64) + G; }

// Separate LDS objects per ring buffer (and for W and x), so that the
// compiler can tell which DMA fills which buffer and adds no waits of its own.
__shared__ uint4 g_wring0[kWSlots];
__shared__ uint4 g_wring1[kWSlots];
__shared__ uint4 g_wring2[kWSlots];
__shared__ uint4 g_wring3[kWSlots];
__shared__ uint4 g_xring0[kXSlots];
__shared__ uint4 g_xring1[kXSlots];
__shared__ uint4 g_xring2[kXSlots];
__shared__ uint4 g_xring3[kXSlots];

template <int B>
__device__ __forceinline__ uint4 *wring()
{
    if constexpr (B == 0) return g_wring0;
    else if constexpr (B == 1) return g_wring1;
    else if constexpr (B == 2) return g_wring2;
    else return g_wring3;
}

template <int B>
__device__ __forceinline__ uint4 *xring()
{
    if constexpr (B == 0) return g_xring0;
    else if constexpr (B == 1) return g_xring1;
    else if constexpr (B == 2) return g_xring2;
    else return g_xring3;
}

// W row r of a stage sits in granules [64 r, 64 r + 64); its column granule c
// (columns 8c .. 8c + 7) is stored at position c ^ 2 (r % 4), so the four
// rows that one transposed read touches fall on different banks.
__device__ __forceinline__ int w_slot(int r, int c) { return r * kRowSlots + (c ^ ((r & 3) << 1)); }

// s_waitcnt immediates (gfx9 encoding): vector-memory count n, LDS count 0.
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (0 << 8); }
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ void block_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

struct GemvArgs {
    const float *x;
    int64_t ldx;
    const uint16_t *w;
    int64_t ldw;
    float *part;      // [chunks][M][2][n_pad] partial sums (chunks > 1)
    float *y;         // written directly when chunks == 1
    int64_t ldy;
    int64_t n_pad;
    int64_t M, N, K;
    int64_t stages;   // ceil(K / 32)
    int64_t chunks;   // the stages split as evenly as possible, in order
    int64_t ntiles;   // ceil(N / 512)
    const float *bias;  // FP32 [N] added to y after the merge, or null
    int geglu;          // partial sums always (a GEGLU merge follows), never y
};

template <int G>
__global__ __launch_bounds__(kT) void gemv_mfma_kernel(GemvArgs g)
{
    constexpr int kLoadsPerStage = loads_per_stage<G>();
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Chunk c holds `base` stages, plus one for the first `extra` chunks.
    const unsigned ntiles = (unsigned)g.ntiles;
    const int tile = (int)(blockIdx.x % ntiles);
    const int chunk = (int)(blockIdx.x / ntiles);
    const int base = (int)(g.stages / g.chunks);
    const int extra = (int)(g.stages % g.chunks);
    const int s_begin = chunk * base + (chunk < extra ? chunk : extra);
    const int ns = base + (chunk < extra ? 1 : 0);  // >= 1: chunks <= stages
    const int64_t s_end = s_begin + ns;
    const int64_t r0 = (int64_t)kBK * s_begin;
    const int64_t n0 = tile * kTileN;
    const int M = (int)g.M;

    const __amdgpu_buffer_rsrc_t rs_w =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(g.w), 0, (int)(g.K * g.ldw * 2), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rs_x =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(g.x), 0, (int)(g.M * g.ldx * 4), kBufferWord3);

    // DMA sources of this lane.  W: the wave loads rows 8 wave + j of a stage,
    // lane l the granule that belongs at position l of that row.  x: load q of
    // the wave fills rows 2 j and 2 j + 1 (j = wave + 4 q) of the stage's x
    // rows (8 granules each), lane l column l % 32.  A load whose
    // row lies past the chunk (or past K), or whose column lies past N, gets
    // an offset no buffer reaches and writes zeros; each limit below is the
    // first stage row offset k0 at which that happens.
    const int k_limit = (int)(kBK * s_end < g.K ? kBK * s_end : g.K);
    const unsigned ldw2 = (unsigned)(g.ldw * 2);
    int w_col[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = lane ^ (q << 1);  // rows with r % 4 == q
        w_col[q] = n0 + 8 * c < g.N ? (int)((n0 + 8 * c) * 2) : -1;
    }
    int w_kend[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w_kend[j] = w_col[j & 3] >= 0 ? k_limit - (8 * wave + j) : INT_MIN;
    const int xk = lane & 31;
    int x_kend[G], x_off[G];
#pragma unroll
    for (int q = 0; q < G; ++q) {
        const int xm = 2 * (wave + 4 * q) + (lane >> 5);
        x_kend[q] = xm < M ? k_limit - xk : INT_MIN;
        x_off[q] = xm < M ? (int)((xm * g.ldx + xk) * 4) : 0;
    }

    auto issue = [&](auto buf_tag, int s) {
        constexpr int B = decltype(buf_tag)::value;
        uint4 *buf = wring<B>();
        const int k0 = (int)r0 + kBK * s;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 8 * wave + j;
            const int o = k0 < w_kend[j] ? w_col[j & 3] + (int)((unsigned)(k0 + r) * ldw2) : kNoOffset;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_w, (CFP32_LDS void *)(buf + r * kRowSlots), 16, o, 0, 0,
                                                     kStreamAux);
        }
#pragma unroll
        for (int q = 0; q < G; ++q) {
            const int ox = k0 < x_kend[q] ? x_off[q] + 4 * k0 : kNoOffset;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_x, (CFP32_LDS void *)(xring<B>() + 16 * (wave + 4 * q)), 4,
                                                     ox, 0, 0, 0);
        }
    };

    // Fragment addresses.  A (group q of 8 x rows): lane l is row i = l % 16
    // (x row 8 q + i / 2, hi for even i, lo for odd i) and k = 8 (l / 16) + e.
    // B (two transposed reads of 4 rows each): lane l's column is
    // 128 wave + 16 t + l % 16; each B fragment serves every group.
    const int ai = lane & 15;
    const int am = ai >> 1;
    const bool a_lo = ai & 1;
    const int kq = lane >> 4;
    const int j4 = (lane & 15) >> 2;
    const int b_row = 8 * kq + j4;                  // + 4 h
    const int b_col = 16 * wave + ((lane & 3) >> 1);  // granule, + 2 t
    const int b_half = (lane & 1) * 8;                // byte within the granule

    floatx4_t acc[G][8];
#pragma unroll
    for (int q = 0; q < G; ++q)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[q][t] = floatx4_t{};

    auto compute = [&](const uint4 *buf, const uint4 *xb) {
        half8_t b[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            short4_t v[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r = b_row + 4 * h;
                const int byte = w_slot(r, b_col + 2 * t) * 16 + b_half;
                v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CFP32_LDS short4_t *)((CFP32_LDS char *)buf + byte));
            }
            const short8_t bv = {v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
            b[t] = __builtin_bit_cast(half8_t, bv);
        }
#pragma unroll
        for (int q = 0; q < G; ++q) {
            // x[8 q + am][8 kq .. 8 kq + 7] (rows of 32 floats = 8 granules).
            const int row = 8 * q + am;
            const floatx4_t x0 = __builtin_bit_cast(floatx4_t, xb[row * 8 + 2 * kq]);
            const floatx4_t x1 = __builtin_bit_cast(floatx4_t, xb[row * 8 + 2 * kq + 1]);
            const bool live = row < M;
            half8_t a;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                _Float16 h, l;
                split_value(e < 4 ? x0[e] : x1[e - 4], h, l);
                a[e] = live ? (a_lo ? l : h) : (_Float16)0.0f;
            }
#pragma unroll
            for (int t = 0; t < 8; ++t)
                acc[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[t], acc[q][t], 0, 0, 0);
        }
    };

    // One stage: refill the buffer read one stage ago with stage s + 3, use
    // stage s, then wait until stage s + 1 has landed (two stages may stay in
    // flight) and this wave's LDS reads are done; the barrier publishes stage
    // s + 1 and frees stage s's buffer for the next refill.
    auto stage = [&](auto buf_tag, int s) {
        constexpr int B = decltype(buf_tag)::value;
        issue(std::integral_constant<int, (B + 3) & 3>{}, s + 3);
        compute(wring<B>(), xring<B>());
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * kLoadsPerStage));
        block_barrier();
    };

    issue(std::integral_constant<int, 0>{}, 0);
    issue(std::integral_constant<int, 1>{}, 1);
    issue(std::integral_constant<int, 2>{}, 2);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kLoadsPerStage));  // stage 0 landed for this wave
    block_barrier();
    int s = 0;
    for (; s + 4 <= ns; s += 4) {
        stage(std::integral_constant<int, 0>{}, s);
        stage(std::integral_constant<int, 1>{}, s + 1);
        stage(std::integral_constant<int, 2>{}, s + 2);
        stage(std::integral_constant<int, 3>{}, s + 3);
    }
    if (s < ns) stage(std::integral_constant<int, 0>{}, s);
    if (s + 1 < ns) stage(std::integral_constant<int, 1>{}, s + 1);
    if (s + 2 < ns) stage(std::integral_constant<int, 2>{}, s + 2);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the trailing zero loads land before the block exits

    // 16x16 accumulator layout: lane l holds column l % 16, rows 4 (l / 16) + e.
    // Rows 4 (l / 16) + 0, 1 are hi, lo of x row 8 grp + 2 (l / 16); + 2, 3 of
    // the next.
    const int64_t col0 = n0 + 128 * wave + (lane & 15);
#pragma unroll
    for (int grp = 0; grp < G; ++grp)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int m = 8 * grp + 2 * kq + q;
        if (m >= M) continue;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int64_t n = col0 + 16 * t;
            const float ch = acc[grp][t][2 * q], cl = acc[grp][t][2 * q + 1];
            if (g.chunks == 1 && !g.geglu) {
                if (n < g.N) {
                    float v = merge_value(ch, cl);
                    if (g.bias) v = v + g.bias[n];
                    __builtin_nontemporal_store(v, g.y + m * g.ldy + n);
                }
            } else {
                // Streaming stores: the merge dispatch reads these from
                // memory anyway (they come from every XCD).
                float *p = g.part + ((chunk * g.M + m) * 2) * g.n_pad + n;
                __builtin_nontemporal_store(ch, p);
                __builtin_nontemporal_store(cl, p + g.n_pad);
            }
        }
    }
}

// M <= 2: the same chunks and partial sums from the vector unit, which for
// one or two rows streams W about a microsecond faster than the matrix-unit
// kernel (its 16 waves per block keep more loads in flight; at M <= 2 the
// FP32 FMAs cost little).  A block of 1024 threads owns one 512-column tile
// of one chunk; wave v takes rows r0 + v, r0 + v + 16, ... and lane l columns
// 8l .. 8l + 7, with 16 rows of loads (1 KiB each, streaming policy) in
// flight (8 measured the same at 1 x 4096 x 14336 and 2.9 us slower at
// 1 x 8192 x 4096, whose 256-row chunks then took two rounds per wave; 92 /
// 126 registers for one / two rows keep four waves per SIMD); x is read
// with scalar loads (every lane needs the same value).
// Products hi * w and lo * w accumulate with FP32 fused multiply-adds (the
// FP16 x FP16 product is exact, so each step rounds once, as in the matrix
// unit).  The 16 waves are summed in index order through LDS; the block then
// writes its chunk's partial sums, or merges and writes y when K is one
// chunk.
constexpr int kValuThreads = 1024;
constexpr int kValuU = 16;

template <int MR>
__global__ __launch_bounds__(kValuThreads) void gemv_valu_kernel(GemvArgs g)
{
    constexpr int WV = kValuThreads / 64;
    __shared__ float red[WV][MR][2][kTileN];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const unsigned ntiles = (unsigned)g.ntiles;
    const int tile = (int)(blockIdx.x % ntiles);
    const int chunk = (int)(blockIdx.x / ntiles);
    const int base = (int)(g.stages / g.chunks);
    const int extra = (int)(g.stages % g.chunks);
    const int s_begin = chunk * base + (chunk < extra ? chunk : extra);
    const int ns = base + (chunk < extra ? 1 : 0);
    const int64_t r0 = (int64_t)kBK * s_begin;
    const int64_t r1 = (kBK * (int64_t)(s_begin + ns) < g.K) ? kBK * (int64_t)(s_begin + ns) : g.K;
    const int64_t n0 = (int64_t)tile * kTileN;
    const int64_t n = n0 + 8 * lane;

    const __amdgpu_buffer_rsrc_t rs_w =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(g.w), 0, (int)(g.K * g.ldw * 2), kBufferWord3);

    float sh[MR][8], sl[MR][8];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) sh[m][e] = 0.0f, sl[m][e] = 0.0f;

    // Rows past r1 load zeros (W) and read x as 0 through selects, not
    // branches: a branch around a load (the x row test) made the compiler
    // wait for every load in flight at the join (M = 2: 24.9 -> 23.8 us).
    // Their products are +0 and leave the sums' bits unchanged (a sum that
    // starts at +0 never becomes -0).  A second set of rows in flight
    // (double-buffered registers) ran slower at M = 1 (23.0 -> 23.6 us).
    const int64_t step = (int64_t)WV * kValuU;
    auto load = [&](uint4 (&wv)[kValuU], float (&xv)[kValuU][MR], int64_t kb) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kValuU; ++u) {
            const int64_t k = kb + (int64_t)u * WV;
            const bool in = k < r1;
            const int off = (in & (n < g.N)) ? (int)((k * g.ldw + n) * 2) : kNoOffset;
            wv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_w, off, 0, kStreamAux));
            const int64_t kc = in ? k : r1 - 1;  // a row inside x, read and then replaced by 0
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const float v = g.x[m * g.ldx + kc];
                xv[u][m] = in ? v : 0.0f;
            }
        }
    };
    auto compute = [&](const uint4 (&wv)[kValuU], const float (&xv)[kValuU][MR]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kValuU; ++u) {
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
    };
    for (int64_t kb = r0 + wave; kb < r1; kb += step) {
        uint4 wv[kValuU];
        float xv[kValuU][MR];
        load(wv, xv, kb);
        compute(wv, xv);
    }

#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            red[wave][m][0][8 * lane + e] = sh[m][e];
            red[wave][m][1][8 * lane + e] = sl[m][e];
        }
    __syncthreads();
    // One thread per (row, column) of the tile: C_hi and C_lo, waves in order.
    for (int o = threadIdx.x; o < MR * kTileN; o += kValuThreads) {
        const int col = o % kTileN;
        const int m = o / kTileN;
        float th = 0.0f, tl = 0.0f;
#pragma unroll
        for (int v = 0; v < WV; ++v) {
            th += red[v][m][0][col];
            tl += red[v][m][1][col];
        }
        const int64_t nn = n0 + col;
        if (g.chunks == 1 && !g.geglu) {
            if (nn < g.N) {
                float val = merge_value(th, tl);
                if (g.bias) val = val + g.bias[nn];
                __builtin_nontemporal_store(val, g.y + m * g.ldy + nn);
            }
        } else {
            float *pp = g.part + ((chunk * g.M + m) * 2) * g.n_pad + nn;
            __builtin_nontemporal_store(th, pp);
            __builtin_nontemporal_store(tl, pp + g.n_pad);
        }
    }
}

// Product dispatch: the vector-unit kernel for M <= 2, the matrix-unit one above.
hipError_t launch_product(const GemvArgs &g, int64_t blocks, hipStream_t stream)
{
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if (g.M == 1)
        gemv_valu_kernel<1><<<dim3((unsigned)blocks), kValuThreads, 0, stream>>>(g);
    else if (g.M == 2)
        gemv_valu_kernel<2><<<dim3((unsigned)blocks), kValuThreads, 0, stream>>>(g);
    else if (g.M <= 8)
        gemv_mfma_kernel<1><<<dim3((unsigned)blocks), kT, 0, stream>>>(g);
    else if (g.M <= 16)
        gemv_mfma_kernel<2><<<dim3((unsigned)blocks), kT, 0, stream>>>(g);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// y[m, n] = merge(sum over chunks of C_hi, sum over chunks of C_lo), chunks in
// order.  The partial sums were written by blocks on every XCD, so they come
// from memory, not from this XCD's L2: all loads of a batch of kMergeBatch
// chunks are issued before the first add, one memory latency per batch.
constexpr int kMergeBatch = 16;

template <int TB>
__global__ __launch_bounds__(TB) void gemv_merge_kernel(const float *__restrict__ part, int64_t n_pad,
                                                         int64_t chunks, int M, int64_t N,
                                                         float *__restrict__ y, int64_t ldy,
                                                         const float *__restrict__ bias)
{
    const int64_t i = (int64_t)blockIdx.x * TB + threadIdx.x;
    if (i >= (int64_t)M * N) return;
    const int m = (int)(i / N);
    const int64_t n = i % N;
    const int64_t stride = (int64_t)M * 2 * n_pad;  // from one chunk to the next
    const float *p = part + (int64_t)m * 2 * n_pad + n;
    float th = 0.0f, tl = 0.0f;
    for (int64_t c0 = 0; c0 < chunks; c0 += kMergeBatch) {
        float vh[kMergeBatch], vl[kMergeBatch];
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
            const bool in = c0 + j < chunks;
            vh[j] = in ? __builtin_nontemporal_load(p + (c0 + j) * stride) : 0.0f;
            vl[j] = in ? __builtin_nontemporal_load(p + (c0 + j) * stride + n_pad) : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
            if (c0 + j < chunks) {
                th += vh[j];
                tl += vl[j];
            }
        }
    }
    float v = merge_value(th, tl);
    if (bias) v = v + bias[n];
    __builtin_nontemporal_store(v, y + m * ldy + n);
}

// The same merge over four consecutive columns per thread: 16-byte loads of
// the partial sums (n_pad is a multiple of 4, the partial sums 16-byte
// aligned), a quarter of the load instructions for the same bytes.  Each
// column is summed exactly as above (from +0, chunks in order).  VY: rows of
// y take 16-byte stores (ldy % 4 == 0, y 16-byte aligned).  TB threads
// per block: 64 where 256 would leave most CUs without a block.
constexpr int kMergeBatch4 = 8;

template <bool VY, int TB>
__global__ __launch_bounds__(TB) void gemv_merge4_kernel(const float *__restrict__ part, int64_t n_pad,
                                                          int64_t chunks, int M, int64_t N,
                                                          float *__restrict__ y, int64_t ldy,
                                                          const float *__restrict__ bias)
{
    const int64_t groups = (N + 3) / 4;
    const int64_t i = (int64_t)blockIdx.x * TB + threadIdx.x;
    if (i >= (int64_t)M * groups) return;
    const int m = (int)(i / groups);
    const int64_t n = 4 * (i % groups);
    const int64_t stride = (int64_t)M * 2 * n_pad;  // from one chunk to the next
    const float *p = part + (int64_t)m * 2 * n_pad + n;
    floatx4_t th = {0.0f, 0.0f, 0.0f, 0.0f}, tl = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t c0 = 0; c0 < chunks; c0 += kMergeBatch4) {
        floatx4_t vh[kMergeBatch4], vl[kMergeBatch4];
#pragma unroll
        for (int j = 0; j < kMergeBatch4; ++j) {
            const bool in = c0 + j < chunks;
            const floatx4_t *q = reinterpret_cast<const floatx4_t *>(p + (c0 + j) * stride);
            vh[j] = in ? __builtin_nontemporal_load(q) : floatx4_t{};
            vl[j] = in ? __builtin_nontemporal_load(reinterpret_cast<const floatx4_t *>(p + (c0 + j) * stride + n_pad))
                       : floatx4_t{};
        }
#pragma unroll
        for (int j = 0; j < kMergeBatch4; ++j) {
            if (c0 + j < chunks) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    th[e] += vh[j][e];
                    tl[e] += vl[j][e];
                }
            }
        }
    }
    floatx4_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[e] = merge_value(th[e], tl[e]);
        if (bias && n + e < N) v[e] = v[e] + bias[n + e];
    }
    float *out = y + m * ldy + n;
    if (VY && n + 4 <= N) {
        __builtin_nontemporal_store(v, reinterpret_cast<floatx4_t *>(out));
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n + e < N) __builtin_nontemporal_store(v[e], out + e);
    }
}

// GEGLU merge (the laya.cpp Vulkan guide's fused GEGLU step, graph
// paragraph): for output (m, n < F), the chunk sums of columns n (gate) and
// F + n (up) in chunk order, each merged (plus its bias), then
// out = gelu(gate) * up.
__global__ __launch_bounds__(256) void gemv_geglu_merge_kernel(const float *__restrict__ part, int64_t n_pad,
                                                               int64_t chunks, int M, int64_t F,
                                                               float *__restrict__ y, int64_t ldy,
                                                               const float *__restrict__ bias)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * F) return;
    const int m = (int)(i / F);
    const int64_t n = i % F;
    const int64_t stride = (int64_t)M * 2 * n_pad;
    float v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // h = 0: gate column n, h = 1: up column F + n
        const float *p = part + (int64_t)m * 2 * n_pad + n + h * F;
        float th = 0.0f, tl = 0.0f;
        for (int64_t c0 = 0; c0 < chunks; c0 += kMergeBatch) {
            float vh[kMergeBatch], vl[kMergeBatch];
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) {
                const bool in = c0 + j < chunks;
                vh[j] = in ? __builtin_nontemporal_load(p + (c0 + j) * stride) : 0.0f;
                vl[j] = in ? __builtin_nontemporal_load(p + (c0 + j) * stride + n_pad) : 0.0f;
            }
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) {
                if (c0 + j < chunks) {
                    th += vh[j];
                    tl += vl[j];
                }
            }
        }
        v[h] = merge_value(th, tl);
        if (bias) v[h] = v[h] + bias[n + h * F];
    }
    __builtin_nontemporal_store(gelu_value(v[0]) * v[1], y + m * ldy + n);
}

// Fallback for W that is not 16-byte aligned or too large for 32-bit buffer
// offsets: a block per 64 columns and all of K, a thread per 8 columns and
// every 64th row, the same fixed-order reduction inside the block, one
// launch, no workspace.
//   FAST (W within 31-bit byte offsets, ldw >= 16): rows 0 .. K - 2 come in
//   batches of kGenericU rows per thread, all of a batch's loads issued
//   before any is used.  The 8 columns at any even byte offset lie in the 20
//   bytes from the dword below it (a 16-byte and a 4-byte buffer load), and
//   a funnel shift by 0 or 16 bits picks them out; for those rows the 20
//   bytes stay inside W (the next row follows), and columns past N only
//   feed sums that are never stored.  The last row, and every row without
//   FAST, is read by load_row8 (dwords, or elements at the row's end).
//   Each thread adds its rows in increasing k either way: the same bits.
constexpr int kGenericThreads = 512;
constexpr int kGenericNB = 64;
constexpr int kGenericU = 8;  // rows per batch up to 4 rows of x (4 beyond; 16 measured no faster)
constexpr int kGenericNoOffset = 0x7FFFFFC0;  // a load here (and 16 bytes on) reads zero

template <int MR, bool FAST>
__global__ __launch_bounds__(kGenericThreads) void gemv_generic_kernel(const float *__restrict__ x, int64_t ldx,
                                                                       const uint16_t *__restrict__ w, int64_t ldw,
                                                                       float *__restrict__ y, int64_t ldy,
                                                                       int64_t N, int64_t K,
                                                                       const float *__restrict__ bias, int geglu_rmw)
{
    constexpr int CH = kGenericNB / 8;
    constexpr int KL = kGenericThreads / CH;
    constexpr int WAVES = kGenericThreads / 64;
    __shared__ float red[WAVES][CH][MR][8][2];

    const int tid = threadIdx.x;
    const int c = tid % CH;
    const int kl = tid / CH;
    const int64_t n0 = (int64_t)blockIdx.x * kGenericNB;
    const int64_t n = n0 + 8 * c;

    float sh[MR][8], sl[MR][8];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) sh[m][e] = 0.0f, sl[m][e] = 0.0f;

    // One row: its 8 weights (FP16 bits, two per dword) times the split of
    // x[m][k] for every row m of x, into the sums.
    auto add_row = [&](const uint32_t (&d)[4], const float (&xv)[MR]) __attribute__((always_inline)) {
        float wf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) wf[e] = half_bits_to_float((d[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            _Float16 h16, l16;
            split_value(xv[m], h16, l16);
            const float h = (float)h16, l = (float)l16;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sh[m][e] = __builtin_fmaf(h, wf[e], sh[m][e]);
                sl[m][e] = __builtin_fmaf(l, wf[e], sl[m][e]);
            }
        }
    };

    int64_t k = kl;
    if constexpr (FAST) {
        const uintptr_t wa = reinterpret_cast<uintptr_t>(w);
        const int delta = (int)(wa & 3);  // W may start at any even byte
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<void *>(wa - (uintptr_t)delta), 0, (int)(delta + ((K - 1) * ldw + N) * 2), kBufferWord3);
        const int64_t kfast = K - 1;
        const bool col_ok = n < N;
        constexpr int U = MR <= 4 ? kGenericU : kGenericU / 2;
        for (; k < kfast; k += (int64_t)KL * U) {
            uint32_t q[U][5];
            int sft[U];
            float xv[U][MR];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t kk = k + (int64_t)KL * u;
                const bool ok = kk < kfast;
                const int off = ok && col_ok ? (int)(delta + (kk * ldw + n) * 2) : kGenericNoOffset;
                const int a = off & ~3;
                sft[u] = (off & 2) << 3;
                const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, a, 0, 0));
                q[u][0] = v.x;
                q[u][1] = v.y;
                q[u][2] = v.z;
                q[u][3] = v.w;
                q[u][4] = __builtin_amdgcn_raw_buffer_load_b32(rs, a + 16, 0, 0);
                // x is read at a valid row either way (no branch around the
                // loads) and the value dropped past the batches' rows.
                const int64_t kx = ok ? kk : kl;
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    const float v = x[m * ldx + kx];
                    xv[u][m] = ok ? v : 0.0f;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (k + (int64_t)KL * u >= kfast) break;
                const uint32_t d[4] = {__builtin_amdgcn_alignbit(q[u][1], q[u][0], sft[u]),
                                       __builtin_amdgcn_alignbit(q[u][2], q[u][1], sft[u]),
                                       __builtin_amdgcn_alignbit(q[u][3], q[u][2], sft[u]),
                                       __builtin_amdgcn_alignbit(q[u][4], q[u][3], sft[u])};
                add_row(d, xv[u]);
            }
        }
        // The first row of this thread past the batches (row K - 1 or none).
        if (kl < kfast) k = kl + (kfast - kl + KL - 1) / KL * KL;
    }
    for (; k < K; k += KL) {
        const uint4 wv = load_row8<false>(w + k * ldw, n, N);
        const uint32_t d[4] = {wv.x, wv.y, wv.z, wv.w};
        float xv[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) xv[m] = x[m * ldx + k];
        add_row(d, xv);
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
    for (int o = tid; o < MR * kGenericNB; o += kGenericThreads) {
        const int m = o / kGenericNB, col = o % kGenericNB;
        const int64_t gn = n0 + col;
        if (gn >= N) continue;
        float th = 0.0f, tl = 0.0f;
#pragma unroll
        for (int v = 0; v < WAVES; ++v) {
            th += red[v][col >> 3][m][col & 7][0];
            tl += red[v][col >> 3][m][col & 7][1];
        }
        float v = merge_value(th, tl);
        if (bias) v = v + bias[gn];
        if (geglu_rmw) v = gelu_value(y[m * ldy + gn]) * v;  // y held the GEGLU gate
        y[m * ldy + gn] = v;
    }
}

// ---- W given as [N, K] (a torch.nn.Linear weight: each output column's
// weights are one K-contiguous row) ----------------------------------------
//
// Every output column streams its own row of W, so the 1 KiB pieces that
// stream fastest lie along K and no partial sums cross blocks: one dispatch.
// A block (8 waves) owns up to 64 W rows (output columns; 48, 56 or 64 as
// the launcher picks, the stage rows past them load zeros) over all of K
// and walks them in stages of 32 KiB through the four-buffer LDS ring:
// stage s holds rows 32 (s & 1) .. + 31 of the block at k = 512 (s >> 1)
// .. + 511, one whole 1 KiB piece of each row, each piece one LDS-DMA load (streaming
// cache policy: every byte of W is read once).  Row r of a stage keeps its
// granule g at slot 64 r + (g ^ (r % 16)), so the 16 rows an MFMA B fragment
// reads at one granule fall in 16 different bank groups, and a B fragment is
// one ds_read_b128.  Wave w multiplies k-steps 2w and 2w + 1 of every piece:
// its A operands (x split in registers, the hi and lo rows interleaved as
// above) are loaded one piece ahead and serve both row halves.  At the end
// the waves' sums are added in wave order through LDS, and the lane that
// holds both rows of an output merges it (and adds the bias).  Measured at
// 1..8 x 4096 x 14336 with W streamed from HBM and 64-row blocks:
// 23.6-24.6 us (56-row blocks, below: 22.4-22.6 us at M = 1), against
// 27-36 us for 16 waves per 16 columns loading their B fragments straight
// from memory (64-byte pieces of each row per wave instruction); 4 or 16
// waves per block, and walking one row half through all of K before the
// other, were slower.  G = 2 and 4 take up to 16 and 32 rows of x as groups
// of 8, each B fragment feeding every group's MFMAs.  Needs K % 8 == 0 (a 16-byte
// granule is all in or all out), W and x 16-byte aligned with ldw % 8 == 0
// and ldx % 4 == 0.
constexpr int kNkWaves = 8;
constexpr int kNkRows = 64;                       // W rows (output columns) per block
constexpr int kNkPiece = 512;                     // k per row piece (1 KiB)
constexpr int kNkLoads = 32 / kNkWaves;           // row pieces per wave per stage
constexpr int kNkSteps = kNkPiece / 32 / kNkWaves;  // k-steps per wave per piece
constexpr int kNkXLoads = 2 * kNkSteps;           // 16-byte x loads per wave, piece and group
static_assert(kNkRows / 2 * (kNkPiece / 8) == kWSlots, "a stage fills one ring buffer");

__device__ __forceinline__ int nk_slot(int r, int g) { return r * (kNkPiece / 8) + (g ^ (r & 15)); }

// ONE (M = 1, G = 1): each wave brings its 64 values of x per piece into
// LDS with one 4-byte LDS-DMA load per lane (instead of four 16-byte loads
// per lane into registers, seven of every eight lanes of which read rows
// past M), into the slot of the piece's parity, and builds its A operands
// from there.  Measured at M = 1, K = 4096: N = 14336 / 57344 in 22.3 /
// 75.0-75.5 us against 23.1-23.4 / 77.2-78.6 us with the register loads.
__shared__ uint4 g_nkx0[kNkWaves * 16];  // x of even pieces: 64 floats per wave
__shared__ uint4 g_nkx1[kNkWaves * 16];  // x of odd pieces
template <int P>
__device__ __forceinline__ uint4 *nk_xslot()
{
    if constexpr (P == 0) return g_nkx0;
    else return g_nkx1;
}

template <int G, bool ONE = false>
__global__ __launch_bounds__(64 * kNkWaves) void gemv_nk_kernel(const float *__restrict__ x, int64_t ldx,
                                                                const uint16_t *__restrict__ w, int64_t ldw,
                                                                float *__restrict__ y, int64_t ldy,
                                                                const float *__restrict__ bias, int M, int64_t N,
                                                                int64_t K, int rows)
{
    // The block owns W rows n0 .. n0 + rows - 1 (rows <= 64, a multiple of
    // 8); stage rows from `rows` up load zeros and are not written.
    static_assert(!ONE || G == 1, "one row of x is one group");
    constexpr int kXLoadsPerPiece = ONE ? 1 : G * kNkXLoads;  // per wave
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n0 = (int64_t)blockIdx.x * rows;
    const int pieces = (int)((K + kNkPiece - 1) / kNkPiece);
    const int nst = 2 * pieces;

    const __amdgpu_buffer_rsrc_t rs_w =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(w), 0, (int)(N * ldw * 2), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rs_x =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(x), 0, (int)(M * ldx * 4), kBufferWord3);

    // DMA sources: the wave loads stage rows kNkLoads wave + j; lane l fills
    // slot l of the row, i.e. granule l ^ (row % 16) of the piece.
    int w_base[2][kNkLoads], w_k[kNkLoads];
#pragma unroll
    for (int j = 0; j < kNkLoads; ++j) {
        const int r = kNkLoads * wave + j;
        const int gr = lane ^ (r & 15);
        w_k[j] = 8 * gr;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t n = n0 + 32 * h + r;
            w_base[h][j] = 32 * h + r < rows && n < N ? (int)((n * ldw + 8 * gr) * 2) : -1;
        }
    }
    auto issue = [&](auto buf_tag, int s) __attribute__((always_inline)) {
        constexpr int B = decltype(buf_tag)::value;
        uint4 *buf = wring<B>();
        const int p = s >> 1;
#pragma unroll
        for (int j = 0; j < kNkLoads; ++j) {
            const int base = (s & 1) ? w_base[1][j] : w_base[0][j];
            // Bitwise conditions, no short circuit: a branch around a load
            // leaves the compiler unsure how many loads are in flight, and it
            // then waits for all of them.
            const int o = ((s < nst) & (base >= 0) & (kNkPiece * p + w_k[j] < (int)K)) ? base + 2 * kNkPiece * p
                                                                                      : kNoOffset;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_w, (CFP32_LDS void *)(buf + 64 * (kNkLoads * wave + j)), 16,
                                                     o, 0, 0, kStreamAux);
        }
    };

    // A operand: lane l is row i = l % 16 (x row i / 2; hi for even i, lo
    // for odd i) at k = 8 (l / 16) .. + 7 of the k-step.
    const int ai = lane & 15, am = ai >> 1, kq = lane >> 4;
    const bool a_lo = ai & 1;
    int x_base[G];
#pragma unroll
    for (int q = 0; q < G; ++q) x_base[q] = 8 * q + am < M ? (int)(((8 * q + am) * ldx + 8 * kq) * 4) : -1;
    // x of one piece: read into the A operands at the start of an even
    // stage, then overwritten by the next piece's loads.
    floatx4_t xs[G][kNkSteps][2];
    // ONE: lane l of the wave loads x[0][512 p + 64 wave + l] into slot p % 2.
    auto load_x1 = [&](auto slot_tag, int p) __attribute__((always_inline)) {
        const int k = kNkPiece * p + 32 * kNkSteps * wave + lane;
        const int o = ((p < pieces) & (k < (int)K)) ? 4 * k : kNoOffset;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_x, (CFP32_LDS void *)(nk_xslot<decltype(slot_tag)::value>() + 16 * wave),
                                                 4, o, 0, 0, 0);
    };
    auto load_x = [&](int p) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < G; ++q)
#pragma unroll
            for (int t = 0; t < kNkSteps; ++t) {
                const int k = kNkPiece * p + 32 * (kNkSteps * wave + t);
                const bool ok = (x_base[q] >= 0) & (p < pieces) & (k + 8 * kq < (int)K);
                const int o = ok ? x_base[q] + 4 * k : kNoOffset;
                const int o2 = ok ? x_base[q] + 4 * k + 16 : kNoOffset;
                xs[q][t][0] = __builtin_bit_cast(floatx4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_x, o, 0, 0));
                xs[q][t][1] = __builtin_bit_cast(floatx4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_x, o2, 0, 0));
            }
    };
    half8_t af[G][kNkSteps];
    // ONE: lane l wants values 32 t + 8 kq .. + 7 of the wave's 64 (granules
    // 8 t + 2 kq and + 1 of its slot); only x row 0 (i = 0, 1) is live.
    auto build_a1 = [&](auto slot_tag) __attribute__((always_inline)) {
        const uint4 *xb = nk_xslot<decltype(slot_tag)::value>() + 16 * wave;
#pragma unroll
        for (int t = 0; t < kNkSteps; ++t) {
            const floatx4_t v0 = __builtin_bit_cast(floatx4_t, xb[8 * t + 2 * kq]);
            const floatx4_t v1 = __builtin_bit_cast(floatx4_t, xb[8 * t + 2 * kq + 1]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                _Float16 h, l;
                split_value(e < 4 ? v0[e] : v1[e - 4], h, l);
                af[0][t][e] = am == 0 ? (a_lo ? l : h) : (_Float16)0.0f;
            }
        }
    };
    auto build_a = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < G; ++q)
#pragma unroll
            for (int t = 0; t < kNkSteps; ++t)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    _Float16 h, l;
                    split_value(e < 4 ? xs[q][t][0][e] : xs[q][t][1][e - 4], h, l);  // rows past M read 0
                    af[q][t][e] = a_lo ? l : h;
                }
    };

    floatx4_t acc[G][4];  // [group][row half][16-column block]
#pragma unroll
    for (int q = 0; q < G; ++q)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[q][b] = floatx4_t{};

    // One stage: (even stages) form this piece's A operands and load the next
    // piece's x; read the B fragments; refill the buffer read one stage ago
    // with stage s + 3; multiply; then wait until stage s + 1 has landed (and,
    // before an even stage, the x it needs) and the LDS reads are done.  The
    // x loads of piece p + 1 go out in stage 2p, before that stage's W loads,
    // so two stages of W loads and one piece of x may stay in flight there.
    auto stage = [&](auto buf_tag, int s) __attribute__((always_inline)) {
        constexpr int S = decltype(buf_tag)::value;
        const uint4 *buf = wring<S>();
        if constexpr ((S & 1) == 0) {
            if constexpr (ONE) {  // piece s / 2 sits in slot (S / 2) % 2 (s = S mod 4)
                build_a1(std::integral_constant<int, (S >> 1) & 1>{});
                load_x1(std::integral_constant<int, ((S >> 1) + 1) & 1>{}, (s >> 1) + 1);
            } else {
                build_a();
                load_x((s >> 1) + 1);
            }
        }
        half8_t bf[kNkSteps][2];
#pragma unroll
        for (int t = 0; t < kNkSteps; ++t)
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
                bf[t][jb] = __builtin_bit_cast(half8_t, buf[nk_slot(16 * jb + (lane & 15), 4 * (kNkSteps * wave + t) + kq)]);
        __builtin_amdgcn_sched_barrier(0);
        issue(std::integral_constant<int, (S + 3) & 3>{}, s + 3);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < kNkSteps; ++t)
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int q = 0; q < G; ++q)
                    acc[q][2 * (S & 1) + jb] =
                        __builtin_amdgcn_mfma_f32_16x16x32_f16(af[q][t], bf[t][jb], acc[q][2 * (S & 1) + jb], 0, 0, 0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((S & 1) ? 2 * kNkLoads : 2 * kNkLoads + kXLoadsPerPiece));
        block_barrier();
    };

    if constexpr (ONE)
        load_x1(std::integral_constant<int, 0>{}, 0);
    else
        load_x(0);
    issue(std::integral_constant<int, 0>{}, 0);
    issue(std::integral_constant<int, 1>{}, 1);
    issue(std::integral_constant<int, 2>{}, 2);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * kNkLoads));  // x of piece 0 and stage 0 landed
    block_barrier();
    // Whole rounds of four stages, then the last pair (nst is even).  A
    // branch inside the loop body made the compiler wait for every load in
    // flight at the head of each round (one vmcnt(1) per round).
    const int nr = nst / 4 * 4;
    for (int s = 0; s < nr; s += 4) {
        stage(std::integral_constant<int, 0>{}, s);
        stage(std::integral_constant<int, 1>{}, s + 1);
        stage(std::integral_constant<int, 2>{}, s + 2);
        stage(std::integral_constant<int, 3>{}, s + 3);
    }
    if (nr < nst) {
        stage(std::integral_constant<int, 0>{}, nr);
        stage(std::integral_constant<int, 1>{}, nr + 1);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));  // the trailing zero loads, before the ring is reused
    if constexpr (!ONE) {
        // The wait counts above count the x register loads of every even
        // stage.  A load whose value is never read may be deleted by the
        // compiler (the last piece's loads are read by nobody), and then the
        // counts would no longer hold back the W stage a wave reads next;
        // reading the registers here keeps every one of those loads issued,
        // whatever shape the stage loop is given.
#pragma unroll
        for (int q = 0; q < G; ++q)
#pragma unroll
            for (int t = 0; t < kNkSteps; ++t) asm volatile("" ::"v"(xs[q][t][0]), "v"(xs[q][t][1]));
    }
    block_barrier();

    // The waves' sums, [wave][block][lane] in ring buffer q for group q,
    // added in wave order.  16x16 accumulator: rows 4 kq + e, column
    // lane % 16; rows 2m, 2m + 1 are hi, lo of x row 8 q + m.
    static_assert(G <= 4 && kNkWaves * 4 * 64 * 16 <= kWSlots * 16, "each group's sums fit one ring buffer");
    auto red = [&](int q) {
        return reinterpret_cast<floatx4_t *>(q == 0 ? wring<0>() : q == 1 ? wring<1>() : q == 2 ? wring<2>() : wring<3>());
    };
#pragma unroll
    for (int q = 0; q < G; ++q)
#pragma unroll
        for (int b = 0; b < 4; ++b) red(q)[(wave * 4 + b) * 64 + lane] = acc[q][b];
    __syncthreads();
    const int b = (threadIdx.x >> 6) & 3;
    const int64_t n = n0 + 16 * b + (lane & 15);
    const bool own = 16 * b + (lane & 15) < rows && n < N;
    for (int q = threadIdx.x >> 8; q < G; q += 64 * kNkWaves / 256) {
        const floatx4_t *rq = red(q);
        floatx4_t t = rq[b * 64 + lane];
        for (int v = 1; v < kNkWaves; ++v) {
            const floatx4_t u = rq[(v * 4 + b) * 64 + lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] += u[e];
        }
        if (!own) continue;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int m = 8 * q + 2 * kq + h;
            if (m >= M) continue;
            float v = merge_value(t[2 * h], t[2 * h + 1]);
            if (bias) v = v + bias[n];
            y[m * ldy + n] = v;
        }
    }
}

// [N, K] fallback for any alignment and K: a wave per output column, lanes
// striding K, FP32 FMAs, a fixed-order butterfly over the wave.
constexpr int kNkGenericU = 8;  // elements per lane in flight

template <int MR>
__global__ __launch_bounds__(256) void gemv_nk_generic_kernel(const float *__restrict__ x, int64_t ldx,
                                                              const uint16_t *__restrict__ w, int64_t ldw,
                                                              float *__restrict__ y, int64_t ldy,
                                                              const float *__restrict__ bias, int64_t N, int64_t K)
{
    const int lane = threadIdx.x & 63;
    const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= N) return;  // wave-uniform
    float sh[MR], sl[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) sh[m] = 0.0f, sl[m] = 0.0f;
    // Batches of kNkGenericU elements per lane, all loads of a batch issued
    // before any is used (past K a lane reloads its batch's first element and
    // drops it); each lane still adds its elements in increasing k.
    const uint16_t *wr = w + n * ldw;
    for (int64_t k = lane; k < K; k += 64 * kNkGenericU) {
        uint32_t wb[kNkGenericU];
        float xv[kNkGenericU][MR];
#pragma unroll
        for (int u = 0; u < kNkGenericU; ++u) {
            const int64_t kk = k + 64 * u;
            const int64_t kc = kk < K ? kk : k;
            wb[u] = wr[kc];
#pragma unroll
            for (int m = 0; m < MR; ++m) xv[u][m] = x[m * ldx + kc];
        }
        // Every product is formed and a select keeps or drops it: with a
        // branch the compiler moves each load down to its use.
#pragma unroll
        for (int u = 0; u < kNkGenericU; ++u) {
            const bool ok = k + 64 * u < K;
            const float wf = half_bits_to_float(wb[u]);
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                _Float16 h16, l16;
                split_value(xv[u][m], h16, l16);
                const float th = __builtin_fmaf((float)h16, wf, sh[m]);
                const float tl = __builtin_fmaf((float)l16, wf, sl[m]);
                sh[m] = ok ? th : sh[m];
                sl[m] = ok ? tl : sl[m];
            }
        }
    }
#pragma unroll
    for (int sft = 1; sft < 64; sft <<= 1)
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            sh[m] += __shfl_xor(sh[m], sft, 64);
            sl[m] += __shfl_xor(sl[m], sft, 64);
        }
    if (lane == 0) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            float v = merge_value(sh[m], sl[m]);
            if (bias) v = v + bias[n];
            y[m * ldy + n] = v;
        }
    }
}

template <int MR>
hipError_t launch_nk_generic(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy,
                             int64_t N, int64_t K, hipStream_t stream, const float *bias)
{
    const int64_t blocks = (N + 3) / 4;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    gemv_nk_generic_kernel<MR><<<dim3((unsigned)blocks), 256, 0, stream>>>(x, ldx, w, ldw, y, ldy, bias, N, K);
    return hipGetLastError();
}

int64_t tiles_of(int64_t N) { return (N + kTileN - 1) / kTileN; }

// 32-bit buffer offsets must reach every byte of W and x.
bool buffer_path_ok(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, int64_t M, int64_t K)
{
    constexpr int64_t kLimit = kNoOffset - (1 << 20);
    return (ldw % 8 == 0) && ((reinterpret_cast<uintptr_t>(w) & 15) == 0) &&
           ((reinterpret_cast<uintptr_t>(x) & 3) == 0) && (K + 1) * ldw * 2 < kLimit && M * ldx * 4 < kLimit;
}

// W rows at any 2-byte offset (ldw >= 16, 31-bit offsets), up to 8 rows of
// x, K cut into the chunks of gemv_plan: a block (4 waves) owns one
// 512-column tile of one chunk.  Lane l owns columns 8 l .. 8 l + 7 of the
// tile, so one wave instruction reads a 1 KiB piece of one row of W (the
// pattern the chunked kernels stream fastest); wave v takes the chunk's
// rows v, v + 4, v + 8, ... in batches whose loads are all issued before
// any is used (a 16-byte and a 4-byte buffer load from the dword below the
// piece, then funnel shifts by 0 or 16 bits, as in gemv_generic_kernel; row
// K - 1 by load_row8).  The four waves' sums are added in wave order
// through LDS and written as the chunk's partial sums ([chunk][m][hi, lo]
// [n_pad]); the merge dispatch adds the chunks in order and merges.
constexpr int kUcWaves = 4;
constexpr int kUcCols = 512;

template <int MR>
__global__ __launch_bounds__(64 * kUcWaves) void gemv_unaligned_chunk_kernel(
    const float *__restrict__ x, int64_t ldx, const uint16_t *__restrict__ w, int64_t ldw, float *__restrict__ part,
    int64_t n_pad, int64_t N, int64_t K, int64_t chunks, int64_t ntiles)
{
    __shared__ float red[kUcWaves - 1][MR][2][8][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tile = (int64_t)blockIdx.x % ntiles;
    const int64_t chunk = (int64_t)blockIdx.x / ntiles;
    const int64_t n = tile * kUcCols + 8 * lane;
    const int64_t k_begin = chunk * K / chunks, k_end = (chunk + 1) * K / chunks;

    float sh[MR][8], sl[MR][8];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) sh[m][e] = 0.0f, sl[m][e] = 0.0f;
    auto add_row = [&](const uint32_t (&d)[4], const float (&xv)[MR]) __attribute__((always_inline)) {
        float wf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) wf[e] = half_bits_to_float((d[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            _Float16 h16, l16;
            split_value(xv[m], h16, l16);
            const float h = (float)h16, l = (float)l16;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sh[m][e] = __builtin_fmaf(h, wf[e], sh[m][e]);
                sl[m][e] = __builtin_fmaf(l, wf[e], sl[m][e]);
            }
        }
    };

    const uintptr_t wa = reinterpret_cast<uintptr_t>(w);
    const int delta = (int)(wa & 3);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void *>(wa - (uintptr_t)delta), 0, (int)(delta + ((K - 1) * ldw + N) * 2), kBufferWord3);
    const int64_t kf = k_end < K - 1 ? k_end : K - 1;  // rows before kf: batched loads
    const bool col_ok = n < N;
    // Rows per batch: 24 for one row of x (8 KiB of W in flight per wave;
    // 1 x 4096 x 14335: 34 -> 31 us against 8), else as gemv_generic_kernel.
    constexpr int U = MR == 1 ? 3 * kGenericU : MR <= 4 ? kGenericU : kGenericU / 2;
    int64_t k = k_begin + wave;
    for (; k < kf; k += (int64_t)kUcWaves * U) {
        uint32_t q[U][5];
        int sft[U];
        float xv[U][MR];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t kk = k + (int64_t)kUcWaves * u;
            const bool ok = kk < kf;
            const int off = ok && col_ok ? (int)(delta + (kk * ldw + n) * 2) : kGenericNoOffset;
            const int a = off & ~3;
            sft[u] = (off & 2) << 3;
            const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, a, 0, 0));
            q[u][0] = v.x;
            q[u][1] = v.y;
            q[u][2] = v.z;
            q[u][3] = v.w;
            q[u][4] = __builtin_amdgcn_raw_buffer_load_b32(rs, a + 16, 0, 0);
            const int64_t kx = ok ? kk : k;  // a valid row either way; the value is dropped
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const float v = x[m * ldx + kx];
                xv[u][m] = ok ? v : 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (k + (int64_t)kUcWaves * u >= kf) break;
            const uint32_t d[4] = {__builtin_amdgcn_alignbit(q[u][1], q[u][0], sft[u]),
                                   __builtin_amdgcn_alignbit(q[u][2], q[u][1], sft[u]),
                                   __builtin_amdgcn_alignbit(q[u][3], q[u][2], sft[u]),
                                   __builtin_amdgcn_alignbit(q[u][4], q[u][3], sft[u])};
            add_row(d, xv[u]);
        }
    }
    // Row K - 1, in the last chunk, by the wave whose rows reach it.
    const int64_t r0 = k_begin + wave;
    if (r0 < kf) k = r0 + (kf - r0 + kUcWaves - 1) / kUcWaves * kUcWaves;
    else k = r0;
    for (; k < k_end; k += kUcWaves) {
        const uint4 wv = load_row8<false>(w + k * ldw, n, N);
        const uint32_t d[4] = {wv.x, wv.y, wv.z, wv.w};
        float xv[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) xv[m] = x[m * ldx + k];
        add_row(d, xv);
    }

    // Waves 1-3 hand their sums to wave 0, which adds them in wave order.
    if (wave > 0) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                red[wave - 1][m][0][e][lane] = sh[m][e];
                red[wave - 1][m][1][e][lane] = sl[m][e];
            }
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int v = 0; v < kUcWaves - 1; ++v)
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sh[m][e] += red[v][m][0][e][lane];
                sl[m][e] += red[v][m][1][e][lane];
            }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        float *ph = part + ((chunk * MR + m) * 2) * n_pad + n;
        const floatx4_t h0 = {sh[m][0], sh[m][1], sh[m][2], sh[m][3]}, h1 = {sh[m][4], sh[m][5], sh[m][6], sh[m][7]};
        const floatx4_t l0 = {sl[m][0], sl[m][1], sl[m][2], sl[m][3]}, l1 = {sl[m][4], sl[m][5], sl[m][6], sl[m][7]};
        __builtin_nontemporal_store(h0, reinterpret_cast<floatx4_t *>(ph));
        __builtin_nontemporal_store(h1, reinterpret_cast<floatx4_t *>(ph + 4));
        __builtin_nontemporal_store(l0, reinterpret_cast<floatx4_t *>(ph + n_pad));
        __builtin_nontemporal_store(l1, reinterpret_cast<floatx4_t *>(ph + n_pad + 4));
    }
}

// The chunked product (partial sums of plan p in `part`) when p cuts K in
// at least two chunks, W fits the kernel's offsets, and either x has one
// row or gemv_generic_kernel would run fewer than 128 blocks (N <= 8128);
// else hipErrorNotSupported, nothing enqueued.  With more rows of x and
// wider W the vector unit bounds both forms and gemv_generic_kernel's eight
// waves per CU do better (4 x 4096 x 14335: 43 against 48 us; 4 x 14336 x
// 4097: 112 against 59 us with 65 blocks).  The plain projection and the
// GEGLU one take it under the same condition (the GEGLU plan is the plan of
// all 2F columns), so both sum every column the same way.
template <int MR>
hipError_t launch_unaligned_product(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, int64_t N,
                                    int64_t K, const GemvPlan &p, float *part, size_t part_bytes,
                                    hipStream_t stream)
{
    static_assert(kUcCols == kTileN, "the plan's column tiles");
    constexpr int64_t kLimit = kGenericNoOffset - (1 << 20);
    if (p.chunks < 2 || !part || part_bytes < p.workspace_bytes || (reinterpret_cast<uintptr_t>(part) & 15) ||
        K < 1 || ldw < 16 || 2 + 2 * ((K - 1) * ldw + N) >= kLimit)
        return hipErrorNotSupported;
    if (MR > 1 && (N + kGenericNB - 1) / kGenericNB >= 128) return hipErrorNotSupported;
    const int64_t ntiles = tiles_of(N);
    const int64_t blocks = ntiles * p.chunks;
    if (blocks > 0x7FFFFFFF) return hipErrorNotSupported;
    gemv_unaligned_chunk_kernel<MR><<<dim3((unsigned)blocks), 64 * kUcWaves, 0, stream>>>(
        x, ldx, w, ldw, part, p.n_pad, N, K, p.chunks, ntiles);
    return hipGetLastError();
}

hipError_t launch_unaligned_product_m(int64_t M, const float *x, int64_t ldx, const uint16_t *w, int64_t ldw,
                                      int64_t N, int64_t K, const GemvPlan &p, float *part, size_t part_bytes,
                                      hipStream_t stream)
{
    switch (M) {
    case 1: return launch_unaligned_product<1>(x, ldx, w, ldw, N, K, p, part, part_bytes, stream);
    case 2: return launch_unaligned_product<2>(x, ldx, w, ldw, N, K, p, part, part_bytes, stream);
    case 3: return launch_unaligned_product<3>(x, ldx, w, ldw, N, K, p, part, part_bytes, stream);
    case 4: return launch_unaligned_product<4>(x, ldx, w, ldw, N, K, p, part, part_bytes, stream);
    case 5: return launch_unaligned_product<5>(x, ldx, w, ldw, N, K, p, part, part_bytes, stream);
    case 6: return launch_unaligned_product<6>(x, ldx, w, ldw, N, K, p, part, part_bytes, stream);
    case 7: return launch_unaligned_product<7>(x, ldx, w, ldw, N, K, p, part, part_bytes, stream);
    case 8: return launch_unaligned_product<8>(x, ldx, w, ldw, N, K, p, part, part_bytes, stream);
    }
    return hipErrorNotSupported;
}

template <int MR>
hipError_t launch_generic(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy,
                          int64_t N, int64_t K, hipStream_t stream, const float *bias, bool geglu_rmw)
{
    const int64_t blocks = (N + kGenericNB - 1) / kGenericNB;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    // FAST: every byte offset into W (at most 2 + 2 ((K - 1) ldw + N) plus
    // 20) stays below the kernel's zero-read offset.
    constexpr int64_t kLimit = kGenericNoOffset - (1 << 20);
    const bool fast = K >= 1 && ldw >= 16 && 2 + 2 * ((K - 1) * ldw + N) < kLimit;
    if (fast)
        gemv_generic_kernel<MR, true><<<dim3((unsigned)blocks), kGenericThreads, 0, stream>>>(
            x, ldx, w, ldw, y, ldy, N, K, bias, geglu_rmw ? 1 : 0);
    else
        gemv_generic_kernel<MR, false><<<dim3((unsigned)blocks), kGenericThreads, 0, stream>>>(
            x, ldx, w, ldw, y, ldy, N, K, bias, geglu_rmw ? 1 : 0);
    return hipGetLastError();
}

}  // namespace

// About one block per CU over all column tiles; a chunk has at least one
// stage of 32 rows.
hipError_t launch_partial_geglu_merge(const float *part, int64_t n_pad, int64_t chunks, int64_t M, int64_t F,
                                      float *out, int64_t ldo, const float *bias, hipStream_t stream)
{
    const int64_t outs = M * F;
    if (M > 0x7FFFFFFF || (outs + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    gemv_geglu_merge_kernel<<<dim3((unsigned)((outs + 255) / 256)), 256, 0, stream>>>(part, n_pad, chunks, (int)M, F,
                                                                                       out, ldo, bias);
    return hipGetLastError();
}

hipError_t launch_partial_merge(const float *part, int64_t n_pad, int64_t chunks, int64_t M, int64_t N, float *y,
                                int64_t ldy, const float *bias, hipStream_t stream)
{
    const auto al16 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    // Blocks of 64 threads while 256 would leave most CUs without one, and
    // one output per thread up to 256 such blocks (1 x 4096 x 4096 decode:
    // 16.8 -> 13.1 us; 1 x 4096 x 14336: 22.9 -> 22.1 us).  Every output is
    // summed the same way in each form: the same bits.
    const int64_t outs = M * N;
    if (M <= 0x7FFFFFFF && outs <= 256 * 64) {
        gemv_merge_kernel<64><<<dim3((unsigned)((outs + 63) / 64)), 64, 0, stream>>>(part, n_pad, chunks, (int)M, N,
                                                                                     y, ldy, bias);
        return hipGetLastError();
    }
    if (n_pad % 4 == 0 && al16(part)) {
        const int64_t threads = M * ((N + 3) / 4);
        if (M > 0x7FFFFFFF || (threads + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        const bool vy = ldy % 4 == 0 && al16(y);
        if (threads < 256 * 256) {
            const dim3 grid((unsigned)((threads + 63) / 64));
            if (vy)
                gemv_merge4_kernel<true, 64><<<grid, 64, 0, stream>>>(part, n_pad, chunks, (int)M, N, y, ldy, bias);
            else
                gemv_merge4_kernel<false, 64><<<grid, 64, 0, stream>>>(part, n_pad, chunks, (int)M, N, y, ldy, bias);
        } else {
            const dim3 grid((unsigned)((threads + 255) / 256));
            if (vy)
                gemv_merge4_kernel<true, 256><<<grid, 256, 0, stream>>>(part, n_pad, chunks, (int)M, N, y, ldy, bias);
            else
                gemv_merge4_kernel<false, 256><<<grid, 256, 0, stream>>>(part, n_pad, chunks, (int)M, N, y, ldy, bias);
        }
        return hipGetLastError();
    }
    if (M > 0x7FFFFFFF || (outs + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    gemv_merge_kernel<256><<<dim3((unsigned)((outs + 255) / 256)), 256, 0, stream>>>(part, n_pad, chunks, (int)M, N,
                                                                                      y, ldy, bias);
    return hipGetLastError();
}


hipError_t launch_gemv(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy,
                       int64_t M, int64_t N, int64_t K, float *part, size_t part_bytes, hipStream_t stream,
                       const float *bias, bool geglu_rmw)
{
    if (M < 1 || M > kGemvMaxRowsKN || (geglu_rmw && M > kGemvMaxRows)) return hipErrorInvalidValue;
    const GemvPlan p = gemv_plan(M, N, K);
    if (!geglu_rmw && p.chunks > 0 && buffer_path_ok(x, ldx, w, ldw, M, K) &&
        (p.workspace_bytes == 0 || (part && part_bytes >= p.workspace_bytes))) {
        const int64_t blocks = tiles_of(N) * p.chunks;
        if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        GemvArgs g{x, ldx, w, ldw, part, y, ldy, p.n_pad, M, N, K, p.stages, p.chunks, tiles_of(N), bias, 0};
        hipError_t e = launch_product(g, blocks, stream);
        if (e != hipSuccess || p.chunks == 1) return e;
        return launch_partial_merge(part, p.n_pad, p.chunks, M, N, y, ldy, bias, stream);
    }
    if (M > kGemvMaxRows) return hipErrorNotSupported;  // the GEMM path takes it
    if (!geglu_rmw) {
        // W rows that do not allow 16-byte loads, K cut into chunks: the
        // chunked product and the merge dispatch (1 x 4096 x 14335: 35 -> 24
        // us), else one launch of gemv_generic_kernel below.
        const hipError_t e = launch_unaligned_product_m(M, x, ldx, w, ldw, N, K, p, part, part_bytes, stream);
        if (e != hipErrorNotSupported) {
            if (e != hipSuccess) return e;
            return launch_partial_merge(part, p.n_pad, p.chunks, M, N, y, ldy, bias, stream);
        }
    }
    switch (M) {
    case 1: return launch_generic<1>(x, ldx, w, ldw, y, ldy, N, K, stream, bias, geglu_rmw);
    case 2: return launch_generic<2>(x, ldx, w, ldw, y, ldy, N, K, stream, bias, geglu_rmw);
    case 3: return launch_generic<3>(x, ldx, w, ldw, y, ldy, N, K, stream, bias, geglu_rmw);
    case 4: return launch_generic<4>(x, ldx, w, ldw, y, ldy, N, K, stream, bias, geglu_rmw);
    case 5: return launch_generic<5>(x, ldx, w, ldw, y, ldy, N, K, stream, bias, geglu_rmw);
    case 6: return launch_generic<6>(x, ldx, w, ldw, y, ldy, N, K, stream, bias, geglu_rmw);
    case 7: return launch_generic<7>(x, ldx, w, ldw, y, ldy, N, K, stream, bias, geglu_rmw);
    default: return launch_generic<8>(x, ldx, w, ldw, y, ldy, N, K, stream, bias, geglu_rmw);
    }
}

// GEGLU for 1 <= M <= 16: the product dispatch over all 2F columns of W
// [K, 2F] (partial sums always, even for a single chunk), then the GEGLU
// merge.  hipErrorNotSupported (nothing enqueued) when W does not allow the
// buffer path or `part` is missing or too small.

hipError_t launch_gemv_geglu(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *out, int64_t ldo,
                             int64_t M, int64_t F, int64_t K, float *part, size_t part_bytes, hipStream_t stream,
                             const float *bias)
{
    if (M < 1 || M > kGemvMaxRowsKN) return hipErrorInvalidValue;
    const GemvPlan p = gemv_geglu_plan(M, F, K);
    const int64_t N = 2 * F;
    if (p.chunks == 0 || !part || part_bytes < p.workspace_bytes || (M * F + 255) / 256 > 0x7FFFFFFF)
        return hipErrorNotSupported;
    hipError_t e;
    if (buffer_path_ok(x, ldx, w, ldw, M, K)) {
        const int64_t blocks = tiles_of(N) * p.chunks;
        if (blocks > 0x7FFFFFFF) return hipErrorNotSupported;
        GemvArgs g{x, ldx, w, ldw, part, nullptr, 0, p.n_pad, M, N, K, p.stages, p.chunks, tiles_of(N), nullptr, 1};
        e = launch_product(g, blocks, stream);
    } else {
        // W rows that do not allow 16-byte loads: the chunked product where
        // the plain projection takes it (up to 8 rows), else the caller's
        // two-pass fallback.
        if (M > kGemvMaxRows) return hipErrorNotSupported;
        e = launch_unaligned_product_m(M, x, ldx, w, ldw, N, K, p, part, part_bytes, stream);
        if (e == hipErrorNotSupported) return e;
    }
    if (e != hipSuccess) return e;
    gemv_geglu_merge_kernel<<<dim3((unsigned)((M * F + 255) / 256)), 256, 0, stream>>>(part, p.n_pad, p.chunks,
                                                                                        (int)M, F, out, ldo, bias);
    return hipGetLastError();
}

hipError_t launch_gemv_nk(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy,
                          int64_t M, int64_t N, int64_t K, hipStream_t stream, const float *bias)
{
    if (M < 1 || M > kGemvMaxRowsNK) return hipErrorInvalidValue;
    constexpr int64_t kLimit = kNoOffset - (1 << 20);
    const bool fast = K > 0 && K % 8 == 0 && ldw % 8 == 0 && ldx % 4 == 0 &&
                      ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(x)) & 15) == 0 &&
                      N * ldw * 2 < kLimit && M * ldx * 4 < kLimit && K < kLimit / 64;
    if (fast) {
        // 64, 56 or 48 rows per block, whichever leaves the fewest rows to
        // the busiest CU (ties: more rows).  A block streams at a rate of
        // its own, so the rows a CU must stream set the time: measured with
        // M = 1, K = 4096, N = 4096 / 12288 / 14336 / 57344 take 14.7 / 19.5
        // / 22.5 / 76.6 us (48, 48, 56, 56 rows) against 16.0 / 21.9 / 23.4
        // / 84.4 us with 64.  Each output's k order is the same either way.
        int rows = kNkRows;
        int64_t busiest = INT64_MAX;
        for (int r = kNkRows; r >= 48; r -= 8) {
            const int64_t per_cu = ((N + r - 1) / r + kTargetBlocks - 1) / kTargetBlocks * r;
            if (per_cu < busiest) {
                busiest = per_cu;
                rows = r;
            }
        }
        const int64_t blocks = (N + rows - 1) / rows;
        if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        if (M == 1)
            gemv_nk_kernel<1, true><<<dim3((unsigned)blocks), 64 * kNkWaves, 0, stream>>>(x, ldx, w, ldw, y, ldy,
                                                                                         bias, 1, N, K, rows);
        else if (M <= kGemvMaxRows)
            gemv_nk_kernel<1><<<dim3((unsigned)blocks), 64 * kNkWaves, 0, stream>>>(x, ldx, w, ldw, y, ldy, bias,
                                                                                   (int)M, N, K, rows);
        else if (M <= 2 * kGemvMaxRows)
            gemv_nk_kernel<2><<<dim3((unsigned)blocks), 64 * kNkWaves, 0, stream>>>(x, ldx, w, ldw, y, ldy, bias,
                                                                                   (int)M, N, K, rows);
        else
            gemv_nk_kernel<4><<<dim3((unsigned)blocks), 64 * kNkWaves, 0, stream>>>(x, ldx, w, ldw, y, ldy, bias,
                                                                                   (int)M, N, K, rows);
        return hipGetLastError();
    }
    if (M > kGemvMaxRows) return hipErrorNotSupported;  // the GEMM path takes it
    switch (M) {
    case 1: return launch_nk_generic<1>(x, ldx, w, ldw, y, ldy, N, K, stream, bias);
    case 2: return launch_nk_generic<2>(x, ldx, w, ldw, y, ldy, N, K, stream, bias);
    case 3: return launch_nk_generic<3>(x, ldx, w, ldw, y, ldy, N, K, stream, bias);
    case 4: return launch_nk_generic<4>(x, ldx, w, ldw, y, ldy, N, K, stream, bias);
    case 5: return launch_nk_generic<5>(x, ldx, w, ldw, y, ldy, N, K, stream, bias);
    case 6: return launch_nk_generic<6>(x, ldx, w, ldw, y, ldy, N, K, stream, bias);
    case 7: return launch_nk_generic<7>(x, ldx, w, ldw, y, ldy, N, K, stream, bias);
    default: return launch_nk_generic<8>(x, ldx, w, ldw, y, ldy, N, K, stream, bias);
    }
}

}  // namespace cfp32
