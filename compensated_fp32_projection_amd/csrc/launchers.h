// Host-side launchers of the gfx950 kernels (internal to libcfp32).
// Arguments are already validated by api.hip; every launcher only enqueues
// kernels on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cfp32 {

// Columns [cols, cols_out) of hi and lo are written as +0 (zero padding for
// the GEMM's 16-byte loads); cols_out == cols for the public split.
hipError_t launch_split(const float *x, int64_t ldx, uint16_t *hi, uint16_t *lo, int64_t ldh,
                        int64_t rows, int64_t cols, int64_t cols_out, hipStream_t stream);

hipError_t launch_merge(const float *c_hi, const float *c_lo, int64_t ldc, float *y, int64_t ldy,
                        int64_t rows, int64_t cols, hipStream_t stream);

// Small-grid projection in one launch (gemm_ksplit.hip): FP32 x split in
// registers, K split across the block's four waves, fixed-order reduction,
// merge (+ bias) into y; W [K, N], or [N, K] with w_nk.  hipErrorNotSupported
// (nothing enqueued) unless K % 8 == 0, ldx % 4 == 0, ldw % 8 == 0, x and w
// 16-byte aligned and the byte offsets fit 31 bits.  ksplit_blocks: its
// grid (one block per 32 x 64 output tile); it runs where that grid fits
// the GPU at once (two blocks per CU: at most kKsplitMaxBlocks).
constexpr int kKsplitTileM = 32, kKsplitTileN = 64;
constexpr int64_t kKsplitMaxBlocks = 512;
hipError_t launch_gemm_ksplit(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy,
                              int64_t M, int64_t N, int64_t K, hipStream_t stream, const float *bias, bool w_nk);
int64_t ksplit_blocks(int64_t M, int64_t N);  // plans.hip
// Whether launch_gemm_ksplit takes these operands (plans.hip).
bool ksplit_supported(const void *x, int64_t ldx, const void *w, int64_t ldw, int64_t M, int64_t N, int64_t K,
                      bool w_nk);
// The same kernel with the GEGLU epilogue: out [M, F] = gelu(x W_gate +
// b_gate) * (x W_up + b_up), W [K, >= up_off + F] with the gate columns at
// 0 and the up columns at up_off (a multiple of 8, >= F), bias [2F] (gate |
// up) or null.  hipErrorNotSupported as launch_gemm_ksplit.
hipError_t launch_gemm_ksplit_geglu(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, int64_t up_off,
                                    float *out, int64_t ldo, int64_t M, int64_t F, int64_t K, hipStream_t stream,
                                    const float *bias);

// W [rows, cols] (ldw, any 2-byte alignment) copied into the first cols_out
// columns of wp [rows, ldp] (ldp and cols_out multiples of 8, wp 16-byte
// aligned), columns [cols, cols_out) written as +0: the form the
// 16-byte-load kernels take.
hipError_t launch_pad_rows(const uint16_t *w, int64_t ldw, uint16_t *wp, int64_t ldp, int64_t rows, int64_t cols,
                           int64_t cols_out, hipStream_t stream);

// y (ldy) and/or c_hi, c_lo (ldc) outputs; any of them may be null.
// bias (FP32 [N], or null): every launcher that writes y adds bias[n] to the
// merged value, as one more FP32 addition (c_hi, c_lo stay the bare products).
// w_nk: W is given as [N, K] (ldw >= K) instead of [K, N] (ldw >= N).
// geglu_rmw (launch_gemm, launch_gemv): y holds the GEGLU gate on entry and
// receives gelu(gate) * (merged value + bias); runs the generic kernels.
// a_zero_padded: A's columns from K to the next multiple of 8 hold +0.
hipError_t launch_gemm(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w,
                       int64_t ldw, float *y, int64_t ldy, float *c_hi, float *c_lo, int64_t ldc,
                       int64_t M, int64_t N, int64_t K, bool a_zero_padded, hipStream_t stream,
                       const float *bias = nullptr, bool w_nk = false, bool geglu_rmw = false);

// Separate-addition accumulation mode: k_steps_per_add is 0 (plain
// accumulation, same tile configuration), 1, 4 or 16 sixteen-deep k-steps per
// separate FP32 addition; hipErrorInvalidValue for anything else.
hipError_t launch_gemm_separate_add(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w,
                                    int64_t ldw, float *y, int64_t ldy, float *c_hi, float *c_lo, int64_t ldc,
                                    int64_t M, int64_t N, int64_t K, int k_steps_per_add, hipStream_t stream);

// LDS-DMA variant for aligned operands (gemm_dma.hip); hipErrorNotSupported
// when the operands do not allow it, in which case nothing was enqueued.
// kchunks > 1: split K as GemmSplitPlan describes and write the unmerged
// per-chunk products to `part` ([kchunks][M][2][n_pad]) instead of y, c_hi,
// c_lo (launch_gemm_chunked adds the merge).
hipError_t launch_gemm_dma(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w,
                           int64_t ldw, float *y, int64_t ldy, float *c_hi, float *c_lo, int64_t ldc,
                           int64_t M, int64_t N, int64_t K, bool a_zero_padded, hipStream_t stream,
                           const float *bias = nullptr, bool w_nk = false, int64_t kchunks = 1,
                           float *part = nullptr, int64_t n_pad = 0);

// Split K on grids too small for the GPU (fewer than 128 output tiles of
// 128 x 256; above 64 rows only where the chunks bring the grid to at least
// 128 blocks, 192 where the small-grid kernel could run it).  K is cut into
// 64-deep units, dealt in order to `chunks` chunks as evenly as possible (at
// least 4 units each; chunks x tiles about 256, a multiple of 8 where one is within
// reach; partial sums at most a quarter of W's bytes up to 64 rows, at most
// W's bytes and 56 MiB above); each chunk's C_hi, C_lo go to FP32
// partial sums ([chunks][M][2][n_pad], workspace_bytes in all) that a merge
// dispatch adds in chunk order, then merges.  chunks == 1 (and no
// workspace) otherwise, or when K % 8 != 0 or K is short.  Depends on M, N,
// K only, so every kernel that takes the plan cuts at the same places and
// gives the same bits.
struct GemmSplitPlan {
    int64_t chunks;
    int64_t n_pad;
    size_t workspace_bytes;
};
GemmSplitPlan gemm_split_plan(int64_t M, int64_t N, int64_t K);

// The split-K GEMM of the plan plus the merge dispatch (y = merge of the
// chunk sums, + bias).  hipErrorNotSupported, with nothing enqueued, when the
// plan has one chunk or `part` is missing or smaller than the plan's
// workspace.  The LDS-DMA kernel when the operands allow it, else the
// generic kernel (same cuts, same bits).  geglu: W is [K, N = 2F] (gate |
// up columns, [K, N] layout only) and y [M, F] receives gelu(gate) * up
// from the GEGLU merge dispatch (bias [2F]).
hipError_t launch_gemm_chunked(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w,
                               int64_t ldw, float *y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                               bool a_zero_padded, hipStream_t stream, const float *bias, bool w_nk, float *part,
                               size_t part_bytes, bool geglu = false);

// Sum of `chunks` partial sums part[c][m][2][n_pad] in chunk order, merged
// into y [M, N] (+ bias) (gemv.hip's merge dispatch); the GEGLU form reads
// gate column n and up column F + n and writes gelu(gate) * up to out [M, F]
// (bias [2F]).
hipError_t launch_partial_merge(const float *part, int64_t n_pad, int64_t chunks, int64_t M, int64_t N, float *y,
                                int64_t ldy, const float *bias, hipStream_t stream);
hipError_t launch_partial_geglu_merge(const float *part, int64_t n_pad, int64_t chunks, int64_t M, int64_t F,
                                      float *out, int64_t ldo, const float *bias, hipStream_t stream);

// LDS-DMA GEMM on FP32 A, split in registers (one launch for the whole
// projection); hipErrorNotSupported, with nothing enqueued, unless K % 4 == 0,
// lda % 4 == 0, ldw % 8 == 0 and A, W are 16-byte aligned.
hipError_t launch_gemm_dma_split(const float *a, int64_t lda, const uint16_t *w, int64_t ldw, float *y,
                                 int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t stream,
                                 const float *bias = nullptr, bool w_nk = false);

// The projection from FP32 x in one launch with the split in registers, for
// the grids the generic kernel runs in its 32 x 128 tile (see gemm.hip);
// the bits of launch_split + launch_gemm.  hipErrorNotSupported, with
// nothing enqueued, for other grids, K == 0, or unless ldx % 4 == 0,
// ldw % 8 == 0, x and W are 16-byte aligned and their byte offsets stay
// below 2^31.
hipError_t launch_gemm_xsplit(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy,
                              int64_t M, int64_t N, int64_t K, hipStream_t stream, const float *bias = nullptr,
                              bool w_nk = false);

// GEGLU-fused GEMM on split planes (see gemm_dma.hip); hipErrorNotSupported,
// with nothing enqueued, when the LDS-DMA conditions do not hold.
hipError_t launch_gemm_dma_geglu(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w,
                                 int64_t ldw, float *out, int64_t ldo, int64_t M, int64_t F, int64_t K,
                                 bool a_zero_padded, hipStream_t stream, const float *bias);

// True-FP32 projection (gemm_f32.hip): y = x W with x in FP32, W widened
// exactly to FP32, FP32 matrix-unit products and sums; any M, N, K >= 0.
hipError_t launch_gemm_f32(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream);

// Q/K/V packing + rotary (qkv_rotary.hip): qkv [T, >= 3HD] (ldq) -> q, k, v
// [H][T][D]; pos (device, T entries) or null for 0 .. T-1; D even.
hipError_t launch_qkv_rotary(const float *qkv, int64_t ldq, const int64_t *pos, double theta, float *q, float *k,
                             float *v, int64_t T, int64_t H, int64_t D, hipStream_t stream);

// Small-M tiling shared by the planner (plans.hip) and the kernels
// (gemv.hip): 512-column tiles (1 KiB of an FP16 row), K in stages of 32
// rows, about one block per CU.
constexpr int kGemvTileN = 512;
constexpr int kGemvStageRows = 32;
constexpr int kGemvTargetBlocks = 256;

constexpr int64_t kGemvMaxRows = 8;
// The small-M dispatches also take 8 < M <= 16 where the operands allow
// 16-byte loads (two groups of 8 rows of x share every W fragment; [K, N]
// weights at M x 4096 x 14336: M = 9 / 16 take 25.7 / 28.0 us against
// 35 / 36 us for split K, while four groups, M = 32, took 42 us against 40).
constexpr int64_t kGemvMaxRowsKN = 16;
// [N, K] weights: up to 32 rows (four groups of 8).
constexpr int64_t kGemvMaxRowsNK = 32;

// Small-M path for W given as [N, K] (ldw >= K): one dispatch, no workspace.
// M <= 8 always; 8 < M <= 32 only with 16-byte loads of W and x, else
// hipErrorNotSupported with nothing enqueued (the GEMM path takes it).
hipError_t launch_gemv_nk(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy,
                          int64_t M, int64_t N, int64_t K, hipStream_t stream, const float *bias = nullptr);

// Small-M (1 <= M <= 16) path: K is cut into `chunks` row chunks of whole
// stages (`stages` = ceil(K / 32) in all); with chunks > 1 the product
// dispatch writes per-chunk FP32 partial sums of C_hi and C_lo
// ([chunks][M][2][n_pad] floats, workspace_bytes in all) that the merge
// dispatch reduces in chunk order; with chunks == 1 it writes y itself and
// needs no workspace.  All fields are 0 when M, N or K is out of range.
struct GemvPlan {
    int64_t chunks;
    int64_t stages;
    int64_t n_pad;
    size_t workspace_bytes;
};
GemvPlan gemv_plan(int64_t M, int64_t N, int64_t K);

// Split + both products + merge for 1 <= M <= 16, K >= 0.  `part` (16-byte
// aligned, part_bytes long) holds the partial sums.  When W does not allow
// 16-byte buffer loads, or `part` is needed but missing or too small, one
// fused generic kernel runs instead for M <= 8 and `part` is not touched;
// for M > 8 nothing is enqueued and hipErrorNotSupported is returned.
// geglu_rmw needs M <= 8.
hipError_t launch_gemv(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y,
                       int64_t ldy, int64_t M, int64_t N, int64_t K, float *part, size_t part_bytes,
                       hipStream_t stream, const float *bias = nullptr, bool geglu_rmw = false);

// GEGLU for 1 <= M <= 16 over W [K, 2F]: out [M, F] = gelu(gate) * up.  The
// plan's workspace holds partial sums for all 2F columns.
GemvPlan gemv_geglu_plan(int64_t M, int64_t F, int64_t K);
hipError_t launch_gemv_geglu(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *out, int64_t ldo,
                             int64_t M, int64_t F, int64_t K, float *part, size_t part_bytes, hipStream_t stream,
                             const float *bias);

}  // namespace cfp32
