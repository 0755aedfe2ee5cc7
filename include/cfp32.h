/*
 * cfp32.h -- C ABI of libcfp32, the compensated-FP32 projection for AMD
 * Instinct MI355X (gfx950).
 *
 * The method (laya.cpp Vulkan backend guide, docs/vulkan.md, compensated-FP32
 * paragraph and the split/merge paragraph that follows it): an FP32
 * projection input x is split into two FP16 parts,
 *
 *     hi = RNE16(x),   lo = RNE16((x - hi) * 1024)
 *
 * (round to nearest even, FP16 subnormals kept; the 1024 scale keeps the
 * residual away from FP16 underflow without overflowing it, per the guide's
 * validation paragraph on large activations), both parts are multiplied by
 * the FP16 weights with FP32 accumulators,
 *
 *     C_hi = A_hi W,   C_lo = A_lo W,
 *
 * and the two products are combined once, in FP32:
 *
 *     y = C_hi + C_lo / 1024.
 *
 * The guide runs the split and the merge as one dispatch each; these calls
 * map onto that: cfp32_split, cfp32_gemm (two products sharing each W tile,
 * merge fused into its epilogue) and cfp32_merge, plus cfp32_linear, which
 * runs the whole projection in one to three dispatches (for M <= 8, and
 * M <= 16 with 16-byte aligned W, the split is done in registers by the
 * product dispatch and a second one reduces the per-chunk partial sums and
 * merges; otherwise the split is a dispatch of its own or, where that is
 * faster, is done by the GEMM as it loads x; small grids split K and add a
 * merge dispatch).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Matrices are row-major; every ld* is a leading dimension in elements
 *   (the distance between consecutive rows) and must be >= the row length.
 * - FP16 data travels as IEEE binary16 bit patterns in uint16_t.
 * - All pointers are device memory owned by the caller.  The library never
 *   allocates, frees, synchronises or prints.  No alignment is required;
 *   kernels use wide loads only where the pointers and ld allow them.  The
 *   one piece of device memory the library owns is the fixed scratch array
 *   of cfp32_linear_noalloc (64 MiB per device, set aside by the loader).
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   Calls are asynchronous and ordered on that stream.  Execution faults
 *   surface at the caller's next synchronisation.
 * - Arguments are validated before anything is enqueued.  A call that
 *   returns an error has enqueued nothing.
 * - Every dimension, and every rows x ld extent of an operand, must be
 *   below 2^48 elements; larger values give CFP32_ERR_INVALID_VALUE.
 * - M == 0 or N == 0 (rows == 0 or cols == 0 for split) is a no-op that
 *   returns CFP32_OK.  K == 0 writes +0 to every output element.
 * - The current HIP device must be gfx950; otherwise
 *   CFP32_ERR_UNSUPPORTED_DEVICE is returned.  There is no CPU fallback
 *   (the guide treats an unavailable backend as an error, never a silent
 *   fallback).
 * - Outputs must not overlap inputs.
 * - The library keeps no mutable state besides a per-device cache of the
 *   architecture check (and cfp32_linear_noalloc's scratch array and the
 *   cache of its address); calls from several threads are safe, except
 *   overlapping cfp32_linear_noalloc calls on one device.
 */
#ifndef CFP32_H
#define CFP32_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define CFP32_API __attribute__((visibility("default")))
#else
#define CFP32_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CFP32_OK = 0,
    CFP32_ERR_INVALID_VALUE = 1,      /* null pointer, negative size, ld too small, workspace too small, size overflow */
    CFP32_ERR_UNSUPPORTED_DEVICE = 2, /* no HIP device, or the current one is not gfx950 */
    CFP32_ERR_HIP = 3,                /* a HIP runtime call or kernel launch failed; see cfp32_last_hip_error */
    CFP32_ERR_TOO_LARGE = 4           /* cfp32_linear_noalloc: the problem needs more than its fixed scratch */
} cfp32_status;

/* Static, NUL-terminated description of a status code (any int: values that
 * are not a cfp32_status give "unknown status"). */
CFP32_API const char *cfp32_status_string(int status);

/* hipError_t value behind the last CFP32_ERR_HIP (or CFP32_ERR_UNSUPPORTED_DEVICE
 * caused by a failing device query) returned on the calling thread; 0 if none. */
CFP32_API int cfp32_last_hip_error(void);

/* Split (guide: split/merge paragraph).
 *   x   : FP32 [rows, cols], leading dimension ldx >= cols.
 *   hi  : FP16 bits [rows, cols], leading dimension ldh >= cols; hi = RNE16(x).
 *   lo  : FP16 bits [rows, cols], same ldh; lo = RNE16((x - hi) * 1024).
 * Bit-exact: FP16 and FP32 subnormals are kept, ties go to even, -0 gives
 * (hi, lo) = (-0, +0).  Out-of-domain inputs follow IEEE: |x| >= 65520 gives
 * hi = +-inf and lo = -+inf; inf or NaN input gives a NaN lo (and hi = x for
 * inf, NaN for NaN).  One kernel launch. */
CFP32_API cfp32_status cfp32_split(const float *x, int64_t ldx, uint16_t *hi, uint16_t *lo, int64_t ldh,
                         int64_t rows, int64_t cols, void *stream);

/* Dual-product GEMM with fused merge (guide: compensated-FP32 paragraph).
 *   a_hi, a_lo : FP16 bits [M, K], leading dimension lda >= K (the split planes).
 *   w          : FP16 bits [K, N], leading dimension ldw >= N (the weights, exact).
 *   y          : FP32 [M, N] or NULL; y = C_hi + C_lo / 1024, merged in FP32.
 *   c_hi, c_lo : FP32 [M, N] or both NULL; the two products before merging.
 *   ldc        : leading dimension (>= N) of every non-NULL output.
 * At least one of y and (c_hi, c_lo) must be given; c_hi and c_lo are given
 * together or not at all.  Both products accumulate in FP32 (FP16 x FP16
 * products are exact in FP32); they are merged once, after both K-reductions,
 * so y equals the FP32 merge of the c_hi, c_lo the same call writes.  The
 * summation order along K is fixed by the kernel, so repeated calls give
 * identical bits.  One kernel launch. */
CFP32_API cfp32_status cfp32_gemm(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda,
                        const uint16_t *w, int64_t ldw,
                        float *y, float *c_hi, float *c_lo, int64_t ldc,
                        int64_t M, int64_t N, int64_t K, void *stream);

/* Dual-product GEMM with the separate-addition accumulation of the guide's
 * AMD path (compensated-FP32 paragraph: cooperative-matrix tile results are
 * added with separate FP32 additions, which reduces the drift of a long dot
 * product kept entirely inside matrix multiply-adds).  Arguments, outputs and
 * errors as cfp32_gemm, plus
 *   k_per_add : 16, 64 or 256 -- the depth of K that the matrix unit
 *               accumulates on its own before that partial tile result is
 *               added to a running FP32 sum with an ordinary vector addition
 *               (16: every MFMA starts from zero); 0 runs the same kernel
 *               configuration with plain accumulation, for comparison.  Any
 *               other value gives CFP32_ERR_INVALID_VALUE.
 * An accuracy mode: one 32 x 128 tile configuration, slower than cfp32_gemm
 * (the cost is measured next to it).  Fixed order, repeatable bits.  One
 * kernel launch. */
CFP32_API cfp32_status cfp32_gemm_separate_add(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda,
                                     const uint16_t *w, int64_t ldw,
                                     float *y, float *c_hi, float *c_lo, int64_t ldc,
                                     int64_t M, int64_t N, int64_t K, int64_t k_per_add, void *stream);

/* Standalone merge (guide: split/merge paragraph; one dispatch).
 *   c_hi, c_lo : FP32 [M, N], leading dimension ldc >= N.
 *   y          : FP32 [M, N], leading dimension ldy >= N.
 * y = fl32(c_hi + fl32(c_lo * 2^-10)), bit-exact, no fused multiply-add. */
CFP32_API cfp32_status cfp32_merge(const float *c_hi, const float *c_lo, int64_t ldc, float *y, int64_t ldy,
                         int64_t M, int64_t N, void *stream);

/* Bytes of device workspace cfp32_linear needs for this shape (0 when none
 * is needed: an empty problem, M, N or K == 0).  Returns 0 for negative
 * sizes.  M <= 8: about chunks * M * N * 8 bytes of FP32 partial sums, with
 * at most 256 chunks (1 MiB for M = 1, N = 14336, K = 4096).
 * M > 8: the FP16 hi and lo planes of x, about 4 * M * K bytes, plus, on
 * small grids, FP32 partial sums of split K (at most a quarter of W's bytes
 * for M <= 64; above, at most W's bytes and 56 MiB); for M <= 16 at least
 * the small-M partial sums.  M > 8
 * with N not a multiple of 8: also a padded copy of W, 2 * K * N8 bytes
 * (N8 = N rounded up to 8).  Returns 0 too when these sizes would pass
 * 2^48 elements; cfp32_linear then refuses the shape. */
CFP32_API size_t cfp32_linear_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* The whole projection y = x W (guide: compensated-FP32 paragraph; small
 * projections run at their real row count, with no padding of M).
 *   x   : FP32 [M, K], leading dimension ldx >= K.
 *   w   : FP16 bits [K, N], leading dimension ldw >= N.
 *   y   : FP32 [M, N], leading dimension ldy >= N.
 *   workspace, workspace_bytes : device scratch of at least
 *         cfp32_linear_workspace_bytes(M, N, K) bytes (may be NULL when that
 *         is 0).  Its contents on entry are ignored; it must not be used by
 *         another call until this call's work on `stream` has completed.
 * M <= 8: a product kernel (split in registers, both products over row
 *         chunks of K, FP32 partial sums into the workspace), then a merge
 *         kernel that sums the chunks in order and merges (two launches).
 *         W that is not 16-byte aligned with ldw % 8 == 0 is read at its
 *         2-byte offsets instead: with one row of x, or N <= 8128, by a
 *         chunked product kernel with the same partial sums and merge;
 *         otherwise (or when K is one chunk, or ldw < 16) by one fused
 *         kernel over all of K that leaves the workspace untouched.
 * 8 < M <= 16 with W 16-byte aligned and ldw % 8 == 0: the same two
 *         launches, two groups of 8 rows of x sharing every W fragment.
 * M  > 8 with N not a multiple of 8 and W rows that do not allow 16-byte
 *         loads: one more launch first copies W into the workspace with
 *         rows of N8 elements (columns past N zero); the paths below then
 *         run on that copy as on a 16-byte-aligned W (the same bits).  The
 *         copy reads and writes W on every call (64 x 4096 x 14335: 93 us
 *         against 45 us for N = 14336); W kept with a leading dimension
 *         that is a multiple of 8 (and 16-byte aligned) needs none, and the
 *         element-load kernels that would avoid it run 2.5-5x slower.
 * M  > 8, small grids (at most 512 output tiles of 32 x 64; above 16 rows
 *         ([K, N]) or 32 rows ([N, K]) where K is not split across blocks
 *         as below; from 9 to 16 rows with [K, N] weights where K <= 1024 and
 *         the small-M dispatches would run fewer than 64 blocks) with
 *         K % 8 == 0, ldx % 4 == 0 and x, W 16-byte loadable: one launch that
 *         splits x in registers and splits K across the four waves of each
 *         tile, the partial tiles summed in a fixed order (its own repeatable
 *         bits; the same for [K, N] and [N, K] weights).
 * M  > 8 otherwise: cfp32_split into the workspace, then cfp32_gemm with
 *         the merged epilogue (two launches); or, for N <= 1024 with at
 *         least 128 output tiles of 128 x 256 and K % 4 == 0, ldx % 4 == 0,
 *         ldw % 8 == 0, x and w 16-byte aligned, one GEMM launch that splits
 *         x on the way into LDS (the workspace is then not touched; both give
 *         identical bits); or, on small grids with K % 8 == 0 (fewer than
 *         128 tiles; above 64 rows only where K is long enough to give each
 *         of at least 128 blocks (192 where the one-launch small-grid
 *         path below could run the grid) four 64-deep units, with the
 *         partial sums
 *         within W's bytes and 56 MiB), the
 *         split, a GEMM over chunks of K writing FP32 partial sums into the
 *         workspace, and a merge dispatch (three launches); or,
 *         on grids the GEMM runs in 32 x 128 tiles (fewer than 128 tiles of
 *         128 x 256, and at most 768 of 32 x 128 or fewer than 256 of
 *         64 x 128) with ldx % 4 == 0,
 *         ldw % 8 == 0 and x, w 16-byte aligned, one GEMM launch that splits
 *         x in registers as it loads it (the workspace is then not touched;
 *         the bits of the two launches).
 * Every path sums in a fixed order: results repeat bit for bit.
 * Results satisfy |y - y_exact| <= 1e-5 * sum_k |x_k w_k| for inputs within
 * the split's domain (|x| < 65520). */
CFP32_API cfp32_status cfp32_linear(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw,
                          float *y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                          void *workspace, size_t workspace_bytes, void *stream);

/* cfp32_linear without a workspace, for callers that cannot allocate device
 * memory: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid allocation.  Arguments, results and errors are those
 * of cfp32_linear (same paths, same kernels, the same bits), except that the
 * scratch the kernels need (hi/lo planes, partial sums) lives in one fixed
 * array of 64 MiB per device that the library owns: device memory set aside
 * when the library's code is loaded on a device and held until the process
 * ends.  This call allocates and frees nothing.
 *   - Problems whose scratch exceeds 64 MiB return CFP32_ERR_TOO_LARGE with
 *     nothing enqueued; above 64 rows, where cfp32_linear does not split K
 *     across blocks, such problems instead run the GEMM that splits x on the
 *     way into LDS and needs no scratch (same bits as cfp32_linear), when x
 *     and W allow it (K % 4 == 0, ldx % 4 == 0, ldw % 8 == 0, 16-byte
 *     aligned), else CFP32_ERR_TOO_LARGE.  cfp32_linear_
 *     workspace_bytes(M, N, K) - 256 is the scratch a shape needs.
 *   - Every call on one device shares that device's array, which keeps the
 *     last call's contents; nothing in it needs to start at zero (each
 *     kernel writes the bytes it reads first).  Calls that may overlap on
 *     one device (different streams without an ordering between them, or
 *     several host threads) race on the array and give wrong results: use
 *     cfp32_linear with a workspace per stream for those.  Calls ordered on
 *     one stream are safe. */
CFP32_API cfp32_status cfp32_linear_noalloc(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw,
                                  float *y, int64_t ldy, int64_t M, int64_t N, int64_t K, void *stream);

/* Weight layouts for cfp32_linear_ex. */
typedef enum {
    CFP32_W_KN = 0, /* w is [K, N], row-major (the layout cfp32_linear takes) */
    CFP32_W_NK = 1  /* w is [N, K], row-major: a torch.nn.Linear weight */
} cfp32_w_layout;

/* Workspace bytes cfp32_linear_ex needs for this shape and weight layout
 * (0 when none is needed; 0 for negative sizes or an unknown layout). */
CFP32_API size_t cfp32_linear_ex_workspace_bytes(int64_t M, int64_t N, int64_t K, int w_layout);

/* The projection with the operations next to it in a model layer (guide:
 * graph paragraph; small projections at their real batch size):
 *   y = x W (+ bias), W in either layout.
 *   x        : FP32 [M, K], leading dimension ldx >= K.
 *   w        : FP16 bits; CFP32_W_KN: [K, N] with ldw >= N;
 *              CFP32_W_NK: [N, K] with ldw >= K.
 *   bias     : FP32 [N] or NULL; added to each merged output as one more
 *              FP32 addition: y = fl32(merge(C_hi, C_lo) + bias[n]).
 *   y        : FP32 [M, N], leading dimension ldy >= N.
 *   workspace, workspace_bytes : as for cfp32_linear, sized by
 *              cfp32_linear_ex_workspace_bytes(M, N, K, w_layout).
 * With CFP32_W_KN and no bias this is exactly cfp32_linear (same kernels,
 * same bits); without the bias, y equals the bias-free call to the bit.
 * CFP32_W_NK, M <= 32: one dispatch with no workspace, each block
 * streaming 64 whole W rows through LDS (M <= 8 always; 8 < M <= 32 when
 * K % 8 == 0, ldw % 8 == 0, ldx % 4 == 0 and w, x are 16-byte aligned,
 * else the GEMM path).  CFP32_W_NK, M > 32: the GEMM paths, with the same
 * bits as CFP32_W_KN.
 * Unknown layouts give CFP32_ERR_INVALID_VALUE. */
CFP32_API cfp32_status cfp32_linear_ex(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, int w_layout,
                             const float *bias, float *y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                             void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes cfp32_linear_geglu needs (0 when none is needed): as
 * cfp32_linear's for the [K, 2F] projection, and for M > 8 with F % 8 != 0
 * also room for a copy of W with rows of 2 F8 elements (F8 = F rounded up
 * to 8). */
CFP32_API size_t cfp32_linear_geglu_workspace_bytes(int64_t M, int64_t F, int64_t K);

/* The feed-forward projection with its GEGLU fused (guide: graph paragraph,
 * the fused GEGLU shader of the FP32 feed-forward layers):
 *   gate = x W[:, :F] (+ bias[:F]),  up = x W[:, F:] (+ bias[F:]),
 *   out  = gelu(gate) * up,  gelu(g) = g * Phi(g) = g/2 (1 + erf(g / sqrt 2)).
 *   x    : FP32 [M, K], ldx >= K.
 *   w    : FP16 bits [K, 2F], ldw >= 2F: gate columns first, then up.
 *   bias : FP32 [2F] or NULL.
 *   out  : FP32 [M, F], ldo >= F.
 *   workspace, workspace_bytes : as for cfp32_linear, sized by
 *          cfp32_linear_geglu_workspace_bytes(M, F, K).
 * gate and up are the projection's merged outputs (the same bits
 * cfp32_linear gives for those columns); the activation and the product run
 * in FP32 in the kernel that merges them (erff and three roundings).
 * M > 8 with at least 256 output tiles of 128 x 128 (and aligned operands):
 * the split, then one GEMM launch with the GEGLU in its epilogue.  M <= 8
 * (M <= 16 with 16-byte aligned W, ldw % 8 == 0): the small-M product
 * dispatch over all 2F columns, then a merge dispatch that forms out.
 * M <= 64 on small grids with K % 8 == 0: the split, a GEMM over chunks of K
 * into FP32 partial sums in the workspace, then that merge dispatch.
 * M > 8 where cfp32_linear_ex takes its one-launch small-grid kernel for
 * the [K, 2F] projection: that kernel with the GEGLU in its epilogue (for
 * F % 8 != 0 after two launches that copy W into the workspace with the up
 * columns at F rounded up to 8).  Other cases run the gate projection into
 * out and the up projection with a read-modify-write epilogue (one more
 * launch). */
CFP32_API cfp32_status cfp32_linear_geglu(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw,
                                const float *bias, float *out, int64_t ldo, int64_t M, int64_t F, int64_t K,
                                void *workspace, size_t workspace_bytes, void *stream);

/* True-FP32 projection (guide: true-FP32 paragraph, the build-time
 * extension's true FP32 matrix kernels, which keep FP32 operands from being
 * converted to FP16): the A/B partner of cfp32_linear on the same operands.
 *   x : FP32 [M, K], ldx >= K, used as FP32 (no split, no FP16 rounding).
 *   w : FP16 bits [K, N], ldw >= N, widened exactly to FP32.
 *   y : FP32 [M, N], ldy >= N.
 * FP32 products and FP32 accumulation on the matrix unit
 * (v_mfma_f32_16x16x4_f32), a fixed summation order (repeatable bits), no
 * workspace, one kernel launch.  Errors and empty problems as cfp32_linear. */
CFP32_API cfp32_status cfp32_linear_f32(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw,
                              float *y, int64_t ldy, int64_t M, int64_t N, int64_t K, void *stream);

/* Q/K/V packing with the rotary multiplication, one dispatch (guide: graph
 * paragraph), applied to a QKV projection's output.
 *   qkv       : FP32 [T, 3*H*D] (ldq >= 3*H*D); row t = [q | k | v], each H
 *               heads of D values, head h at h*D.
 *   positions : int64 [T] device array of token positions, or NULL for
 *               0 .. T-1.
 *   theta     : rotary base (> 0), e.g. 10000.
 *   q, k, v   : FP32 [H, T, D] each, contiguous (head-major).
 *   D         : even.
 * q and k are rotated in the half-split pairing: dims i and i + D/2 turn by
 * pos * theta^(-2i/D), x1' = x1 cos - x2 sin, x2' = x2 cos + x1 sin; v is
 * copied.  FP32 arithmetic (sincosf of the FP32 angle).  One kernel launch. */
CFP32_API cfp32_status cfp32_qkv_rotary(const float *qkv, int64_t ldq, const int64_t *positions, double theta,
                              float *q, float *k, float *v, int64_t T, int64_t H, int64_t D, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CFP32_H */
