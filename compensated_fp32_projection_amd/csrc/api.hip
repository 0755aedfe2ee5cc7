// C ABI of libcfp32 (declared in include/cfp32.h): argument validation,
// the per-device architecture check, workspace layout and path selection.
// Every call validates all of its arguments before it enqueues anything.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "../../include/cfp32.h"
#include "launchers.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
// 0 = not checked yet, 1 = gfx950, 2 = something else.
std::atomic<int> g_arch_state[kMaxDevices];

// Every dimension, and every rows x ld extent, stays below 2^48 elements
// (far above any device memory): size products formed on the host and in
// the launchers, such as (M + tile rows) * ld * 4 or chunks * M * N * 8,
// then cannot overflow 64 bits.
constexpr int64_t kMaxDim = ((int64_t)1 << 48) - 1;

cfp32_status hip_fail(hipError_t e)
{
    g_last_hip_error = (int)e;
    return CFP32_ERR_HIP;
}

// The current device must be gfx950.  The answer is cached per device.
cfp32_status check_device()
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return CFP32_ERR_UNSUPPORTED_DEVICE;
    }
    if (dev < 0 || dev >= kMaxDevices) return CFP32_ERR_UNSUPPORTED_DEVICE;
    int state = g_arch_state[dev].load(std::memory_order_acquire);
    if (state == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) {
            g_last_hip_error = (int)e;
            return CFP32_ERR_UNSUPPORTED_DEVICE;
        }
        state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_arch_state[dev].store(state, std::memory_order_release);
    }
    return state == 1 ? CFP32_OK : CFP32_ERR_UNSUPPORTED_DEVICE;
}

bool dims_ok(int64_t a, int64_t b) { return a >= 0 && b >= 0 && a <= kMaxDim && b <= kMaxDim; }

// rows x ld elements within the 2^48-element limit.
bool extent_ok(int64_t rows, int64_t ld) { return rows == 0 || ld <= kMaxDim / rows; }

cfp32_status launched(hipError_t e) { return e == hipSuccess ? CFP32_OK : hip_fail(e); }

constexpr size_t kAlign = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace layout, from the caller's pointer rounded up to 256 bytes.
// GEMM path (M > 8): the hi plane, then the lo plane, each [M, ldh] FP16
// with ldh = K rounded up to 8 (16-byte rows), each starting on a 256-byte
// boundary, then the split-K partial sums when K is split.
// Small-M path (M <= 8, and M <= 16 with [K, N] weights): the FP32
// per-chunk partial sums (GemvPlan) from the start.  For 8 < M <= 16 the
// size covers both, since the small-M dispatch may decline the operands.
// [K, N] weights with N not a multiple of 8 and M > 8: after those, a
// padded copy of W, [K, N rounded up to 8] FP16 (see linear_paths).
int64_t split_ld(int64_t K) { return (K + 7) / 8 * 8; }

size_t plane_bytes(int64_t M, int64_t K) { return round_up((size_t)M * (size_t)split_ld(K) * 2u, kAlign); }

// Bytes from the aligned base to the padded W copy: the larger of the GEMM
// path's planes and partial sums and the small-M path's partial sums.
// M > kGemvMaxRows, K > 0, extent_ok(M, split_ld(K)).
size_t gemm_region_bytes(int64_t M, int64_t N, int64_t K, bool w_kn)
{
    const cfp32::GemmSplitPlan sp = cfp32::gemm_split_plan(M, N, K);
    const size_t gemm_path = 2 * plane_bytes(M, K) + (sp.chunks > 1 ? round_up(sp.workspace_bytes, kAlign) : 0);
    // [K, N] with 8 < M <= 16 takes the small-M dispatches when W allows
    // 16-byte loads, else the GEMM path: room for either.
    const size_t small_m =
        (w_kn && M <= cfp32::kGemvMaxRowsKN) ? round_up(cfp32::gemv_plan(M, N, K).workspace_bytes, kAlign) : 0;
    return gemm_path > small_m ? gemm_path : small_m;
}

// Whether the projection takes the small-grid kernel (gemm_ksplit.hip) when
// its operands allow it; M > kGemvMaxRows, K > 0.  Its grid must fit the
// GPU at once (two blocks per CU: at most 512 blocks).
//  * [K, N] weights, up to 16 rows: where the small-M dispatches would run
//    a grid of fewer than 64 blocks and K <= 1024 (at most 8 stages per
//    wave).  16 x 256 x 384: 11.5 -> 7.2 us; 12 x 256 x 2048: 11.5 -> 7.3
//    us; 16 x 1024 x 1024: 13.9 -> 10.2 us; with K = 4096 (32 stages per
//    wave) it lost (16 x 4096 x 1024: 16.4 -> 20.5 us).
//  * [N, K] weights up to 32 rows: never (the small-M [N, K] dispatch).
//  * Above: where K is not split across blocks and the generic kernel's
//    32 x 128 tiles would number fewer than 128 (half the CUs); from there
//    that one-launch form is faster (256 x 4096 x 4096: 46 -> 35 us; 200 x
//    1024 x 4096: 19 -> 13 us; 1024^3: 20 -> 13.4 us; 512 x 1024 x 1024:
//    13.6 -> 12.3 us), below it this kernel (96 x 4096 x 4096: 26.6 against
//    33.2 us; 128 x 2048 x 2048: 17.6 against 19.1 us; 333 x 1000 x 784:
//    12.7 against 14.5 us).  Beyond 512 blocks its 32 x 64 tiles re-read x
//    and W more than the large tiles do.
bool ksplit_route(int64_t M, int64_t N, int64_t K, bool nk)
{
    if (cfp32::ksplit_blocks(M, N) > cfp32::kKsplitMaxBlocks) return false;
    if (nk && M <= cfp32::kGemvMaxRowsNK) return false;
    if (!nk && M <= cfp32::kGemvMaxRowsKN) {
        const cfp32::GemvPlan p = cfp32::gemv_plan(M, N, K);
        return K <= 1024 && p.chunks * ((N + cfp32::kGemvTileN - 1) / cfp32::kGemvTileN) < 64;
    }
    const int64_t small_tiles = ((M + 31) / 32) * ((N + 127) / 128);  // the generic kernel's 32 x 128 tiles
    return small_tiles < 128 && cfp32::gemm_split_plan(M, N, K).chunks <= 1;
}

// GEGLU (M > kGemvMaxRows): as cfp32_linear_ex over the [K, 2F] weight, the
// GEMM path (planes, plus split-K partial sums on small grids), or up to 16
// rows the small-M dispatches when W allows 16-byte loads; then, for F % 8
// != 0, a padded copy of W for the small-grid kernel: gate columns at 0, up
// columns at F rounded up to 8, [K, 2 F8] FP16.
size_t geglu_region_bytes(int64_t M, int64_t F, int64_t K)
{
    const cfp32::GemmSplitPlan sp = cfp32::gemm_split_plan(M, 2 * F, K);
    const size_t gemm_path = 2 * plane_bytes(M, K) + (sp.chunks > 1 ? round_up(sp.workspace_bytes, kAlign) : 0);
    const size_t small_m =
        M <= cfp32::kGemvMaxRowsKN ? round_up(cfp32::gemv_geglu_plan(M, F, K).workspace_bytes, kAlign) : 0;
    return gemm_path > small_m ? gemm_path : small_m;
}

size_t geglu_padded_w_bytes(int64_t F, int64_t K) { return round_up((size_t)K * (size_t)split_ld(F) * 4u, kAlign); }

bool pads_w(int64_t M, int64_t N, int64_t K, bool w_kn) { return w_kn && M > cfp32::kGemvMaxRows && K > 0 && N % 8; }

size_t padded_w_bytes(int64_t N, int64_t K) { return round_up((size_t)K * (size_t)split_ld(N) * 2u, kAlign); }

cfp32_status linear_paths(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, bool nk, const float *bias,
                          float *y, int64_t ldy, int64_t M, int64_t N, int64_t K, uintptr_t base, size_t need,
                          hipStream_t s);

}  // namespace

extern "C" {

const char *cfp32_status_string(int status)
{
    // An int, not the enum: C callers may pass any value, and an out-of-range
    // value of an enum type is not a valid C++ enum value.
    switch (status) {
    case CFP32_OK: return "success";
    case CFP32_ERR_INVALID_VALUE: return "invalid argument (null pointer, negative size, leading dimension or workspace too small)";
    case CFP32_ERR_UNSUPPORTED_DEVICE: return "no usable device: the current HIP device is not gfx950 (there is no CPU fallback)";
    case CFP32_ERR_HIP: return "HIP runtime error (see cfp32_last_hip_error)";
    case CFP32_ERR_TOO_LARGE:
        return "problem too large for the no-allocation entry point (its fixed scratch holds 64 MiB per device)";
    }
    return "unknown status";
}

int cfp32_last_hip_error(void) { return g_last_hip_error; }

cfp32_status cfp32_split(const float *x, int64_t ldx, uint16_t *hi, uint16_t *lo, int64_t ldh,
                         int64_t rows, int64_t cols, void *stream)
{
    if (!dims_ok(rows, cols)) return CFP32_ERR_INVALID_VALUE;
    if (rows == 0 || cols == 0) return CFP32_OK;
    if (!x || !hi || !lo || ldx < cols || ldh < cols) return CFP32_ERR_INVALID_VALUE;
    if (!extent_ok(rows, ldx) || !extent_ok(rows, ldh)) return CFP32_ERR_INVALID_VALUE;
    cfp32_status st = check_device();
    if (st != CFP32_OK) return st;
    return launched(cfp32::launch_split(x, ldx, hi, lo, ldh, rows, cols, cols, (hipStream_t)stream));
}

cfp32_status cfp32_merge(const float *c_hi, const float *c_lo, int64_t ldc, float *y, int64_t ldy,
                         int64_t M, int64_t N, void *stream)
{
    if (!dims_ok(M, N)) return CFP32_ERR_INVALID_VALUE;
    if (M == 0 || N == 0) return CFP32_OK;
    if (!c_hi || !c_lo || !y || ldc < N || ldy < N) return CFP32_ERR_INVALID_VALUE;
    if (!extent_ok(M, ldc) || !extent_ok(M, ldy)) return CFP32_ERR_INVALID_VALUE;
    cfp32_status st = check_device();
    if (st != CFP32_OK) return st;
    return launched(cfp32::launch_merge(c_hi, c_lo, ldc, y, ldy, M, N, (hipStream_t)stream));
}

cfp32_status cfp32_gemm(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w,
                        int64_t ldw, float *y, float *c_hi, float *c_lo, int64_t ldc, int64_t M,
                        int64_t N, int64_t K, void *stream)
{
    if (!dims_ok(M, N) || !dims_ok(K, 0)) return CFP32_ERR_INVALID_VALUE;
    if (M == 0 || N == 0) return CFP32_OK;
    if ((c_hi == nullptr) != (c_lo == nullptr)) return CFP32_ERR_INVALID_VALUE;
    if (!y && !c_hi) return CFP32_ERR_INVALID_VALUE;
    if (ldc < N || !extent_ok(M, ldc)) return CFP32_ERR_INVALID_VALUE;
    if (K > 0) {
        if (!a_hi || !a_lo || !w || lda < K || ldw < N) return CFP32_ERR_INVALID_VALUE;
        if (!extent_ok(M, lda) || !extent_ok(K, ldw)) return CFP32_ERR_INVALID_VALUE;
    }
    cfp32_status st = check_device();
    if (st != CFP32_OK) return st;
    return launched(cfp32::launch_gemm(a_hi, a_lo, lda, w, ldw, y, ldc, c_hi, c_lo, ldc, M, N, K,
                                       /*a_zero_padded=*/false, (hipStream_t)stream));
}

cfp32_status cfp32_gemm_separate_add(const uint16_t *a_hi, const uint16_t *a_lo, int64_t lda, const uint16_t *w,
                                     int64_t ldw, float *y, float *c_hi, float *c_lo, int64_t ldc, int64_t M,
                                     int64_t N, int64_t K, int64_t k_per_add, void *stream)
{
    if (!dims_ok(M, N) || !dims_ok(K, 0)) return CFP32_ERR_INVALID_VALUE;
    if (k_per_add != 0 && k_per_add != 16 && k_per_add != 64 && k_per_add != 256) return CFP32_ERR_INVALID_VALUE;
    if (M == 0 || N == 0) return CFP32_OK;
    if ((c_hi == nullptr) != (c_lo == nullptr)) return CFP32_ERR_INVALID_VALUE;
    if (!y && !c_hi) return CFP32_ERR_INVALID_VALUE;
    if (ldc < N || !extent_ok(M, ldc)) return CFP32_ERR_INVALID_VALUE;
    if (K > 0) {
        if (!a_hi || !a_lo || !w || lda < K || ldw < N) return CFP32_ERR_INVALID_VALUE;
        if (!extent_ok(M, lda) || !extent_ok(K, ldw)) return CFP32_ERR_INVALID_VALUE;
    }
    cfp32_status st = check_device();
    if (st != CFP32_OK) return st;
    return launched(cfp32::launch_gemm_separate_add(a_hi, a_lo, lda, w, ldw, y, ldc, c_hi, c_lo, ldc, M, N, K,
                                                    (int)(k_per_add / 16), (hipStream_t)stream));
}

size_t cfp32_linear_ex_workspace_bytes(int64_t M, int64_t N, int64_t K, int w_layout)
{
    if (w_layout != CFP32_W_KN && w_layout != CFP32_W_NK) return 0;
    if (!dims_ok(M, N) || !dims_ok(K, 0)) return 0;
    if (M == 0 || N == 0 || K == 0) return 0;
    // + kAlign: slack to realign the caller's pointer.
    if (M <= cfp32::kGemvMaxRows) {
        if (w_layout == CFP32_W_NK) return 0;  // one dispatch, no partial sums
        const size_t b = cfp32::gemv_plan(M, N, K).workspace_bytes;
        return b == 0 ? 0 : b + kAlign;
    }
    if (!extent_ok(M, split_ld(K))) return 0;
    const bool w_kn = w_layout == CFP32_W_KN;
    if (pads_w(M, N, K, w_kn) && !extent_ok(K, split_ld(N))) return 0;
    const size_t region = gemm_region_bytes(M, N, K, w_kn);
    return region + (pads_w(M, N, K, w_kn) ? padded_w_bytes(N, K) : 0) + kAlign;
}

size_t cfp32_linear_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    return cfp32_linear_ex_workspace_bytes(M, N, K, CFP32_W_KN);
}

cfp32_status cfp32_linear_ex(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, int w_layout,
                             const float *bias, float *y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                             void *workspace, size_t workspace_bytes, void *stream)
{
    if (w_layout != CFP32_W_KN && w_layout != CFP32_W_NK) return CFP32_ERR_INVALID_VALUE;
    const bool nk = w_layout == CFP32_W_NK;
    if (!dims_ok(M, N) || !dims_ok(K, 0)) return CFP32_ERR_INVALID_VALUE;
    if (M == 0 || N == 0) return CFP32_OK;
    if (!y || ldy < N || !extent_ok(M, ldy)) return CFP32_ERR_INVALID_VALUE;
    if (K > 0) {
        if (!x || !w || ldx < K || ldw < (nk ? K : N)) return CFP32_ERR_INVALID_VALUE;
        if (!extent_ok(M, ldx) || !extent_ok(nk ? N : K, ldw)) return CFP32_ERR_INVALID_VALUE;
    }
    const size_t need = cfp32_linear_ex_workspace_bytes(M, N, K, w_layout);
    // Above 8 rows every path with K > 0 needs a workspace; a size of 0 there
    // means its extents would pass the 2^48-element limit.
    if (need == 0 && M > cfp32::kGemvMaxRows && K > 0) return CFP32_ERR_INVALID_VALUE;
    if (need > 0 && (!workspace || workspace_bytes < need)) return CFP32_ERR_INVALID_VALUE;
    cfp32_status st = check_device();
    if (st != CFP32_OK) return st;
    const uintptr_t base = round_up(reinterpret_cast<uintptr_t>(workspace), kAlign);
    return linear_paths(x, ldx, w, ldw, nk, bias, y, ldy, M, N, K, base, need, (hipStream_t)stream);
}

}  // extern "C"

namespace {

// The projection's paths, after validation, on a workspace at `base`
// (256-byte aligned) holding at least need - kAlign bytes (need as
// cfp32_linear_ex_workspace_bytes gives it, 0 when none is needed).
cfp32_status linear_paths(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, bool nk, const float *bias,
                          float *y, int64_t ldy, int64_t M, int64_t N, int64_t K, uintptr_t base, size_t need,
                          hipStream_t s)
{
    if (M <= cfp32::kGemvMaxRows && nk)
        return launched(cfp32::launch_gemv_nk(x, ldx, w, ldw, y, ldy, M, N, K, s, bias));
    if (M <= cfp32::kGemvMaxRows) {
        // need == 0: K == 0, or K is one chunk and the product kernel merges itself.
        float *part = need > 0 ? reinterpret_cast<float *>(base) : nullptr;
        return launched(cfp32::launch_gemv(x, ldx, w, ldw, y, ldy, M, N, K, part, need > 0 ? need - kAlign : 0, s,
                                           bias));
    }

    if (pads_w(M, N, K, !nk) && !(ldw % 8 == 0 && (reinterpret_cast<uintptr_t>(w) & 15) == 0)) {
        // W rows that do not allow 16-byte loads (N not a multiple of 8): a
        // padded copy of W in the workspace first, one more dispatch that
        // reads and writes W once, so that the small-M dispatches or the
        // matrix-unit GEMM below can take it instead of the element-load
        // kernels (333 x 1000 x 777: 29 us this way, 70 us and more with
        // those).  The same values in the same k order: the same bits.
        uint16_t *wp = reinterpret_cast<uint16_t *>(base + gemm_region_bytes(M, N, K, !nk));
        const int64_t ldp = split_ld(N);
        const hipError_t e = cfp32::launch_pad_rows(w, ldw, wp, ldp, K, N, ldp, s);
        if (e != hipSuccess) return hip_fail(e);
        w = wp;
        ldw = ldp;
    }
    if (K > 0 && ksplit_route(M, N, K, nk)) {
        // The small-grid kernel: one launch, x split in registers, K split
        // across the four waves of each 32 x 64 tile (see ksplit_route); it
        // enqueues nothing and returns hipErrorNotSupported when x or W do
        // not allow its 16-byte loads.
        const hipError_t e = cfp32::launch_gemm_ksplit(x, ldx, w, ldw, y, ldy, M, N, K, s, bias, nk);
        if (e != hipErrorNotSupported) return launched(e);
    }
    if (nk && M <= cfp32::kGemvMaxRowsNK && K > 0) {
        // Up to 32 rows of x with [N, K] weights: the small-M [N, K] dispatch
        // with two or four groups of 8 rows; it enqueues nothing and returns
        // hipErrorNotSupported when W or x do not allow 16-byte loads, and the
        // GEMM path below runs instead.
        const hipError_t e = cfp32::launch_gemv_nk(x, ldx, w, ldw, y, ldy, M, N, K, s, bias);
        if (e != hipErrorNotSupported) return launched(e);
    }
    if (!nk && M <= cfp32::kGemvMaxRowsKN && K > 0) {
        // Up to 16 rows of x: the small-M product and merge dispatches (each W
        // fragment serves two groups of 8 rows, W streams once); they
        // enqueue nothing and return hipErrorNotSupported when W does not
        // allow 16-byte loads, and the GEMM path below runs instead.
        // Their partial sums take the front of the workspace, before any
        // padded copy of W.
        const hipError_t e = cfp32::launch_gemv(x, ldx, w, ldw, y, ldy, M, N, K, reinterpret_cast<float *>(base),
                                                gemm_region_bytes(M, N, K, true), s, bias);
        if (e != hipErrorNotSupported) return launched(e);
    }
    if (K == 0)  // nothing to split: the product of an empty sum is +0
        return launched(cfp32::launch_gemm(nullptr, nullptr, 0, nullptr, 0, y, ldy, nullptr, nullptr, ldy, M,
                                           N, 0, false, s, bias));

    // One launch with the split inside the GEMM (launch_gemm_dma_split: the
    // operands and k order of the two-launch path, so the same bits) for
    // narrow W: N <= 1024 with at least 128 output tiles of 128 x 256.
    // There the separate split pass is large against the GEMM and saving it
    // pays (8192 x 1024 x 768: 38 vs 54 us; 32768 x 4096 x 512: 327 vs
    // 416 us; 16384 x 4096 x 1024: 304 vs 322 us).  From N = 1536 on, the
    // conversion each block repeats per 256 columns lengthens every stage's
    // memory phase more than the pass costs (4096 x 4096 x 1536: 130 vs
    // 121 us; 4096^3: 297 vs 253 us; interleaved runs under sustained load
    // on MI355X).
    if (N <= 1024 && ((M + 127) / 128) * ((N + 255) / 256) >= 128) {
        const hipError_t e = cfp32::launch_gemm_dma_split(x, ldx, w, ldw, y, ldy, M, N, K, s, bias, nk);
        if (e != hipErrorNotSupported) return launched(e);
    }

    // Grids too small for the GPU: K split into chunks (partial sums after the
    // planes in the workspace) and a merge dispatch.  Otherwise, on grids of
    // the generic kernel's 32 x 128 tile, the split happens in its registers
    // (one launch, the bits of the two below).
    const cfp32::GemmSplitPlan sp = cfp32::gemm_split_plan(M, N, K);
    if (sp.chunks <= 1) {
        const hipError_t e = cfp32::launch_gemm_xsplit(x, ldx, w, ldw, y, ldy, M, N, K, s, bias, nk);
        if (e != hipErrorNotSupported) return launched(e);
    }
    uint16_t *hi = reinterpret_cast<uint16_t *>(base);
    uint16_t *lo = reinterpret_cast<uint16_t *>(base + plane_bytes(M, K));
    const int64_t ldh = split_ld(K);
    // The planes are written with zeros in columns [K, ldh), so the GEMM may
    // read whole 16-byte groups past K.
    hipError_t e = cfp32::launch_split(x, ldx, hi, lo, ldh, M, K, ldh, s);
    if (e != hipSuccess) return hip_fail(e);
    if (sp.chunks > 1) {
        float *part = reinterpret_cast<float *>(base + 2 * plane_bytes(M, K));
        e = cfp32::launch_gemm_chunked(hi, lo, ldh, w, ldw, y, ldy, M, N, K, /*a_zero_padded=*/true, s, bias, nk,
                                       part, sp.workspace_bytes);
        if (e != hipErrorNotSupported) return launched(e);
    }
    return launched(cfp32::launch_gemm(hi, lo, ldh, w, ldw, y, ldy, nullptr, nullptr, ldy, M, N, K,
                                       /*a_zero_padded=*/true, s, bias, nk));
}

// ---- scratch of the no-allocation entry point -------------------------------
// One fixed array per device, in device memory that the loader provides with
// this code object; its host-side name is only a stand-in for the symbol, so
// host code uses the address hipGetSymbolAddress reports for the current
// device, looked up on the first call on that device and kept.
constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

cfp32_status scratch_of_current_device(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return CFP32_ERR_UNSUPPORTED_DEVICE;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return CFP32_OK;
}

}  // namespace

extern "C" {

cfp32_status cfp32_linear_noalloc(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y,
                                  int64_t ldy, int64_t M, int64_t N, int64_t K, void *stream)
{
    if (!dims_ok(M, N) || !dims_ok(K, 0)) return CFP32_ERR_INVALID_VALUE;
    if (M == 0 || N == 0) return CFP32_OK;
    if (!y || ldy < N || !extent_ok(M, ldy)) return CFP32_ERR_INVALID_VALUE;
    if (K > 0) {
        if (!x || !w || ldx < K || ldw < N) return CFP32_ERR_INVALID_VALUE;
        if (!extent_ok(M, ldx) || !extent_ok(K, ldw)) return CFP32_ERR_INVALID_VALUE;
    }
    const size_t need = cfp32_linear_ex_workspace_bytes(M, N, K, CFP32_W_KN);
    if (need == 0 && M > cfp32::kGemvMaxRows && K > 0) return CFP32_ERR_INVALID_VALUE;  // as in cfp32_linear_ex
    // Where cfp32_linear does not split K it splits x into planes and runs
    // one GEMM, or splits inside the GEMM; both give the same bits.  When the
    // planes do not fit the scratch, only the second is possible; a split of
    // K needs its partial sums, so without room for them there is no path
    // with cfp32_linear's bits.
    const bool fits = need == 0 || need - kAlign <= kScratchBytes;
    if (!fits && (M <= 64 || cfp32::gemm_split_plan(M, N, K).chunks > 1)) return CFP32_ERR_TOO_LARGE;
    cfp32_status st = check_device();
    if (st != CFP32_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (!fits) {
        const hipError_t e = cfp32::launch_gemm_dma_split(x, ldx, w, ldw, y, ldy, M, N, K, s, nullptr, false);
        return e == hipErrorNotSupported ? CFP32_ERR_TOO_LARGE : launched(e);
    }
    void *scr = nullptr;
    st = scratch_of_current_device(&scr);
    if (st != CFP32_OK) return st;
    return linear_paths(x, ldx, w, ldw, false, nullptr, y, ldy, M, N, K, reinterpret_cast<uintptr_t>(scr), need, s);
}

cfp32_status cfp32_linear(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y,
                          int64_t ldy, int64_t M, int64_t N, int64_t K, void *workspace,
                          size_t workspace_bytes, void *stream)
{
    return cfp32_linear_ex(x, ldx, w, ldw, CFP32_W_KN, nullptr, y, ldy, M, N, K, workspace, workspace_bytes,
                           stream);
}

size_t cfp32_linear_geglu_workspace_bytes(int64_t M, int64_t F, int64_t K)
{
    if (!dims_ok(M, F) || !dims_ok(K, 0) || F > kMaxDim / 2) return 0;
    if (M == 0 || F == 0 || K == 0) return 0;
    if (M <= cfp32::kGemvMaxRows) {
        const size_t b = cfp32::gemv_geglu_plan(M, F, K).workspace_bytes;
        return b == 0 ? 0 : b + kAlign;
    }
    if (!extent_ok(M, split_ld(K))) return 0;
    if (F % 8 && !extent_ok(K, 2 * split_ld(F))) return 0;
    return geglu_region_bytes(M, F, K) + (F % 8 ? geglu_padded_w_bytes(F, K) : 0) + kAlign;
}

cfp32_status cfp32_linear_geglu(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, const float *bias,
                                float *out, int64_t ldo, int64_t M, int64_t F, int64_t K, void *workspace,
                                size_t workspace_bytes, void *stream)
{
    if (!dims_ok(M, F) || !dims_ok(K, 0) || F > kMaxDim / 2) return CFP32_ERR_INVALID_VALUE;
    if (M == 0 || F == 0) return CFP32_OK;
    if (!out || ldo < F || !extent_ok(M, ldo)) return CFP32_ERR_INVALID_VALUE;
    if (K > 0) {
        if (!x || !w || ldx < K || ldw < 2 * F) return CFP32_ERR_INVALID_VALUE;
        if (!extent_ok(M, ldx) || !extent_ok(K, ldw)) return CFP32_ERR_INVALID_VALUE;
    }
    const size_t need = cfp32_linear_geglu_workspace_bytes(M, F, K);
    if (need == 0 && M > cfp32::kGemvMaxRows && K > 0) return CFP32_ERR_INVALID_VALUE;  // as in cfp32_linear_ex
    if (need > 0 && (!workspace || workspace_bytes < need)) return CFP32_ERR_INVALID_VALUE;
    cfp32_status st = check_device();
    if (st != CFP32_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    const uint16_t *w_up = K > 0 ? w + F : nullptr;
    const float *bias_up = bias ? bias + F : nullptr;
    const uintptr_t base = round_up(reinterpret_cast<uintptr_t>(workspace), kAlign);

    if (M <= cfp32::kGemvMaxRows) {
        if (K > 0) {
            const hipError_t e = cfp32::launch_gemv_geglu(x, ldx, w, ldw, out, ldo, M, F, K,
                                                          reinterpret_cast<float *>(base), need - kAlign, s, bias);
            if (e != hipErrorNotSupported) return launched(e);
        }
        // Fallback: the gate projection into out (generic small-M kernel via
        // the read-modify-write switch being off), then the up projection,
        // whose epilogue turns out's gate into gelu(gate) * up.
        hipError_t e = cfp32::launch_gemv(x, ldx, w, ldw, out, ldo, M, F, K, nullptr, 0, s, bias, false);
        if (e != hipSuccess) return hip_fail(e);
        return launched(cfp32::launch_gemv(x, ldx, w_up, ldw, out, ldo, M, F, K, nullptr, 0, s, bias_up, true));
    }

    // Small grids: the small-grid kernel with the GEGLU epilogue exactly where
    // cfp32_linear_ex takes the small-grid kernel for the [K, 2F] projection
    // (W 16-byte loadable, or copied because 2F % 8 != 0), so that every gate
    // and up sum is that projection's.  The kernel needs the up columns
    // 16-byte aligned: for F % 8 != 0 it runs on a copy of W with the up
    // columns moved to F rounded up to 8 (the same values in the same order).
    if (M > cfp32::kGemvMaxRows && K > 0 && ksplit_route(M, 2 * F, K, false)) {
        const bool w16 = ldw % 8 == 0 && (reinterpret_cast<uintptr_t>(w) & 15) == 0;
        // Whether cfp32_linear_ex takes the small-grid kernel: on W itself, or,
        // when 2F % 8 != 0, on its compact copy (rows of 2F rounded up to 8 at
        // a 256-byte aligned address, which `base` stands in for here).
        const bool linear_ksplit =
            w16 ? cfp32::ksplit_supported(x, ldx, w, ldw, M, 2 * F, K, false)
                : (2 * F) % 8 != 0 && cfp32::ksplit_supported(x, ldx, reinterpret_cast<const void *>(base),
                                                              split_ld(2 * F), M, 2 * F, K, false);
        if (linear_ksplit && w16 && F % 8 == 0) {
            const hipError_t e = cfp32::launch_gemm_ksplit_geglu(x, ldx, w, ldw, F, out, ldo, M, F, K, s, bias);
            if (e != hipErrorNotSupported) return launched(e);
        } else if (linear_ksplit) {  // F % 8 != 0: the copy with the up columns at F8
            uint16_t *wp = reinterpret_cast<uint16_t *>(base + geglu_region_bytes(M, F, K));
            const int64_t f8 = split_ld(F);
            hipError_t e = cfp32::launch_pad_rows(w, ldw, wp, 2 * f8, K, F, f8, s);
            if (e != hipSuccess) return hip_fail(e);
            e = cfp32::launch_pad_rows(w + F, ldw, wp + f8, 2 * f8, K, F, f8, s);
            if (e != hipSuccess) return hip_fail(e);
            e = cfp32::launch_gemm_ksplit_geglu(x, ldx, wp, 2 * f8, f8, out, ldo, M, F, K, s, bias);
            if (e != hipErrorNotSupported) return launched(e);
        }
    }

    if (M <= cfp32::kGemvMaxRowsKN && K > 0) {
        // Up to 16 rows: the small-M product dispatch over all 2F columns and
        // the GEGLU merge, when W allows 16-byte loads (else the GEMM path).
        const hipError_t e = cfp32::launch_gemv_geglu(x, ldx, w, ldw, out, ldo, M, F, K,
                                                      reinterpret_cast<float *>(base), need - kAlign, s, bias);
        if (e != hipErrorNotSupported) return launched(e);
    }

    if (K == 0) {
        hipError_t e = cfp32::launch_gemm(nullptr, nullptr, 0, nullptr, 0, out, ldo, nullptr, nullptr, ldo, M, F, 0,
                                          false, s, bias);
        if (e != hipSuccess) return hip_fail(e);
        return launched(cfp32::launch_gemm(nullptr, nullptr, 0, nullptr, 0, out, ldo, nullptr, nullptr, ldo, M, F,
                                           0, false, s, bias_up, false, true));
    }

    uint16_t *hi = reinterpret_cast<uint16_t *>(base);
    uint16_t *lo = reinterpret_cast<uint16_t *>(base + plane_bytes(M, K));
    const int64_t ldh = split_ld(K);
    hipError_t e = cfp32::launch_split(x, ldx, hi, lo, ldh, M, K, ldh, s);
    if (e != hipSuccess) return hip_fail(e);
    // One GEMM with the GEGLU in its epilogue when the grid fills the chip
    // (the rule of the plain GEMM: at least one 128 x 256 W tile per CU).
    if (((M + 127) / 128) * ((F + 127) / 128) >= 256) {
        e = cfp32::launch_gemm_dma_geglu(hi, lo, ldh, w, ldw, out, ldo, M, F, K, /*a_zero_padded=*/true, s, bias);
        if (e != hipErrorNotSupported) return launched(e);
    }
    // Small grids: split K over all 2F columns (the cuts cfp32_linear_ex
    // makes for the [K, 2F] projection) and the GEGLU merge.
    const cfp32::GemmSplitPlan sp = cfp32::gemm_split_plan(M, 2 * F, K);
    if (sp.chunks > 1) {
        float *part = reinterpret_cast<float *>(base + 2 * plane_bytes(M, K));
        e = cfp32::launch_gemm_chunked(hi, lo, ldh, w, ldw, out, ldo, M, 2 * F, K, /*a_zero_padded=*/true, s, bias,
                                       false, part, sp.workspace_bytes, /*geglu=*/true);
        if (e != hipErrorNotSupported) return launched(e);
    }
    e = cfp32::launch_gemm(hi, lo, ldh, w, ldw, out, ldo, nullptr, nullptr, ldo, M, F, K, true, s, bias);
    if (e != hipSuccess) return hip_fail(e);
    return launched(cfp32::launch_gemm(hi, lo, ldh, w_up, ldw, out, ldo, nullptr, nullptr, ldo, M, F, K, true, s,
                                       bias_up, false, true));
}

cfp32_status cfp32_linear_f32(const float *x, int64_t ldx, const uint16_t *w, int64_t ldw, float *y, int64_t ldy,
                              int64_t M, int64_t N, int64_t K, void *stream)
{
    if (!dims_ok(M, N) || !dims_ok(K, 0)) return CFP32_ERR_INVALID_VALUE;
    if (M == 0 || N == 0) return CFP32_OK;
    if (!y || ldy < N || !extent_ok(M, ldy)) return CFP32_ERR_INVALID_VALUE;
    if (K > 0) {
        if (!x || !w || ldx < K || ldw < N) return CFP32_ERR_INVALID_VALUE;
        if (!extent_ok(M, ldx) || !extent_ok(K, ldw)) return CFP32_ERR_INVALID_VALUE;
    }
    cfp32_status st = check_device();
    if (st != CFP32_OK) return st;
    return launched(cfp32::launch_gemm_f32(x, ldx, w, ldw, y, ldy, M, N, K, (hipStream_t)stream));
}

cfp32_status cfp32_qkv_rotary(const float *qkv, int64_t ldq, const int64_t *positions, double theta, float *q,
                              float *k, float *v, int64_t T, int64_t H, int64_t D, void *stream)
{
    if (T < 0 || H < 0 || D < 0 || D % 2 || !(theta > 0.0)) return CFP32_ERR_INVALID_VALUE;
    if (H > kMaxDim / 3 || (H > 0 && D > kMaxDim / (3 * H))) return CFP32_ERR_INVALID_VALUE;
    if (T == 0 || H == 0 || D == 0) return CFP32_OK;
    if (!qkv || !q || !k || !v || ldq < 3 * H * D || !extent_ok(T, ldq) || !extent_ok(T, H * D))
        return CFP32_ERR_INVALID_VALUE;
    cfp32_status st = check_device();
    if (st != CFP32_OK) return st;
    return launched(cfp32::launch_qkv_rotary(qkv, ldq, positions, theta, q, k, v, T, H, D, (hipStream_t)stream));
}

}  // extern "C"
