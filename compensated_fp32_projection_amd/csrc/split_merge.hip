// Split and merge kernels (laya.cpp Vulkan guide, split/merge paragraph: each
// runs as a single dispatch).  Both are elementwise and bound by HBM
// bandwidth: the split reads 4 bytes and writes 2 + 2 per element, the merge
// reads 8 and writes 4.  Threads of a block cover consecutive columns of one
// row, so every wave reads and writes contiguous runs; rows go to grid.y.
// Every byte is touched once, so the vector paths use non-temporal loads and
// stores (streaming cache policy).
#include "device_common.h"
#include "launchers.h"

namespace cfp32 {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxGridY = 65535;

// VEC: cols, ldx, ldh multiples of 4 and pointers aligned, so each thread
// moves one 16-byte FP32 group and two 8-byte FP16 groups.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void split_kernel(const float *__restrict__ x, int64_t ldx,
                                                         uint16_t *__restrict__ hi,
                                                         uint16_t *__restrict__ lo, int64_t ldh,
                                                         int64_t rows, int64_t cols, int64_t cols_out)
{
    constexpr int kPer = VEC ? 4 : 1;
    const int64_t c = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kPer;
    if (c >= cols_out) return;
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
        if (c >= cols) {  // zero padding (whole group: cols and cols_out are multiples of kPer)
            if constexpr (VEC) {
                __builtin_nontemporal_store(half4_t{}, reinterpret_cast<half4_t *>(hi + r * ldh + c));
                __builtin_nontemporal_store(half4_t{}, reinterpret_cast<half4_t *>(lo + r * ldh + c));
            } else {
                hi[r * ldh + c] = 0;
                lo[r * ldh + c] = 0;
            }
        } else if constexpr (VEC) {
            const floatx4_t v = __builtin_nontemporal_load(reinterpret_cast<const floatx4_t *>(x + r * ldx + c));
            _Float16 h0, h1, h2, h3, l0, l1, l2, l3;
            split_value(v[0], h0, l0);
            split_value(v[1], h1, l1);
            split_value(v[2], h2, l2);
            split_value(v[3], h3, l3);
            __builtin_nontemporal_store(half4_t{h0, h1, h2, h3}, reinterpret_cast<half4_t *>(hi + r * ldh + c));
            __builtin_nontemporal_store(half4_t{l0, l1, l2, l3}, reinterpret_cast<half4_t *>(lo + r * ldh + c));
        } else {
            _Float16 h, l;
            split_value(x[r * ldx + c], h, l);
            hi[r * ldh + c] = __builtin_bit_cast(uint16_t, h);
            lo[r * ldh + c] = __builtin_bit_cast(uint16_t, l);
        }
    }
}

// Rows of FP16 W copied to rows of ldp elements, the first cols_out of
// each written (columns [cols, cols_out) zero; cols_out and ldp multiples
// of 8): one thread per 8 columns of a row, each writing one 16-byte piece;
// the source may sit at any 2-byte offset (load_row8 reads it in dwords, or
// element by element at the row's end).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void pad_rows_kernel(const uint16_t *__restrict__ w, int64_t ldw,
                                                            uint16_t *__restrict__ wp, int64_t ldp, int64_t rows,
                                                            int64_t cols, int64_t cols_out)
{
    const int64_t c = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 8;
    if (c >= cols_out) return;
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
        const uint4 v = load_row8<false>(w + r * ldw, c, cols);
        __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t *>(wp + r * ldp + c));
    }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void merge_kernel(const float *__restrict__ c_hi,
                                                         const float *__restrict__ c_lo, int64_t ldc,
                                                         float *__restrict__ y, int64_t ldy,
                                                         int64_t rows, int64_t cols)
{
    constexpr int kPer = VEC ? 4 : 1;
    const int64_t c = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kPer;
    if (c >= cols) return;
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
        if constexpr (VEC) {
            const floatx4_t a = __builtin_nontemporal_load(reinterpret_cast<const floatx4_t *>(c_hi + r * ldc + c));
            const floatx4_t b = __builtin_nontemporal_load(reinterpret_cast<const floatx4_t *>(c_lo + r * ldc + c));
            const floatx4_t o = {merge_value(a[0], b[0]), merge_value(a[1], b[1]), merge_value(a[2], b[2]),
                                 merge_value(a[3], b[3])};
            __builtin_nontemporal_store(o, reinterpret_cast<floatx4_t *>(y + r * ldy + c));
        } else {
            y[r * ldy + c] = merge_value(c_hi[r * ldc + c], c_lo[r * ldc + c]);
        }
    }
}

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Column groups go to grid.x (at most 2^31 - 1 blocks: cols < 2^39 per row).
dim3 grid_for(int64_t rows, int64_t cols, int per)
{
    const int64_t groups = (cols + per - 1) / per;
    const int64_t bx = (groups + kThreads - 1) / kThreads;
    const int64_t by = rows < kMaxGridY ? rows : kMaxGridY;
    return dim3((unsigned)bx, (unsigned)by, 1);
}

}  // namespace

hipError_t launch_split(const float *x, int64_t ldx, uint16_t *hi, uint16_t *lo, int64_t ldh,
                        int64_t rows, int64_t cols, int64_t cols_out, hipStream_t stream)
{
    if ((cols_out + kThreads - 1) / kThreads > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const bool vec = (cols % 4 == 0) && (cols_out % 4 == 0) && (ldx % 4 == 0) && (ldh % 4 == 0) &&
                     aligned(x, 16) && aligned(hi, 8) && aligned(lo, 8);
    if (vec) {
        split_kernel<true><<<grid_for(rows, cols_out, 4), kThreads, 0, stream>>>(x, ldx, hi, lo, ldh, rows, cols,
                                                                                  cols_out);
    } else {
        split_kernel<false><<<grid_for(rows, cols_out, 1), kThreads, 0, stream>>>(x, ldx, hi, lo, ldh, rows, cols,
                                                                                   cols_out);
    }
    return hipGetLastError();
}

hipError_t launch_pad_rows(const uint16_t *w, int64_t ldw, uint16_t *wp, int64_t ldp, int64_t rows, int64_t cols,
                           int64_t cols_out, hipStream_t stream)
{
    if (ldp % 8 || cols_out % 8 || cols_out < cols || cols_out > ldp || !aligned(wp, 16)) return hipErrorInvalidValue;
    if ((cols_out / 8 + kThreads - 1) / kThreads > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    pad_rows_kernel<<<grid_for(rows, cols_out, 8), kThreads, 0, stream>>>(w, ldw, wp, ldp, rows, cols, cols_out);
    return hipGetLastError();
}

hipError_t launch_merge(const float *c_hi, const float *c_lo, int64_t ldc, float *y, int64_t ldy,
                        int64_t rows, int64_t cols, hipStream_t stream)
{
    if ((cols + kThreads - 1) / kThreads > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const bool vec = (cols % 4 == 0) && (ldc % 4 == 0) && (ldy % 4 == 0) && aligned(c_hi, 16) &&
                     aligned(c_lo, 16) && aligned(y, 16);
    if (vec) {
        merge_kernel<true><<<grid_for(rows, cols, 4), kThreads, 0, stream>>>(c_hi, c_lo, ldc, y, ldy, rows, cols);
    } else {
        merge_kernel<false><<<grid_for(rows, cols, 1), kThreads, 0, stream>>>(c_hi, c_lo, ldc, y, ldy, rows, cols);
    }
    return hipGetLastError();
}

}  // namespace cfp32
