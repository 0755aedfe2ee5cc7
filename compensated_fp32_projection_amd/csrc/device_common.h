// Device helpers shared by the gfx950 kernels of libcfp32.
//
// Build flags that the arithmetic below relies on (see build.py):
//   -ffp-contract=off              no implicit fused multiply-add, so the merge
//                                  rounds its scale and its add separately;
//   -fno-gpu-flush-denormals-to-zero  FP32 subnormals are kept (the split of a
//                                  negative FP32 subnormal needs its sign);
//   no -ffast-math.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cfp32 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// The split of one FP32 value (laya.cpp Vulkan guide, split/merge paragraph):
// hi = RNE16(x); lo = RNE16((x - hi) * 1024).  The FP32 -> FP16 conversion
// rounds to nearest even and produces FP16 subnormals (gfx950's default
// rounding and FP16 denormal modes).  x - hi is exact in FP32 (hi is the
// FP16 value nearest to x, so the difference needs at most 14 significant
// bits at x's own scale), and the power-of-two scale is exact, so lo is
// rounded once.
__device__ __forceinline__ void split_value(float x, _Float16 &hi, _Float16 &lo)
{
    hi = (_Float16)x;
    float r = x - (float)hi;
    lo = (_Float16)(r * 1024.0f);
}

// The merge (guide, compensated-FP32 paragraph): y = C_hi + C_lo / 1024 in
// FP32, as a rounded scale (exact unless the result is FP32-subnormal) and a
// rounded add.  With -ffp-contract=off these stay two operations.
__device__ __forceinline__ float merge_value(float c_hi, float c_lo)
{
    float t = c_lo * 0x1p-10f;
    return c_hi + t;
}

// GELU in its exact form, x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), in FP32
// (the GEGLU activation of the laya.cpp Vulkan guide's graph paragraph, which
// names the fused GEGLU shader but not a GELU approximation).
__device__ __forceinline__ float gelu_value(float x)
{
    const float t = x * 0.70710678118654752f;
    const float c = 1.0f + erff(t);
    return (0.5f * x) * c;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// Eight consecutive FP16 values [col, col + 8) of one row holding `ncols`
// valid entries, as 16 bytes; entries at or past ncols read as +0.  With
// ALIGNED (row start and col 16-byte aligned) a full group is one 16-byte
// load.  Otherwise a full group at a 4-byte boundary is four dword loads, and
// one 2 bytes past a boundary is five dword loads from the element before it
// (which must be in the row, as must the element after it) joined by 16-bit
// funnel shifts; every load is dword aligned, so none relies on the
// hardware's unaligned-access mode (333 x 1000 x 777: 107 -> 70 us against
// element gathers; the same five loads for both alignments, without the
// branch, measured 80 us).  The ragged end is gathered element by element.
template <bool ALIGNED>
__device__ __forceinline__ uint4 load_row8(const uint16_t *__restrict__ row, int64_t col, int64_t ncols)
{
    if (ALIGNED && col + 8 <= ncols) return *reinterpret_cast<const uint4 *>(row + col);
    if (!ALIGNED && col + 8 <= ncols) {
        const uint16_t *p = row + col;
        if ((reinterpret_cast<uintptr_t>(p) & 3) == 0) {
            const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
            return make_uint4(q[0], q[1], q[2], q[3]);
        }
        if (col >= 1 && col + 9 <= ncols) {
            const uint32_t *q = reinterpret_cast<const uint32_t *>(p - 1);  // elements col - 1 .. col + 8
            const uint32_t d0 = q[0], d1 = q[1], d2 = q[2], d3 = q[3], d4 = q[4];
            return make_uint4(__builtin_amdgcn_alignbit(d1, d0, 16), __builtin_amdgcn_alignbit(d2, d1, 16),
                              __builtin_amdgcn_alignbit(d3, d2, 16), __builtin_amdgcn_alignbit(d4, d3, 16));
        }
    }
    uint32_t v[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (col + e < ncols) v[e >> 1] |= (uint32_t)row[col + e] << (16 * (e & 1));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

}  // namespace cfp32
