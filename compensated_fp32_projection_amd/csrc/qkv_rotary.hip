// Q/K/V packing with the rotary multiplication, one dispatch (laya.cpp Vulkan
// guide, graph paragraph: packing and rotary share one shader dispatch).
//
// Input: the QKV projection output, row t = [q | k | v], each H heads of D
// FP32 values (head h at h*D).  Output: q, k, v head-major [H][T][D].  q and
// k are rotated in the half-split pairing: dims i and i + D/2 (i < D/2) turn
// by pos[t] * theta^(-2i/D); v is copied.  One thread per (t, h, i): it reads
// the pair from q, k and v and writes both dims of each; consecutive threads
// take consecutive i, so a wave reads and writes contiguous runs.
//
// FP32 throughout, as written (-ffp-contract=off): the frequency as
// exp2(-(2i/D) log2 theta), the angle as pos * frequency, sincosf, and four
// products and two sums per rotated pair.
#include "device_common.h"
#include "launchers.h"

namespace cfp32 {

namespace {

__global__ __launch_bounds__(256) void qkv_rotary_kernel(const float *__restrict__ qkv, int64_t ldq,
                                                         const int64_t *__restrict__ pos, float log2_theta,
                                                         float *__restrict__ q, float *__restrict__ k,
                                                         float *__restrict__ v, int64_t T, int64_t H, int64_t D)
{
    const int64_t half = D / 2;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= T * H * half) return;
    const int64_t i = idx % half;
    const int64_t th = idx / half;
    const int64_t h = th % H;
    const int64_t t = th / H;
    const float p = (float)(pos ? pos[t] : t);
    const float freq = exp2f(-((float)(2 * i) / (float)D) * log2_theta);
    const float ang = p * freq;
    float s, c;
    sincosf(ang, &s, &c);
    const float *row = qkv + t * ldq + h * D;
    const int64_t o = (h * T + t) * D;
#pragma unroll
    for (int part = 0; part < 2; ++part) {  // q, then k
        const float x1 = row[part * H * D + i], x2 = row[part * H * D + i + half];
        float *dst = part == 0 ? q : k;
        const float a = x1 * c, b = x2 * s, e = x2 * c, f = x1 * s;
        dst[o + i] = a - b;
        dst[o + i + half] = e + f;
    }
    v[o + i] = row[2 * H * D + i];
    v[o + i + half] = row[2 * H * D + i + half];
}

}  // namespace

hipError_t launch_qkv_rotary(const float *qkv, int64_t ldq, const int64_t *pos, double theta, float *q, float *k,
                             float *v, int64_t T, int64_t H, int64_t D, hipStream_t stream)
{
    const int64_t n = T * H * (D / 2);
    if (n == 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    qkv_rotary_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(qkv, ldq, pos, (float)log2(theta), q, k, v, T,
                                                                  H, D);
    return hipGetLastError();
}

}  // namespace cfp32
