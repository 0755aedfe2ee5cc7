/*
 * CPU oracle for the compensated-FP32 projection.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists so that the tests, the
 * smoke check and the CPU-baseline leg of the benchmark can check the GPU
 * library against a plain, slow, obviously correct host implementation.
 * Nothing in the product path may link or call it, and it shares no source
 * with the GPU library.
 *
 * What it follows: the laya.cpp Vulkan backend guide (docs/vulkan.md),
 *   - its compensated-FP32 paragraph: each projection input is split into two
 *     FP16 parts, both products use FP32 accumulators, the two are combined
 *     in FP32, and the FP16 weights are taken as exact;
 *   - its split/merge paragraph: the split rounds to nearest-even, keeps FP16
 *     subnormals, and scales the residual by 1024 before rounding it;
 *   - its validation paragraph on the residual scale (1024 avoids FP16
 *     overflow for large activations).
 * Written out, for an FP32 value x:
 *   hi = RNE16(x),  lo = RNE16((x - hi) * 1024),
 *   C_hi = A_hi W,  C_lo = A_lo W  (FP32 accumulation),
 *   y = C_hi + C_lo / 1024 in FP32.
 *
 * Arithmetic rules kept here on purpose (build with -O2 -ffp-contract=off,
 * never -ffast-math, so that MXCSR keeps FTZ/DAZ clear):
 *   - RNE16 is written from its definition (nearest FP16 value, ties to the
 *     even significand) in exact double arithmetic, not with bit tricks;
 *   - every FP32 operation that must round (the merge, the FP32 accumulators)
 *     is a separate IEEE single-precision operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <xmmintrin.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* Floating-point environment                                                */
/* ------------------------------------------------------------------------- */

/* Returns 1 when the x86 MXCSR has flush-to-zero and denormals-are-zero off
 * and rounding is to nearest: the state every routine below assumes. */
int o_fp_env_ok(void)
{
    unsigned int csr = _mm_getcsr();
    const unsigned int ftz = 1u << 15, daz = 1u << 6, rc = 3u << 13;
    return (csr & (ftz | daz | rc)) == 0;
}

int o_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------- */
/* O1, O2: IEEE binary16 rounding and widening                               */
/* ------------------------------------------------------------------------- */

/* Nearest integer to t >= 0, ties to the even integer.  t is exact. */
static double round_half_even(double t)
{
    double f = floor(t);
    double d = t - f; /* exact: t and f share an exponent range */
    if (d > 0.5) return f + 1.0;
    if (d < 0.5) return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* RNE16: the binary16 value nearest to v, ties to the even significand,
 * returned as its bit pattern.  FP16 has 10 fraction bits, exponents -14..15
 * and subnormals spaced 2^-24.  With an unbounded exponent the rounded value
 * is q * 2^(e-10) for the binade e of |v| (e clamped below at -14 so that the
 * subnormal spacing is used); a rounded value above the largest finite FP16
 * (65504) becomes infinity.  NaN gives a quiet NaN (its payload is not part
 * of the definition).  v is any double; FP32 inputs are exact in it. */
uint16_t o_rne16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | 0x7E00u);
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0) return sign;

    int ex;
    (void)frexp(a, &ex);       /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;            /* binade: 2^e <= a < 2^(e+1) */
    if (e < -14) e = -14;      /* subnormal range keeps the 2^-24 spacing */
    double t = ldexp(a, 10 - e);           /* a / 2^(e-10), exact */
    double q = round_half_even(t);         /* q in [0, 2048] */
    if (ldexp(q, e - 10) > 65504.0) return (uint16_t)(sign | 0x7C00u);
    if (q == 0.0) return sign;
    /* Encoding: for e >= -14, bits = (e + 15) * 1024 + (q - 1024).  This also
     * covers q = 2048 (carry into the next binade) and, at e = -14 with
     * q < 1024, the subnormal encoding bits = q. */
    long bits = (long)(e + 15) * 1024 + (long)q - 1024;
    return (uint16_t)(sign | (uint16_t)bits);
}

uint16_t o_f16_rne(float x) { return o_rne16((double)x); }

/* Exact widening of a binary16 bit pattern. */
double o_f16_value(uint16_t h)
{
    int s = (h >> 15) & 1;
    int ef = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (ef == 0x1F) v = m ? NAN : INFINITY;
    else if (ef == 0) v = ldexp((double)m, -24);              /* subnormal */
    else v = ldexp((double)(1024 + m), ef - 25);              /* normal */
    return s ? -v : v;
}

float o_f16_to_f32(uint16_t h) { return (float)o_f16_value(h); }

void o_f16_rne_array(const float *x, uint16_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = o_rne16((double)x[i]);
}

void o_f16_widen_array(const uint16_t *h, float *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = o_f16_to_f32(h[i]);
}

/* ------------------------------------------------------------------------- */
/* O3: the split                                                             */
/* ------------------------------------------------------------------------- */

/* hi = RNE16(x); r = x - hi; lo = RNE16(r * 1024).
 * In double, x - hi is exact (both are FP32-representable and within a few
 * FP16 ulps of each other), and so is the power-of-two scale, so lo is rounded
 * exactly once.  IEEE subtraction of equal values gives +0, so x = -0 gives
 * lo = +0; for |x| >= 65520 hi is infinite and the residual is -inf * sign
 * (or NaN when x itself is infinite). */
void o_split1(float x, uint16_t *hi, uint16_t *lo)
{
    uint16_t h = o_rne16((double)x);
    double r = (double)x - o_f16_value(h);
    *hi = h;
    *lo = o_rne16(r * 1024.0);
}

/* Split a rows x cols FP32 matrix (leading dimension ldx) into two FP16
 * planes with leading dimension ldh. */
void o_split(const float *x, int64_t ldx, uint16_t *hi, uint16_t *lo,
             int64_t ldh, int64_t rows, int64_t cols)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j)
            o_split1(x[i * ldx + j], &hi[i * ldh + j], &lo[i * ldh + j]);
}

/* Compare a split produced elsewhere against the definition.  Exact match on
 * the bit patterns, except that NaN results match any NaN (payload and sign
 * of NaN are outside the definition).  Returns the number of mismatching
 * elements; *first gets the index of the first one (or -1). */
static int is_nan16(uint16_t h) { return (h & 0x7C00u) == 0x7C00u && (h & 0x3FFu) != 0; }

static int same16(uint16_t want, uint16_t got)
{
    if (is_nan16(want)) return is_nan16(got);
    return want == got;
}

int64_t o_split_mismatches(const float *x, const uint16_t *hi, const uint16_t *lo,
                           int64_t n, int64_t *first)
{
    int64_t bad = 0, first_bad = -1;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t i = 0; i < n; ++i) {
        uint16_t h, l;
        o_split1(x[i], &h, &l);
        if (!same16(h, hi[i]) || !same16(l, lo[i])) {
            ++bad;
#pragma omp critical
            {
                if (first_bad < 0 || i < first_bad) first_bad = i;
            }
        }
    }
    if (first) *first = first_bad;
    return bad;
}

/* ------------------------------------------------------------------------- */
/* O4: the merge                                                             */
/* ------------------------------------------------------------------------- */

/* y = C_hi + C_lo / 1024, as two IEEE single-precision operations: the scale
 * by 2^-10 (exact unless the result is FP32-subnormal) and one rounded add.
 * Going through double and back would round twice, so it is not done. */
float o_merge1(float c_hi, float c_lo)
{
    volatile float t = c_lo * 0x1p-10f;
    volatile float y = c_hi + t;
    return y;
}

void o_merge(const float *c_hi, const float *c_lo, int64_t ldc, float *y,
             int64_t ldy, int64_t rows, int64_t cols)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j)
            y[i * ldy + j] = o_merge1(c_hi[i * ldc + j], c_lo[i * ldc + j]);
}

/* ------------------------------------------------------------------------- */
/* O5: products                                                              */
/* ------------------------------------------------------------------------- */

/* O5(b): the method on the CPU.  A is FP32 [M,K] (lda), W is FP16 bits
 * [K,N] (ldw), outputs are FP32 [M,N] (ldc).  Each row of A is split, the two
 * products are accumulated in FP32 with k ascending (an FP16 x FP16 product is
 * exact in FP32, so each step rounds once, at the add), and the merge is
 * applied once, after both sums are complete.  Any of the three outputs may
 * be NULL.  Rows are independent and shared among threads. */
void o_linear_cf32(const float *A, int64_t lda, const uint16_t *W, int64_t ldw,
                   float *y, float *c_hi, float *c_lo, int64_t ldc,
                   int64_t M, int64_t N, int64_t K)
{
#pragma omp parallel
    {
        float *hi = (float *)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
        float *lo = (float *)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
        float *sh = (float *)malloc(sizeof(float) * (size_t)(N > 0 ? N : 1));
        float *sl = (float *)malloc(sizeof(float) * (size_t)(N > 0 ? N : 1));
        float *wrow = (float *)malloc(sizeof(float) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < M; ++i) {
            for (int64_t k = 0; k < K; ++k) {
                uint16_t h, l;
                o_split1(A[i * lda + k], &h, &l);
                hi[k] = o_f16_to_f32(h);
                lo[k] = o_f16_to_f32(l);
            }
            for (int64_t j = 0; j < N; ++j) sh[j] = 0.0f, sl[j] = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                const uint16_t *wk = W + k * ldw;
                for (int64_t j = 0; j < N; ++j) wrow[j] = o_f16_to_f32(wk[j]);
                const float h = hi[k], l = lo[k];
                for (int64_t j = 0; j < N; ++j) {
                    sh[j] = sh[j] + h * wrow[j];
                    sl[j] = sl[j] + l * wrow[j];
                }
            }
            for (int64_t j = 0; j < N; ++j) {
                if (c_hi) c_hi[i * ldc + j] = sh[j];
                if (c_lo) c_lo[i * ldc + j] = sl[j];
                if (y) y[i * ldc + j] = o_merge1(sh[j], sl[j]);
            }
        }
        free(hi);
        free(lo);
        free(sh);
        free(sl);
        free(wrow);
    }
}

/* O5(c): the plain FP32 product, y = sum_k fma(a, w, acc) with k ascending;
 * the activation is used as FP32, with no FP16 conversion. */
void o_linear_f32(const float *A, int64_t lda, const uint16_t *W, int64_t ldw,
                  float *y, int64_t ldy, int64_t M, int64_t N, int64_t K)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            float acc = 0.0f;
            for (int64_t k = 0; k < K; ++k)
                acc = fmaf(A[i * lda + k], o_f16_to_f32(W[k * ldw + j]), acc);
            y[i * ldy + j] = acc;
        }
}

/* O5(a) at chosen output positions: y64 = sum_k a*w and abs64 = sum_k |a*w|
 * in double, k ascending.  Each product of an FP32 and an FP16 value is exact
 * in double; the sum carries at most K double roundings, far below any FP32
 * effect.  rows[i], cols[i] give the positions. */
void o_dot64_at(const float *A, int64_t lda, const uint16_t *W, int64_t ldw,
                int64_t K, const int64_t *rows, const int64_t *cols, int64_t n,
                double *y64, double *abs64)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        const float *a = A + rows[t] * lda;
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = (double)a[k] * o_f16_value(W[k * ldw + cols[t]]);
            s += p;
            sa += fabs(p);
        }
        y64[t] = s;
        abs64[t] = sa;
    }
}

/* O5(e) at chosen positions: sum_k (hi + lo/1024) * w in double, which keeps
 * only the representation error of the split and drops every FP32 rounding. */
void o_ideal64_at(const float *A, int64_t lda, const uint16_t *W, int64_t ldw,
                  int64_t K, const int64_t *rows, const int64_t *cols, int64_t n,
                  double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        const float *a = A + rows[t] * lda;
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            uint16_t h, l;
            o_split1(a[k], &h, &l);
            double v = o_f16_value(h) + o_f16_value(l) / 1024.0;
            s += v * o_f16_value(W[k * ldw + cols[t]]);
        }
        out[t] = s;
    }
}

/* ------------------------------------------------------------------------- */
/* GEGLU (laya.cpp Vulkan guide, graph paragraph: the FP32 feed-forward      */
/* layers apply GEGLU to the projection output in one fused step).  The      */
/* guide names no GELU approximation; the exact form x * Phi(x) is used:     */
/*   gelu(g) = g / 2 * (1 + erf(g / sqrt 2)),  out = gelu(gate) * up,        */
/* in double precision from the FP32 gate and up values.                     */
/* ------------------------------------------------------------------------- */

double o_gelu64(double g) { return 0.5 * g * (1.0 + erf(g / sqrt(2.0))); }

void o_geglu64(const float *gate, const float *up, int64_t n, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = o_gelu64((double)gate[i]) * (double)up[i];
}

/* ------------------------------------------------------------------------- */
/* Q/K/V packing with rotary multiplication (laya.cpp Vulkan guide, graph    */
/* paragraph: one dispatch packs the projection output into Q, K and V and   */
/* applies the rotary multiplication).  The guide gives no convention; the   */
/* one taken here: row t of the projection output holds [q | k | v], each    */
/* H heads of D values (head h at h*D); outputs are head-major [H][T][D];    */
/* q and k are rotated in the half-split pairing, dims d and d + D/2 forming */
/* pair i = d < D/2 with angle pos[t] * theta^(-2i/D):                       */
/*   x1' = x1 cos - x2 sin,  x2' = x2 cos + x1 sin;  v is copied.             */
/* Everything in double, from the FP32 inputs.                                */
/* ------------------------------------------------------------------------- */

void o_qkv_rotary(const float *qkv, int64_t ldq, const int64_t *pos, double theta, int64_t T, int64_t H,
                  int64_t D, double *q, double *k, double *v)
{
    const int64_t half = D / 2;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h) {
            const float *row = qkv + t * ldq;
            for (int64_t i = 0; i < half; ++i) {
                const double ang = (double)pos[t] * pow(theta, -2.0 * (double)i / (double)D);
                const double c = cos(ang), s = sin(ang);
                for (int p = 0; p < 2; ++p) {  /* p = 0: q, 1: k */
                    const float *src = row + p * H * D + h * D;
                    double *dst = (p == 0 ? q : k) + (h * T + t) * D;
                    const double x1 = src[i], x2 = src[i + half];
                    dst[i] = x1 * c - x2 * s;
                    dst[i + half] = x2 * c + x1 * s;
                }
            }
            for (int64_t d = 0; d < D; ++d) v[(h * T + t) * D + d] = row[2 * H * D + h * D + d];
        }
}
