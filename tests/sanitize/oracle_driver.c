/* The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer:
 * every function of oracle/cfp32_oracle.c on buffers allocated to the exact
 * extent a call may touch (the last row of a strided matrix holds only its
 * own columns), so that any read or write past an operand is reported; plus
 * a few values fixed by the definitions (binary16 round trips, split vectors,
 * a merge tie, an exact product).  Exit status 0 when every check holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int o_fp_env_ok(void);
int o_num_threads(void);
uint16_t o_rne16(double v);
uint16_t o_f16_rne(float x);
double o_f16_value(uint16_t h);
float o_f16_to_f32(uint16_t h);
void o_f16_rne_array(const float *x, uint16_t *out, int64_t n);
void o_f16_widen_array(const uint16_t *h, float *out, int64_t n);
void o_split1(float x, uint16_t *hi, uint16_t *lo);
void o_split(const float *x, int64_t ldx, uint16_t *hi, uint16_t *lo, int64_t ldh, int64_t rows, int64_t cols);
int64_t o_split_mismatches(const float *x, const uint16_t *hi, const uint16_t *lo, int64_t n, int64_t *first);
float o_merge1(float c_hi, float c_lo);
void o_merge(const float *c_hi, const float *c_lo, int64_t ldc, float *y, int64_t ldy, int64_t rows, int64_t cols);
void o_linear_cf32(const float *A, int64_t lda, const uint16_t *W, int64_t ldw, float *y, float *c_hi, float *c_lo,
                   int64_t ldc, int64_t M, int64_t N, int64_t K);
void o_linear_f32(const float *A, int64_t lda, const uint16_t *W, int64_t ldw, float *y, int64_t ldy, int64_t M,
                  int64_t N, int64_t K);
void o_dot64_at(const float *A, int64_t lda, const uint16_t *W, int64_t ldw, int64_t K, const int64_t *rows,
                const int64_t *cols, int64_t n, double *y64, double *abs64);
void o_ideal64_at(const float *A, int64_t lda, const uint16_t *W, int64_t ldw, int64_t K, const int64_t *rows,
                  const int64_t *cols, int64_t n, double *out);
double o_gelu64(double g);
void o_geglu64(const float *gate, const float *up, int64_t n, double *out);
void o_qkv_rotary(const float *qkv, int64_t ldq, const int64_t *pos, double theta, int64_t T, int64_t H, int64_t D,
                  double *q, double *k, double *v);

static int failures = 0;
#define CHECK(cond)                                                             \
    do {                                                                        \
        if (!(cond)) {                                                          \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);  \
            ++failures;                                                         \
        }                                                                       \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uniform(void) /* xorshift64*, in [-1, 1) */
{
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}

/* A strided rows x cols matrix allocated to exactly (rows - 1) * ld + cols
 * elements. */
static void *strided(size_t elem, int64_t rows, int64_t cols, int64_t ld)
{
    size_t n = rows > 0 ? (size_t)((rows - 1) * ld + cols) : 1;
    return malloc(elem * n);
}

static float f32_bits(uint32_t b)
{
    float f;
    memcpy(&f, &b, 4);
    return f;
}

int main(void)
{
    CHECK(o_fp_env_ok());
    CHECK(o_num_threads() >= 1);

    /* every binary16 pattern: widen and round back */
    int bad = 0;
    for (uint32_t h = 0; h < 65536; ++h) {
        double v = o_f16_value((uint16_t)h);
        if (isnan(v)) continue;
        if (o_rne16(v) != h) ++bad;
        if (o_f16_rne(o_f16_to_f32((uint16_t)h)) != h) ++bad;
    }
    CHECK(bad == 0);

    /* split vectors fixed by the definition: 1/3, -0, 32784, 3 * 2^-25, -2^-149 */
    uint16_t hi, lo;
    o_split1(f32_bits(0x3EAAAAABu), &hi, &lo);
    CHECK(hi == 0x3555 && lo == 0x2D56);
    o_split1(-0.0f, &hi, &lo);
    CHECK(hi == 0x8000 && lo == 0x0000);
    o_split1(32784.0f, &hi, &lo);
    CHECK(hi == 0x7800 && lo == 0x7400);
    o_split1(3.0f * ldexpf(1.0f, -25), &hi, &lo);
    CHECK(hi == 0x0002 && lo == 0x8200);
    o_split1(f32_bits(0x80000001u), &hi, &lo);
    CHECK(hi == 0x8000 && lo == 0x8000);
    /* merge tie: 1 + 2^-14 / 1024 rounds to the even 1 */
    CHECK(o_merge1(1.0f, ldexpf(1.0f, -14)) == 1.0f);

    /* arrays at exact sizes */
    const int64_t n = 1000;
    float *xs = malloc(sizeof(float) * n);
    uint16_t *hs = malloc(sizeof(uint16_t) * n);
    float *ws = malloc(sizeof(float) * n);
    for (int64_t i = 0; i < n; ++i) xs[i] = (float)(uniform() * 70000.0);
    o_f16_rne_array(xs, hs, n);
    o_f16_widen_array(hs, ws, n);
    for (int64_t i = 0; i < n; ++i) CHECK(o_f16_rne(xs[i]) == hs[i]);

    /* strided split, merge and mismatch count */
    const int64_t R = 7, C = 33, ldx = 37, ldh = 35;
    float *x = strided(4, R, C, ldx);
    uint16_t *ph = strided(2, R, C, ldh), *pl = strided(2, R, C, ldh);
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c) x[r * ldx + c] = (float)(uniform() * 3e4);
    o_split(x, ldx, ph, pl, ldh, R, C);
    uint16_t h0, l0;
    o_split1(x[3 * ldx + 5], &h0, &l0);
    CHECK(ph[3 * ldh + 5] == h0 && pl[3 * ldh + 5] == l0);
    float *dense = malloc(sizeof(float) * R * C);
    uint16_t *dh = malloc(2 * R * C), *dl = malloc(2 * R * C);
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c) {
            dense[r * C + c] = x[r * ldx + c];
            dh[r * C + c] = ph[r * ldh + c];
            dl[r * C + c] = pl[r * ldh + c];
        }
    int64_t first = 0;
    CHECK(o_split_mismatches(dense, dh, dl, R * C, &first) == 0 && first == -1);
    dl[R * C - 1] ^= 1;
    CHECK(o_split_mismatches(dense, dh, dl, R * C, &first) == 1 && first == R * C - 1);
    float *ch = strided(4, R, C, ldx), *cl = strided(4, R, C, ldx), *y = strided(4, R, C, ldh);
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c) ch[r * ldx + c] = (float)uniform(), cl[r * ldx + c] = (float)uniform();
    o_merge(ch, cl, ldx, y, ldh, R, C);
    CHECK(y[2 * ldh + 7] == o_merge1(ch[2 * ldx + 7], cl[2 * ldx + 7]));

    /* products on strided operands: A [M, K] (lda), W [K, N] (ldw), outputs (ldc) */
    const int64_t M = 5, K = 67, N = 19, lda = 70, ldw = 24, ldc = 21;
    float *A = strided(4, M, K, lda);
    uint16_t *W = strided(2, K, N, ldw);
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k) A[i * lda + k] = (float)(uniform() * 8.0);
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j) W[k * ldw + j] = o_f16_rne((float)(uniform() * 0.05));
    float *yc = strided(4, M, N, ldc), *yh = strided(4, M, N, ldc), *yl = strided(4, M, N, ldc);
    float *yf = strided(4, M, N, ldc);
    o_linear_cf32(A, lda, W, ldw, yc, yh, yl, ldc, M, N, K);
    o_linear_cf32(A, lda, W, ldw, NULL, yh, NULL, ldc, M, N, K);
    o_linear_cf32(A, lda, W, ldw, yc, NULL, NULL, ldc, M, N, K);
    o_linear_f32(A, lda, W, ldw, yf, ldc, M, N, K);
    int64_t rows[3] = {0, 2, M - 1}, cols[3] = {N - 1, 4, 0};
    double y64[3], abs64[3], ideal[3];
    o_dot64_at(A, lda, W, ldw, K, rows, cols, 3, y64, abs64);
    o_ideal64_at(A, lda, W, ldw, K, rows, cols, 3, ideal);
    for (int t = 0; t < 3; ++t) {
        const double got_c = yc[rows[t] * ldc + cols[t]], got_f = yf[rows[t] * ldc + cols[t]];
        CHECK(fabs(got_c - y64[t]) <= 1e-5 * abs64[t]);
        CHECK(fabs(got_f - y64[t]) <= 1e-5 * abs64[t]);
        CHECK(fabs(ideal[t] - y64[t]) <= 1e-6 * abs64[t]);
    }
    /* K = 0 and M = 0 touch nothing beyond their (empty) extents */
    o_linear_cf32(A, lda, W, ldw, yc, yh, yl, ldc, M, N, 0);
    CHECK(yc[0] == 0.0f && yh[ldc + 3] == 0.0f);
    o_linear_f32(A, lda, W, ldw, yf, ldc, 0, N, K);

    /* GEGLU and Q/K/V + rotary */
    CHECK(o_gelu64(0.0) == 0.0 && fabs(o_gelu64(1.0) - o_gelu64(-1.0) - 1.0) < 1e-15);
    double *gg = malloc(sizeof(double) * n);
    o_geglu64(xs, ws, n, gg);
    const int64_t T = 5, H = 2, D = 6, ldq = 3 * H * D + 3;
    float *qkv = strided(4, T, 3 * H * D, ldq);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < 3 * H * D; ++c) qkv[t * ldq + c] = (float)uniform();
    int64_t pos[5] = {0, 1, 2, 7, 100};
    double *q = malloc(sizeof(double) * H * T * D), *k = malloc(sizeof(double) * H * T * D);
    double *v = malloc(sizeof(double) * H * T * D);
    o_qkv_rotary(qkv, ldq, pos, 10000.0, T, H, D, q, k, v);
    CHECK(q[0] == (double)qkv[0]); /* position 0: no rotation */
    CHECK(v[(1 * T + 3) * D + 5] == (double)qkv[3 * ldq + 2 * H * D + 1 * D + 5]);

    free(xs); free(hs); free(ws); free(x); free(ph); free(pl); free(dense); free(dh); free(dl);
    free(ch); free(cl); free(y); free(A); free(W); free(yc); free(yh); free(yl); free(yf);
    free(gg); free(qkv); free(q); free(k); free(v);
    fprintf(stderr, "oracle_driver: %d failure(s)\n", failures);
    return failures == 0 ? 0 : 1;
}
