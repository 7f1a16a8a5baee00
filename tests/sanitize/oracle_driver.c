/* Drives the C oracle (oracle/qmat_oracle.c) under a host sanitizer: every bit pattern of the
 * number-format conversions, the dequantizers, the multi-threaded reference product and the
 * encoders on small ragged inputs, and their error returns.  Buffers are allocated at exactly
 * the documented size, so a read or write past one is caught.  The checks are consistency
 * checks between the oracle's own functions and plain bit arithmetic; the numerical pins live
 * in the Python tests.  Exits 0 when every check holds, 1 otherwise. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double qo_half_to_double(uint16_t h);
double qo_bf16_to_double(uint16_t b);
double qo_e4m3_to_double(uint8_t b);
uint16_t qo_double_to_half_rne(double v);
int qo_dequant_groupwise(int bits, int64_t M, int64_t K, const int8_t *codes, const uint16_t *scales, float *w);
int qo_dequant_fp8(int64_t M, int64_t K, const uint8_t *bytes, const float *r, float *w);
int qo_gemv(int fmt, int64_t M, int64_t K, int64_t T, const void *codes, const void *scales, const uint16_t *x,
            const int64_t *rows, int64_t nrows, double *y, double *A, int nthreads);
int qo_rtn_encode(int bits, int64_t ngroups, const double *w, int8_t *codes, uint16_t *scales);
int qo_grouped_search_encode(int bits, int64_t ngroups, const double *w, const double *h, int8_t *codes,
                             uint16_t *scales);
uint8_t qo_float_to_e4m3_rne_sat(float q);
int qo_fp8_row_encode(int64_t M, int64_t K, const float *w, uint8_t *bytes, float *r);

static int failures = 0;

static void check(int cond, const char *what, long long a, long long b)
{
    if (!cond) {
        printf("FAIL %s (%lld, %lld)\n", what, a, b);
        ++failures;
    }
}

/* xorshift64*: the driver's own input draws */
static uint64_t rng_state = 0x853C49E6748FEA9BULL;
static uint64_t rng_next(void)
{
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1DULL;
}
static double uniform(void) { return (double)(rng_next() >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0; }

static void conversions(void)
{
    for (uint32_t h = 0; h < 65536; ++h) {
        const double v = qo_half_to_double((uint16_t)h);
        if ((h & 0x7C00) == 0x7C00 && (h & 0x3FF)) {
            check(isnan(v), "half NaN", h, 0);
        } else {
            /* every finite half and both infinities convert back to the same bits */
            check(qo_double_to_half_rne(v) == h, "half round trip", h, qo_double_to_half_rne(v));
        }
        /* bf16 is the top half of a binary32 */
        const uint32_t f32 = h << 16;
        float f;
        memcpy(&f, &f32, 4);
        const double b = qo_bf16_to_double((uint16_t)h);
        check((isnan(f) && isnan(b)) || b == (double)f, "bf16 value", h, 0);
        check(!signbit(b) == !signbit(f), "bf16 sign", h, 0);
    }
    for (int e = 0; e < 256; ++e) {
        const double v = qo_e4m3_to_double((uint8_t)e);
        if ((e & 0x7F) == 0x7F) {
            check(isnan(v), "E4M3 NaN", e, 0);
            continue;
        }
        check(fabs(v) <= 448.0, "E4M3 range", e, 0);
        check(qo_float_to_e4m3_rne_sat((float)v) == e, "E4M3 round trip", e, qo_float_to_e4m3_rne_sat((float)v));
    }
    check(qo_float_to_e4m3_rne_sat(1.0e30f) == 0x7E, "E4M3 saturates", 0, 0);
    check(qo_float_to_e4m3_rne_sat(-1.0e30f) == 0xFE, "E4M3 saturates (negative)", 0, 0);
}

static void products(int fmt, int64_t M, int64_t K, int64_t T)
{
    const int bits = fmt == 9 ? 8 : fmt;
    const int64_t G = K / 64;
    uint8_t *codes = (uint8_t *)malloc((size_t)(M * K));
    void *scales = malloc(fmt == 8 ? (size_t)M * 4 : (size_t)(M * G) * 2);
    float *w = (float *)malloc(sizeof(float) * (size_t)(M * K));
    uint16_t *x = (uint16_t *)malloc(2 * (size_t)(T * K));
    for (int64_t i = 0; i < M * K; ++i) {
        if (fmt == 8) {
            uint8_t b = (uint8_t)rng_next();
            codes[i] = (b & 0x7F) == 0x7F ? 0x00 : b;
        } else {
            codes[i] = (uint8_t)(int8_t)((int)(rng_next() % (1u << bits)) - (1 << (bits - 1)));
        }
    }
    if (fmt == 8) {
        for (int64_t i = 0; i < M; ++i) ((float *)scales)[i] = (float)(uniform() * 0.01);
    } else {
        for (int64_t i = 0; i < M * G; ++i) ((uint16_t *)scales)[i] = qo_double_to_half_rne(uniform() * 0.02);
    }
    for (int64_t i = 0; i < T * K; ++i) {
        const float f = (float)uniform();
        uint32_t u;
        memcpy(&u, &f, 4);
        x[i] = (uint16_t)(u >> 16);
    }
    const int st = fmt == 8 ? qo_dequant_fp8(M, K, codes, (const float *)scales, w)
                            : qo_dequant_groupwise(bits, M, K, (const int8_t *)codes, (const uint16_t *)scales, w);
    check(st == 0, "dequant", fmt, M);

    double *y = (double *)malloc(sizeof(double) * (size_t)(T * M));
    double *A = (double *)malloc(sizeof(double) * (size_t)(T * M));
    check(qo_gemv(fmt, M, K, T, codes, scales, x, NULL, M, y, A, 3) == 0, "gemv all rows", fmt, M);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < M; ++n) {
            double s = 0.0, a = 0.0;
            for (int64_t j = 0; j < K; ++j) {
                /* FP8: the exact product of the row scale and the E4M3 value (the dequantized
                 * fp32 weight is that product rounded once); groupwise: the fp32 weight is exact */
                const double wd = fmt == 8 ? (double)((const float *)scales)[n] * qo_e4m3_to_double(codes[n * K + j])
                                           : (double)w[n * K + j];
                if (fmt == 8) check(w[n * K + j] == (float)wd, "fp8 dequant = rounded product", n, j);
                const double p = wd * qo_bf16_to_double(x[t * K + j]);
                s += p;
                a += fabs(p);
            }
            check(s == y[t * M + n] && a == A[t * M + n], "gemv = sum of dequantized products", t, n);
        }
    /* a row subset, single-threaded, without A: the same values at those rows */
    int64_t rows[3] = {M - 1, 0, M / 2};
    double *ys = (double *)malloc(sizeof(double) * (size_t)(T * 3));
    check(qo_gemv(fmt, M, K, T, codes, scales, x, rows, 3, ys, NULL, 1) == 0, "gemv row subset", fmt, M);
    for (int64_t t = 0; t < T; ++t)
        for (int r = 0; r < 3; ++r) check(ys[t * 3 + r] == y[t * M + rows[r]], "gemv subset value", t, r);
    free(ys);
    free(A);
    free(y);
    free(x);
    free(w);
    free(scales);
    free(codes);
}

static void encoders(int bits, int64_t ngroups)
{
    double *w = (double *)malloc(sizeof(double) * (size_t)(64 * ngroups));
    double *h = (double *)malloc(sizeof(double) * (size_t)(64 * ngroups));
    int8_t *c = (int8_t *)malloc((size_t)(64 * ngroups));
    uint16_t *s = (uint16_t *)malloc(2 * (size_t)ngroups);
    for (int64_t i = 0; i < 64 * ngroups; ++i) {
        w[i] = i / 64 == 1 ? 0.0 : uniform() * (i % 11 == 0 ? 5.0 : 1.0); /* group 1 all zero */
        h[i] = i % 7 == 0 ? 0.0 : 1.0 + uniform();
    }
    const int lo = -(1 << (bits - 1)), hi = (1 << (bits - 1)) - 1;
    for (int enc = 0; enc < 2; ++enc) {
        const int st = enc ? qo_grouped_search_encode(bits, ngroups, w, h, c, s) : qo_rtn_encode(bits, ngroups, w, c, s);
        check(st == 0, enc ? "grouped search" : "rtn", bits, ngroups);
        for (int64_t i = 0; i < 64 * ngroups; ++i) check(c[i] >= lo && c[i] <= hi, "code range", bits, i);
        for (int64_t g = 0; g < ngroups; ++g) check((s[g] & 0x7C00) != 0x7C00, "finite scale", bits, g);
        if (ngroups > 1) check(s[1] == 0, "all-zero group scale", bits, enc);
    }
    w[64 * ngroups - 1] = NAN;
    check(qo_rtn_encode(bits, ngroups, w, c, s) == -2, "rtn NaN", bits, 0);
    w[64 * ngroups - 1] = 0.5;
    h[64 * ngroups - 1] = -1.0;
    check(qo_grouped_search_encode(bits, ngroups, w, h, c, s) == -2, "grouped search negative h", bits, 0);
    w[0] = 1.0e9; /* max|w| / qmax overflows FP16 */
    check(qo_rtn_encode(bits, ngroups, w, c, s) == -2, "rtn FP16 overflow", bits, 0);
    check(qo_rtn_encode(3, ngroups, w, c, s) == -1, "rtn bad bits", 3, 0);
    free(s);
    free(c);
    free(h);
    free(w);
}

static void fp8_encoder(int64_t M, int64_t K)
{
    float *w = (float *)malloc(sizeof(float) * (size_t)(M * K));
    uint8_t *b = (uint8_t *)malloc((size_t)(M * K));
    float *r = (float *)malloc(sizeof(float) * (size_t)M);
    float *back = (float *)malloc(sizeof(float) * (size_t)(M * K));
    for (int64_t i = 0; i < M * K; ++i) w[i] = i / K == 1 ? 0.0f : (float)uniform();
    check(qo_fp8_row_encode(M, K, w, b, r) == 0, "fp8 encode", M, K);
    check(r[1] == 0.0f, "fp8 all-zero row", M, K);
    for (int64_t i = 0; i < M * K; ++i) check((b[i] & 0x7F) != 0x7F, "fp8 no NaN byte", i, b[i]);
    check(qo_dequant_fp8(M, K, b, r, back) == 0, "fp8 dequant", M, K);
    w[M * K - 1] = INFINITY;
    check(qo_fp8_row_encode(M, K, w, b, r) == -2, "fp8 inf weight", M, K);
    b[M * K - 1] = 0x7F;
    check(qo_dequant_fp8(M, K, b, r, back) == -2, "fp8 NaN byte", M, K);
    free(back);
    free(r);
    free(b);
    free(w);
}

static void error_returns(void)
{
    int8_t c[64] = {0};
    uint16_t s[1] = {0x3C00};
    float w[64];
    double y[1];
    uint16_t x[64] = {0};
    check(qo_dequant_groupwise(7, 1, 64, c, s, w) == -1, "dequant bits", 7, 0);
    check(qo_dequant_groupwise(4, 1, 96, c, s, w) == -1, "dequant K % 64", 4, 96);
    c[63] = 8;
    check(qo_dequant_groupwise(4, 1, 64, c, s, w) == -2, "dequant code range", 4, 8);
    check(qo_gemv(7, 1, 64, 1, c, s, x, NULL, 1, y, NULL, 1) == -1, "gemv format", 7, 0);
    check(qo_gemv(4, 1, 64, 1, c, s, x, NULL, 2, y, NULL, 1) == -1, "gemv nrows != M", 4, 2);
    check(qo_gemv(4, 1, 64, 0, c, s, x, NULL, 1, y, NULL, 1) == 0, "gemv T = 0", 4, 0);
    check(qo_gemv(4, 1, 64, 1, c, s, x, NULL, 1, y, NULL, 1) == -2, "gemv code range", 4, 8);
}

/* With "--canary", hand qo_dequant_groupwise an output one float short: under AddressSanitizer
 * the run must abort, which shows the oracle code is instrumented. */
static int canary(void)
{
    int8_t c[128] = {0};
    uint16_t s[2] = {0x3C00, 0x3C00};
    float *w = (float *)malloc(sizeof(float) * 127);
    const int st = qo_dequant_groupwise(4, 1, 128, c, s, w);
    free(w);
    printf("canary: no sanitizer report (status %d)\n", st);
    return 0;
}

int main(int argc, char **argv)
{
    if (argc > 1 && strcmp(argv[1], "--canary") == 0)
        return canary();
    conversions();
    /* groupwise 4/5/6/8 and FP8; ragged row counts, K of one group up to several units */
    const int fmts[5] = {4, 5, 6, 9, 8};
    const int64_t shapes[3][3] = {{1, 64, 1}, {7, 192, 3}, {17, 320, 2}};
    for (int f = 0; f < 5; ++f)
        for (int i = 0; i < 3; ++i) products(fmts[f], shapes[i][0], shapes[i][1], shapes[i][2]);
    for (int bits = 4; bits <= 8; ++bits)
        if (bits != 7) encoders(bits, 5);
    fp8_encoder(5, 192);
    error_returns();
    if (failures) {
        printf("%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
