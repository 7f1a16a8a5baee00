/*
 * CPU oracle for the weight-only quantized matrix-activation product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header, table or constant with the GPU
 * library: it works on the logical (unpacked) arrays and never sees the packed
 * layout.
 *
 * Everything is plain and slow on purpose: scalar decoders written from the IEEE
 * and OCP definitions, products and sums in double precision in index order.
 *
 * What it computes (sources: the NInfer model cards):
 *  - Groupwise Qb weights ("Qwen3.8-27B for NInfer on the RTX 3090", section
 *    "What is different from the upstream artifact"): each run of 64 weights
 *    along a row has one FP16 scale; a weight is scale times a two's-complement
 *    code; a negative scale is legal (it lets a group map a positive largest weight to
 *    -2^(b-1): -8 for 4 bits, -16 for 5 bits).  The upstream encoder there picks
 *    scale = absmax / qmax and the nearest code.  The same cards store the token
 *    embedding, the upstream output head and several projections as groupwise Q8
 *    (the "Token embedding / output head" and "Attention ... projections" rows of
 *    their format tables); here that is the same definition with 8-bit codes.
 *  - Row-scaled FP8 weights ("Qwen3.8-27B NVFP4 for NInfer", introduction and
 *    "Artifact"): one scale per matrix row times an FP8 value.  The FP8 variant
 *    is OCP E4M3 (finite-only, bias 7) and the row scale is an IEEE fp32 value.
 *  - The product y[t][i] = sum_j w[i][j] * x[t][j] with bf16 activations.
 *
 * Precision: every decoded value is exact in double.  A groupwise weight times a
 * bf16 activation has at most 11+6+8 significant bits, an FP8 weight
 * (fp32 scale * E4M3 value) times an activation at most 24+4+8, so every term is
 * exact in double and the only error of y is the summation (<= K * 2^-53 * A
 * with A = sum_j |w x|).
 *
 * Parity pins for every function live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QO_OK 0
#define QO_EINVAL (-1)
#define QO_ERANGE (-2)

/* ---------------------------------------------------------------- decoders */

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double qo_half_to_double(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return s ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double qo_bf16_to_double(uint16_t b)
{
    int s = b >> 15, e = (b >> 7) & 0xff, m = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133); /* subnormal: m * 2^-7 * 2^-126 */
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + m), e - 134); /* (1 + m/128) * 2^(e-127) */
    return s ? -v : v;
}

/* OCP 8-bit floating point, E4M3 ("FN": no infinities; S.1111.111 is NaN). */
double qo_e4m3_to_double(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 0xf, m = b & 7;
    double v;
    if ((b & 0x7f) == 0x7f)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9); /* subnormal: (m/8) * 2^-6 */
    else
        v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* double -> binary16, round to nearest, ties to even; overflow -> infinity. */
uint16_t qo_double_to_half_rne(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7e00;
    if (a >= 65520.0) /* halfway between 65504 and 2^16 rounds to even, i.e. up */
        return sign | 0x7c00;
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1; /* a in [2^E, 2^(E+1)) */
    if (E < -14) {
        /* subnormal range: the quantum is 2^-24; q == 1024 is the smallest normal */
        double q = rint(ldexp(a, 24));
        return sign | (uint16_t)q;
    }
    double q = rint(ldexp(a, 10 - E)); /* in [1024, 2048] */
    if (q == 2048.0) {
        q = 1024.0;
        E += 1;
    }
    if (E > 15)
        return sign | 0x7c00;
    return sign | (uint16_t)(((E + 15) << 10) | ((int)q - 1024));
}

/* ---------------------------------------------------------------- helpers */

static int code_in_range(int bits, int c)
{
    return c >= -(1 << (bits - 1)) && c <= (1 << (bits - 1)) - 1;
}

static int bits_ok(int bits) { return bits == 4 || bits == 5 || bits == 6 || bits == 8; }

/* Format ids of qo_gemv: 4, 5, 6 groupwise with that many bits; 9 groupwise 8-bit;
 * 8 row-scaled FP8.  Returns the code width of a groupwise format, 0 otherwise. */
static int group_bits(int fmt)
{
    return (fmt == 4 || fmt == 5 || fmt == 6) ? fmt : fmt == 9 ? 8 : 0;
}

/* ---------------------------------------------------------------- dequant */

/* w[i][j] = fp32(scale[i][j/64]) * code[i][j].  The product has at most
 * 11 + 6 significant bits, so it is exact in fp32: computed in double, then
 * converted (the conversion is exact, and keeps the sign of zero). */
int qo_dequant_groupwise(int bits, int64_t M, int64_t K, const int8_t *codes,
                         const uint16_t *scales, float *w)
{
    if (!bits_ok(bits) || M < 0 || K <= 0 || K % 64)
        return QO_EINVAL;
    int64_t G = K / 64;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < K; ++j) {
            int c = codes[i * K + j];
            if (!code_in_range(bits, c))
                return QO_ERANGE;
            double s = qo_half_to_double(scales[i * G + j / 64]);
            w[i * K + j] = (float)(s * (double)c);
        }
    return QO_OK;
}

/* w[i][j] = fl32(r[i] * e4m3(b[i][j])): the exact product (24 + 4 bits, exact in
 * double) rounded once to fp32, nearest-even. */
int qo_dequant_fp8(int64_t M, int64_t K, const uint8_t *bytes, const float *r, float *w)
{
    if (M < 0 || K <= 0)
        return QO_EINVAL;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < K; ++j) {
            uint8_t b = bytes[i * K + j];
            if ((b & 0x7f) == 0x7f)
                return QO_ERANGE;
            w[i * K + j] = (float)((double)r[i] * qo_e4m3_to_double(b));
        }
    return QO_OK;
}

/* ---------------------------------------------------------------- product */

typedef struct {
    int fmt; /* 4, 5, 6, 9 groupwise; 8 FP8 rows */
    int64_t M, K, T;
    const void *codes;
    const void *scales;
    const uint16_t *x;
    const int64_t *rows; /* NULL: all rows */
    int64_t nrows;
    double *y, *A; /* [T][nrows] */
    int64_t r0, r1;
    int status;
} job_t;

static void *gemv_worker(void *arg)
{
    job_t *jb = (job_t *)arg;
    int64_t K = jb->K, G = K / 64, T = jb->T;
    double *wrow = (double *)malloc(sizeof(double) * (size_t)K);
    double *xd = (double *)malloc(sizeof(double) * (size_t)(K * T));
    if (!wrow || !xd) {
        jb->status = QO_EINVAL;
        free(wrow);
        free(xd);
        return NULL;
    }
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < K; ++j)
            xd[t * K + j] = qo_bf16_to_double(jb->x[t * K + j]);
    for (int64_t n = jb->r0; n < jb->r1; ++n) {
        int64_t i = jb->rows ? jb->rows[n] : n;
        if (i < 0 || i >= jb->M) {
            jb->status = QO_EINVAL;
            break;
        }
        /* exact dequantized row in double */
        if (jb->fmt == 8) {
            const uint8_t *b = (const uint8_t *)jb->codes + i * K;
            double r = (double)((const float *)jb->scales)[i];
            for (int64_t j = 0; j < K; ++j) {
                if ((b[j] & 0x7f) == 0x7f) {
                    jb->status = QO_ERANGE;
                    goto done;
                }
                wrow[j] = r * qo_e4m3_to_double(b[j]);
            }
        } else {
            const int8_t *c = (const int8_t *)jb->codes + i * K;
            const uint16_t *s = (const uint16_t *)jb->scales + i * G;
            const int bits = group_bits(jb->fmt);
            for (int64_t j = 0; j < K; ++j) {
                if (!code_in_range(bits, c[j])) {
                    jb->status = QO_ERANGE;
                    goto done;
                }
                wrow[j] = qo_half_to_double(s[j / 64]) * (double)c[j];
            }
        }
        for (int64_t t = 0; t < T; ++t) {
            const double *xt = xd + t * K;
            double acc = 0.0, aabs = 0.0;
            for (int64_t j = 0; j < K; ++j) {
                double p = wrow[j] * xt[j];
                acc += p;
                aabs += fabs(p);
            }
            jb->y[t * jb->nrows + n] = acc;
            if (jb->A)
                jb->A[t * jb->nrows + n] = aabs;
        }
    }
done:
    free(wrow);
    free(xd);
    return NULL;
}

/* y[t][n] = sum_j w[rows[n]][j] * x[t][j] and A[t][n] = sum_j |w x|, in double,
 * sequential over j.  fmt 4/5/6/9 (groupwise 4, 5, 6, 8 bits): codes int8 [M][K],
 * scales binary16 [M][K/64]; fmt 8: codes E4M3 bytes [M][K], scales float [M].
 * x: bf16 bits [T][K].  rows == NULL means every row (nrows must equal M).  A may be
 * NULL. */
int qo_gemv(int fmt, int64_t M, int64_t K, int64_t T, const void *codes, const void *scales,
            const uint16_t *x, const int64_t *rows, int64_t nrows, double *y, double *A,
            int nthreads)
{
    if (!(group_bits(fmt) || fmt == 8) || M < 0 || K <= 0 || K % 64 || T < 0 || nrows < 0)
        return QO_EINVAL;
    if (!rows && nrows != M)
        return QO_EINVAL;
    if (nrows == 0 || T == 0)
        return QO_OK;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > nrows)
        nthreads = (int)nrows;
    job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return QO_EINVAL;
    }
    for (int k = 0; k < nthreads; ++k) {
        job_t *jb = &jobs[k];
        jb->fmt = fmt;
        jb->M = M;
        jb->K = K;
        jb->T = T;
        jb->codes = codes;
        jb->scales = scales;
        jb->x = x;
        jb->rows = rows;
        jb->nrows = nrows;
        jb->y = y;
        jb->A = A;
        jb->r0 = nrows * k / nthreads;
        jb->r1 = nrows * (k + 1) / nthreads;
        jb->status = QO_OK;
    }
    for (int k = 1; k < nthreads; ++k)
        pthread_create(&th[k], NULL, gemv_worker, &jobs[k]);
    gemv_worker(&jobs[0]);
    for (int k = 1; k < nthreads; ++k)
        pthread_join(th[k], NULL);
    int st = QO_OK;
    for (int k = 0; k < nthreads; ++k)
        if (jobs[k].status != QO_OK)
            st = jobs[k].status;
    free(jobs);
    free(th);
    return st;
}

/* ---------------------------------------------------------------- encoder */

/* Round-to-nearest groupwise encoder, as the upstream artifact describes it
 * ("Qwen3.8-27B for NInfer on the RTX 3090", "What is different from the
 * upstream artifact"): per 64-weight group, a = max |w|, scale = a / qmax
 * (qmax = 2^(b-1) - 1) stored as FP16, and each code is the nearest integer to
 * w / scale.  Readings where the page is silent: a / qmax is formed in double
 * and rounded once to FP16 (nearest-even); codes are taken against the stored
 * FP16 scale, rounded half-to-even, then clamped to [-2^(b-1), qmax]; an
 * all-zero group gets scale +0 and codes 0.  Returns QO_ERANGE if a / qmax
 * overflows FP16.  w: [ngroups][64] doubles. */
int qo_rtn_encode(int bits, int64_t ngroups, const double *w, int8_t *codes, uint16_t *scales)
{
    if (!bits_ok(bits) || ngroups < 0)
        return QO_EINVAL;
    const int qmax = (1 << (bits - 1)) - 1, qmin = -(1 << (bits - 1));
    for (int64_t g = 0; g < ngroups; ++g) {
        const double *wg = w + g * 64;
        double a = 0.0;
        for (int j = 0; j < 64; ++j) {
            if (!isfinite(wg[j]))
                return QO_ERANGE;
            if (fabs(wg[j]) > a)
                a = fabs(wg[j]);
        }
        uint16_t sb = qo_double_to_half_rne(a / (double)qmax);
        if ((sb & 0x7c00) == 0x7c00)
            return QO_ERANGE;
        scales[g] = sb;
        double s = qo_half_to_double(sb);
        for (int j = 0; j < 64; ++j) {
            double q = (s == 0.0) ? 0.0 : rint(wg[j] / s);
            if (q > qmax)
                q = qmax;
            if (q < qmin)
                q = qmin;
            codes[g * 64 + j] = (int8_t)q;
        }
    }
    return QO_OK;
}

/* ---------------------------------------------------------------- grouped search encoder */

/* The "grouped_search" encoder of "Qwen3.8-27B for NInfer on the RTX 3090" ("What is
 * different from the upstream artifact").  For each 64-weight group a fixed set of 50 FP16
 * scales is tried, and the kept one minimises E(s) = sum_j h_j (w_j - s c_j)^2, c_j being w_j/s
 * rounded and clamped to the code range and h_j >= 0 a per-input-channel weight (the page
 * derives it from the channel's mean squared activation).  The set holds both signs of every
 * magnitude, so that a group whose largest weight is positive can
 * map it to -2^(b-1), the code without a positive twin.
 *
 * The page does not list the candidates.  Reading: with a = max_j |w_j|, the 25 magnitudes
 * a / (qmax + i/24), i = 0..24, run from upstream's a/qmax (the group's largest weight lands
 * on +-qmax) to a/2^(b-1) (it lands on +-2^(b-1), the full range), each with both signs:
 * candidate order +m_0, -m_0, +m_1, -m_1, ...  Each candidate is rounded once to FP16
 * (nearest-even), codes are the nearest integers to w/s (half to even) clamped to the code
 * range, the error is evaluated in double in index order, and the first candidate with the
 * smallest error wins.  An all-zero group gets scale +0 and codes 0; QO_ERANGE if a/qmax
 * overflows FP16.  w and h: [ngroups][64] doubles (h >= 0). */
int qo_grouped_search_encode(int bits, int64_t ngroups, const double *w, const double *h, int8_t *codes,
                             uint16_t *scales)
{
    if (!bits_ok(bits) || ngroups < 0)
        return QO_EINVAL;
    const int qmax = (1 << (bits - 1)) - 1, qmin = -(1 << (bits - 1));
    for (int64_t g = 0; g < ngroups; ++g) {
        const double *wg = w + g * 64, *hg = h + g * 64;
        double a = 0.0;
        for (int j = 0; j < 64; ++j) {
            if (!isfinite(wg[j]) || !isfinite(hg[j]) || hg[j] < 0)
                return QO_ERANGE;
            if (fabs(wg[j]) > a)
                a = fabs(wg[j]);
        }
        if (a == 0.0) {
            scales[g] = 0;
            for (int j = 0; j < 64; ++j)
                codes[g * 64 + j] = 0;
            continue;
        }
        if ((qo_double_to_half_rne(a / (double)qmax) & 0x7c00) == 0x7c00)
            return QO_ERANGE;
        double best_err = INFINITY;
        uint16_t best_sb = 0;
        int8_t best_c[64];
        for (int cand = 0; cand < 50; ++cand) {
            const int i = cand / 2;
            const double mag = a / ((double)qmax + (double)i / 24.0);
            const uint16_t sb = qo_double_to_half_rne(cand % 2 ? -mag : mag);
            const double s = qo_half_to_double(sb);
            int8_t c[64];
            double err = 0.0;
            for (int j = 0; j < 64; ++j) {
                double q = (s == 0.0) ? 0.0 : rint(wg[j] / s);
                if (q > qmax)
                    q = qmax;
                if (q < qmin)
                    q = qmin;
                c[j] = (int8_t)q;
                const double d = wg[j] - s * q;
                err += hg[j] * (d * d);
            }
            if (err < best_err) {
                best_err = err;
                best_sb = sb;
                memcpy(best_c, c, sizeof(c));
            }
        }
        scales[g] = best_sb;
        memcpy(codes + g * 64, best_c, sizeof(best_c));
    }
    return QO_OK;
}

/* ---------------------------------------------------------------- row-scaled FP8 encoder */

/* float -> OCP E4M3 byte, round to nearest even, saturating at +-448 (the FN variant has no
 * infinity; NaN input is not allowed).  Subnormals (exponent field 0) have quantum 2^-9. */
uint8_t qo_float_to_e4m3_rne_sat(float q)
{
    uint8_t sign = signbit(q) ? 0x80 : 0;
    double a = fabs((double)q);
    if (a >= 448.0)
        return sign | 0x7e;
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2); /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    if (E < -6) {
        double n = rint(ldexp(a, 9)); /* multiples of 2^-9; 8 is the smallest normal */
        return sign | (uint8_t)n;
    }
    double n = rint(ldexp(a, 3 - E)); /* in [8, 16] */
    if (n == 16.0) {
        n = 8.0;
        E += 1;
    }
    if (E > 8 || (E == 8 && n > 14.0))
        return sign | 0x7e; /* beyond 448 after rounding */
    return sign | (uint8_t)(((E + 7) << 3) | ((int)n - 8));
}

/* Row-scaled FP8 encoding ("Qwen3.8-27B NVFP4 for NInfer", "Artifact": a tensor encoded
 * locally as row-scaled FP8; the method is not given).  Reading: r = fl32(a / 448) with a the
 * row's largest |w|, each byte the nearest E4M3 value (even ties, saturating) to fl32(w / r);
 * an all-zero row gets r = 0 and zero bytes.  w: float [M][K]. */
int qo_fp8_row_encode(int64_t M, int64_t K, const float *w, uint8_t *bytes, float *r)
{
    if (M < 0 || K <= 0)
        return QO_EINVAL;
    for (int64_t i = 0; i < M; ++i) {
        float a = 0.0f;
        for (int64_t j = 0; j < K; ++j) {
            if (!isfinite(w[i * K + j]))
                return QO_ERANGE;
            if (fabsf(w[i * K + j]) > a)
                a = fabsf(w[i * K + j]);
        }
        const float ri = (float)((double)a / 448.0);
        r[i] = ri;
        for (int64_t j = 0; j < K; ++j) {
            if (ri == 0.0f) {
                bytes[i * K + j] = 0;
                continue;
            }
            const float q = w[i * K + j] / ri;
            bytes[i * K + j] = qo_float_to_e4m3_rne_sat(q);
        }
    }
    return QO_OK;
}
