// Host encoders of the qmat C ABI: fp32 weights -> the logical arrays qmat_pack takes.
//
//  - RTN (upstream's encoder, "Qwen3.8-27B for NInfer on the RTX 3090", "What is different from
//    the upstream artifact"): per 64-weight group, scale = max|w| / qmax stored as FP16, codes
//    the nearest integers to w / scale.
//  - Grouped search (the same section: that artifact's encoder): 50 FP16 scales are tried per
//    group and the one with the smallest E(s) = sum_j h_j (w_j - s c_j)^2 is kept, c_j the
//    rounded, clamped code of w_j / s and h_j >= 0 a weight per input channel.  Both signs of
//    each magnitude are tried (with a negative scale a group whose largest weight is positive
//    maps it to -2^(b-1), the code without a positive twin).
//    The magnitudes (the page does not list them) are a / (qmax + i/24), i = 0..24,
//    a = max|w|: from upstream's a/qmax to the full range a/2^(b-1), tried in the order
//    +m0, -m0, +m1, -m1, ...
//  - Row-scaled FP8 ("Qwen3.8-27B NVFP4 for NInfer", "Artifact": a tensor encoded locally as
//    row-scaled FP8): r = fl32(max|w| / 448), bytes the nearest E4M3 values (even ties,
//    saturating at +-448) to fl32(w / r).
// Rounding everywhere is to nearest, ties to even; the FP16 scale is rounded once from the
// double quotient, and codes are taken against the stored FP16 value and clamped to the range.
// An all-zero group (row) gets scale +0 and zero codes.
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "../../include/qmat.h"
#include "qmat_host.h"
#include "qmat_layout.h"

// the weighted errors are compared for exact ties: keep every product and sum separately rounded
#pragma clang fp contract(off)

using qmath::fail;
using qmath::ok;

namespace {

uint16_t half_bits(double v)
{
    const _Float16 h = (_Float16)v;  // IEEE nearest-even conversion (overflow -> infinity)
    uint16_t b;
    memcpy(&b, &h, 2);
    return b;
}

double half_value(uint16_t b)
{
    _Float16 h;
    memcpy(&h, &b, 2);
    return (double)h;
}

bool half_is_inf_or_nan(uint16_t b) { return (b & 0x7C00) == 0x7C00; }

// E4M3 (OCP, FN) byte nearest to q, ties to even, saturating at +-448; from the float's bits
uint8_t e4m3_from_float(float q)
{
    uint32_t u;
    memcpy(&u, &q, 4);
    const uint8_t sign = (u >> 24) & 0x80;
    u &= 0x7FFFFFFFu;
    if (u >= 0x43E00000u) return sign | 0x7E;  // |q| >= 448
    if (u < 0x00800000u) return sign;            // zero or an fp32 subnormal (< 2^-126)
    int E = (int)(u >> 23) - 127;
    const uint32_t mant = (u & 0x7FFFFFu) | 0x800000u;  // 1.f as a 24-bit integer
    if (E >= -6) {
        // 3 fraction bits: drop 20
        uint32_t r = mant >> 20;
        const uint32_t rem = mant & 0xFFFFFu;
        if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
        if (r == 16) {
            r = 8;
            ++E;
        }
        if (E > 8 || (E == 8 && r > 14)) return sign | 0x7E;
        return sign | (uint8_t)(((E + 7) << 3) | (int)(r - 8));
    }
    // E4M3 subnormals: n * 2^-9 with n = q * 2^9 = mant * 2^(E - 14)
    const int sh = 14 - E;  // >= 21
    if (sh >= 26) return sign;  // below 2^-10 (half the smallest subnormal): 0
    uint32_t r = mant >> sh;
    const uint32_t rem = mant & ((1u << sh) - 1u), half = 1u << (sh - 1);
    if (rem > half || (rem == half && (r & 1u))) ++r;
    return sign | (uint8_t)r;  // r == 8 is the smallest normal, 0x08
}

struct GroupJob {
    int bits, encoder;
    int64_t M, K;
    const float *w, *h;
    int8_t *codes;
    uint16_t *scales;
};

// one group of 64 weights of a row: returns 0, or QMAT_ERANGE
int encode_group(const GroupJob &jb, int64_t row, int64_t g)
{
    const int qmax = (1 << (jb.bits - 1)) - 1, qmin = -(1 << (jb.bits - 1));
    const float *w = jb.w + row * jb.K + g * 64;
    const float *h = jb.h ? jb.h + g * 64 : nullptr;
    int8_t *c = jb.codes + row * jb.K + g * 64;
    uint16_t &sb = jb.scales[row * (jb.K / 64) + g];
    double a = 0.0;
    for (int j = 0; j < 64; ++j) {
        if (!std::isfinite(w[j])) return QMAT_ERANGE;
        a = std::fmax(a, std::fabs((double)w[j]));
    }
    if (a == 0.0) {
        sb = 0;
        memset(c, 0, 64);
        return 0;
    }
    if (half_is_inf_or_nan(half_bits(a / (double)qmax))) return QMAT_ERANGE;
    auto codes_for = [&](double s, int8_t *out) {
        for (int j = 0; j < 64; ++j) {
            double q = s == 0.0 ? 0.0 : std::nearbyint((double)w[j] / s);
            q = q > qmax ? qmax : q < qmin ? qmin : q;
            out[j] = (int8_t)q;
        }
    };
    if (jb.encoder == QMAT_ENCODE_RTN) {
        sb = half_bits(a / (double)qmax);
        codes_for(half_value(sb), c);
        return 0;
    }
    double best = INFINITY;
    int8_t trial[64];
    for (int i = 0; i < 25; ++i) {
        const double mag = a / ((double)qmax + (double)i / 24.0);
        for (int neg = 0; neg < 2; ++neg) {
            const uint16_t cb = half_bits(neg ? -mag : mag);
            const double s = half_value(cb);
            codes_for(s, trial);
            double err = 0.0;
            for (int j = 0; j < 64; ++j) {
                const double d = (double)w[j] - s * (double)trial[j];
                err += (h ? (double)h[j] : 1.0) * (d * d);
            }
            if (err < best) {
                best = err;
                sb = cb;
                memcpy(c, trial, 64);
            }
        }
    }
    return 0;
}

template <typename F> int parallel_rows(int64_t M, F body)
{
    const unsigned nth = qmath::host_threads(M);
    std::vector<int> st(nth, 0);
    auto work = [&](unsigned k) {
        for (int64_t r = (int64_t)k; r < M && !st[k]; r += nth) st[k] = body(r);
    };
    std::vector<std::thread> th;
    try {
        for (unsigned k = 1; k < nth; ++k) th.emplace_back(work, k);
    } catch (...) {
        for (auto &t : th) t.join();
        return QMAT_ENOMEM;
    }
    work(0);
    for (auto &t : th) t.join();
    for (int s : st)
        if (s) return s;
    return 0;
}

}  // namespace

extern "C" int qmat_quantize(int fmt, int64_t M, int64_t K, const float *w, const float *importance, int encoder,
                             void *codes_out, void *scales_out)
{
    using namespace qmatk;
    if (!format_ok(fmt)) return fail(QMAT_EINVAL, "qmat_quantize: unknown format %d", fmt);
    if (!qmath::shape_ok(M, K))
        return fail(QMAT_ESHAPE, "qmat_quantize: bad shape M=%lld K=%lld", (long long)M, (long long)K);
    if (!w || !codes_out || !scales_out) return fail(QMAT_EINVAL, "qmat_quantize: null pointer");
    if (encoder != QMAT_ENCODE_RTN && encoder != QMAT_ENCODE_GROUPED_SEARCH)
        return fail(QMAT_EINVAL, "qmat_quantize: unknown encoder %d", encoder);
    if (fmt == kFmtFp8) {
        if (encoder != QMAT_ENCODE_RTN)
            return fail(QMAT_EINVAL, "qmat_quantize: row-scaled FP8 has only the row-max encoder (QMAT_ENCODE_RTN)");
        uint8_t *b = static_cast<uint8_t *>(codes_out);
        float *r = static_cast<float *>(scales_out);
        const int st = parallel_rows(M, [&](int64_t i) -> int {
            const float *wr = w + i * K;
            float a = 0.0f;
            for (int64_t j = 0; j < K; ++j) {
                if (!std::isfinite(wr[j])) return QMAT_ERANGE;
                a = std::fmax(a, std::fabs(wr[j]));
            }
            const float ri = (float)((double)a / 448.0);
            r[i] = ri;
            for (int64_t j = 0; j < K; ++j) b[i * K + j] = ri == 0.0f ? 0 : e4m3_from_float(wr[j] / ri);
            return 0;
        });
        if (st == QMAT_ERANGE) return fail(QMAT_ERANGE, "qmat_quantize: non-finite weight");
        if (st) return fail(st, "qmat_quantize: could not start threads");
        return ok();
    }
    if (importance) {
        if (encoder == QMAT_ENCODE_GROUPED_SEARCH)
            for (int64_t j = 0; j < K; ++j)
                if (!std::isfinite(importance[j]) || importance[j] < 0.0f)
                    return fail(QMAT_ERANGE, "qmat_quantize: importance[%lld] is negative or not finite", (long long)j);
    }
    GroupJob jb{group_code_bits(fmt), encoder, M, K, w, encoder == QMAT_ENCODE_GROUPED_SEARCH ? importance : nullptr,
                static_cast<int8_t *>(codes_out), static_cast<uint16_t *>(scales_out)};
    const int64_t G = K / 64;
    const int st = parallel_rows(M, [&](int64_t i) -> int {
        for (int64_t g = 0; g < G; ++g)
            if (int e = encode_group(jb, i, g)) return e;
        return 0;
    });
    if (st == QMAT_ERANGE)
        return fail(QMAT_ERANGE, "qmat_quantize: non-finite weight, or a group whose max|w|/qmax overflows FP16");
    if (st) return fail(st, "qmat_quantize: could not start threads");
    return ok();
}
