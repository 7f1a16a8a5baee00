// The packer of the qmat C ABI (host, pure): validated codes and scales into the tile layout the
// kernels stream (qmat_layout.h).  No HIP here.
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "../../include/qmat.h"
#include "qmat_host.h"
#include "qmat_layout.h"

using namespace qmatk;
using qmath::fail;
using qmath::ok;
using qmath::shape_ok;

namespace {

struct PackSrc {
    int fmt;
    int64_t M, K;
    const int8_t *codes;    // groupwise
    const uint8_t *bytes;   // FP8
    const uint16_t *hs;     // groupwise scales [M][K/64]
    const float *rs;        // FP8 row scales [M]
};

// code of (row, k) as the low b bits (two's complement) or the E4M3 byte; 0 outside the matrix
inline uint32_t code_at(const PackSrc &p, int64_t row, int64_t k)
{
    if (row >= p.M || k >= p.K) return 0;
    if (p.fmt == kFmtFp8) return p.bytes[row * p.K + k];
    return (uint32_t)(uint8_t)p.codes[row * p.K + k] & ((1u << group_code_bits(p.fmt)) - 1u);
}

void pack_tile(const PackSrc &p, int64_t tile, uint8_t *out)
{
    const int fmt = p.fmt, NB = blocks_per_unit(fmt);
    const int64_t NU = num_units(p.K), NT = num_tiles(p.M);
    uint8_t *codes = out;
    uint8_t *scales = out + code_bytes(fmt, p.M, p.K);
    for (int64_t u = 0; u < NU; ++u) {
        for (int L = 0; L < 64; ++L) {
            const int r16 = L & 15, q = L >> 4;
            auto c = [&](int m, int ka, int e) -> uint32_t {
                return code_at(p, tile * kTileRows + 16 * m + r16, u * kUnitK + 32 * ka + 8 * q + e);
            };
            uint32_t W[32];
            memset(W, 0, sizeof(W));
            for (int ka = 0; ka < 4; ++ka) {
                if (fmt == 4) {
                    // byte i: e = i in bits [3:0], e = 4 + i in bits [7:4], two's complement
                    for (int m = 0; m < 4; ++m) {
                        uint32_t n = 0;
                        for (int i = 0; i < 4; ++i) n |= (c(m, ka, i) | (c(m, ka, 4 + i) << 4)) << (8 * i);
                        W[4 * ka + m] = n;
                    }
                } else if (fmt == 5) {
                    // output dword o: row o/2, e = 4*(o%2) + i in byte i, stored as code << 3
                    auto oc = [&](int o, int i) { return c(o >> 1, ka, 4 * (o & 1) + i); };
                    uint32_t E = 0;
                    for (int d = 0; d < 4; ++d) {
                        uint32_t X = 0;
                        for (int i = 0; i < 4; ++i) {
                            const uint32_t main = oc(d, i), extra = oc(4 + d, i);
                            X |= ((main << 3) | (extra >> 2)) << (8 * i);
                            E |= (extra & 3u) << (8 * i + 2 * d);
                        }
                        W[5 * ka + d] = X;
                    }
                    W[5 * ka + 4] = E;
                } else if (fmt == 6) {
                    for (int pp = 0; pp < 2; ++pp) {
                        const int m0 = 2 * pp, m1 = m0 + 1;
                        uint32_t A = 0, B = 0, C = 0;
                        for (int i = 0; i < 4; ++i) {
                            const uint32_t x3 = c(m1, ka, 4 + i);
                            A |= ((c(m0, ka, i) << 2) | ((x3 >> 4) & 3u)) << (8 * i);
                            B |= ((c(m0, ka, 4 + i) << 2) | ((x3 >> 2) & 3u)) << (8 * i);
                            C |= ((c(m1, ka, i) << 2) | (x3 & 3u)) << (8 * i);
                        }
                        W[6 * ka + 3 * pp + 0] = A;
                        W[6 * ka + 3 * pp + 1] = B;
                        W[6 * ka + 3 * pp + 2] = C;
                    }
                } else {  // FP8 bytes, or Q8 codes as bytes
                    for (int m = 0; m < 4; ++m)
                        for (int h = 0; h < 2; ++h) {
                            uint32_t w = 0;
                            for (int i = 0; i < 4; ++i) w |= c(m, ka, 4 * h + i) << (8 * i);
                            W[8 * ka + 2 * m + h] = w;
                        }
                }
            }
            for (int j = 0; j < NB; ++j)
                memcpy(codes + ((tile * NU + u) * NB + j) * kBlockBytes + 16 * L, &W[4 * j], 16);
        }
        if (fmt != kFmtFp8) {
            const int64_t G = p.K / kGroup;
            uint16_t *sb = reinterpret_cast<uint16_t *>(scales + (tile * NU + u) * kScaleBlockBytes);
            for (int r16 = 0; r16 < 16; ++r16)
                for (int g = 0; g < 2; ++g)
                    for (int m = 0; m < 4; ++m) {
                        const int64_t row = tile * kTileRows + 16 * m + r16, grp = 2 * u + g;
                        sb[r16 * 8 + 4 * g + m] = (row < p.M && grp < G) ? p.hs[row * G + grp] : 0;
                    }
        }
    }
    if (fmt == kFmtFp8) {
        float *sb = reinterpret_cast<float *>(scales + tile * kScaleBlockBytes);
        for (int r16 = 0; r16 < 16; ++r16)
            for (int m = 0; m < 4; ++m) {
                const int64_t row = tile * kTileRows + 16 * m + r16;
                sb[r16 * 4 + m] = row < p.M ? p.rs[row] : 0.0f;
            }
    }
    (void)NT;
}

}  // namespace

extern "C" {

size_t qmat_packed_bytes(int fmt, int64_t M, int64_t K)
{
    if (!format_ok(fmt) || !shape_ok(M, K)) return 0;
    return code_bytes(fmt, M, K) + scale_bytes(fmt, M, K);
}

int qmat_pack(int fmt, int64_t M, int64_t K, const void *codes, const void *scales, void *out, size_t out_bytes)
{
    if (!format_ok(fmt)) return fail(QMAT_EINVAL, "qmat_pack: unknown format %d", fmt);
    if (!shape_ok(M, K)) return fail(QMAT_ESHAPE, "qmat_pack: bad shape M=%lld K=%lld (K must be a positive multiple of 64)", (long long)M, (long long)K);
    if (!codes || !scales || !out) return fail(QMAT_EINVAL, "qmat_pack: null pointer");
    const size_t need = qmat_packed_bytes(fmt, M, K);
    if (out_bytes < need) return fail(QMAT_ESIZE, "qmat_pack: out_bytes %zu < %zu", out_bytes, need);
    PackSrc p{fmt, M, K, nullptr, nullptr, nullptr, nullptr};
    if (fmt == kFmtFp8) {
        p.bytes = static_cast<const uint8_t *>(codes);
        p.rs = static_cast<const float *>(scales);
        for (int64_t i = 0; i < M * K; ++i)
            if ((p.bytes[i] & 0x7F) == 0x7F)
                return fail(QMAT_ERANGE, "qmat_pack: NaN E4M3 byte 0x%02x at row %lld col %lld", p.bytes[i], (long long)(i / K), (long long)(i % K));
        for (int64_t i = 0; i < M; ++i)
            if (!std::isfinite(p.rs[i])) return fail(QMAT_ERANGE, "qmat_pack: non-finite row scale at row %lld", (long long)i);
    } else {
        p.codes = static_cast<const int8_t *>(codes);
        p.hs = static_cast<const uint16_t *>(scales);
        const int bits = group_code_bits(fmt);
        const int lo = -(1 << (bits - 1)), hi = (1 << (bits - 1)) - 1;
        for (int64_t i = 0; i < M * K; ++i)
            if (p.codes[i] < lo || p.codes[i] > hi)
                return fail(QMAT_ERANGE, "qmat_pack: code %d outside [%d,%d] at row %lld col %lld", p.codes[i], lo, hi, (long long)(i / K), (long long)(i % K));
        const int64_t G = K / kGroup;
        for (int64_t i = 0; i < M * G; ++i)
            if ((p.hs[i] & 0x7C00) == 0x7C00)
                return fail(QMAT_ERANGE, "qmat_pack: non-finite FP16 scale 0x%04x at row %lld group %lld", p.hs[i], (long long)(i / G), (long long)(i % G));
    }
    uint8_t *o = static_cast<uint8_t *>(out);
    const int64_t NT = num_tiles(M);
    const unsigned nth = qmath::host_threads(NT);
    auto work = [&](unsigned k) {
        for (int64_t t = (int64_t)k; t < NT; t += nth) pack_tile(p, t, o);
    };
    if (nth == 1) {
        work(0);
    } else {
        std::vector<std::thread> th;
        try {
            for (unsigned k = 1; k < nth; ++k) th.emplace_back(work, k);
        } catch (...) {
            for (auto &t : th) t.join();
            return fail(QMAT_ENOMEM, "qmat_pack: could not start threads");
        }
        work(0);
        for (auto &t : th) t.join();
    }
    return ok();
}

}  // extern "C"
