// Drives the HIP-free host sources of the library (qmat_host.cpp, qmat_pack.cpp,
// qmat_encode.cpp) under a host sanitizer: every format and encoder on ragged shapes, every
// documented error path, and concurrent callers.  Buffers are allocated at exactly the size
// the API documents, so a write or read past one is caught.  Exits 0 when every check holds;
// prints the failing check and exits 1 otherwise.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "../../include/qmat.h"

namespace {

int failures = 0;

void check(bool cond, const char *what, int fmt, int64_t M, int64_t K)
{
    if (!cond) {
        std::printf("FAIL %s (fmt %d, M %lld, K %lld): %s\n", what, fmt, (long long)M, (long long)K,
                    qmat_last_error());
        ++failures;
    }
}

// xorshift64*: the driver's own input draws
struct Rng {
    uint64_t s;
    uint64_t next()
    {
        s ^= s >> 12;
        s ^= s << 25;
        s ^= s >> 27;
        return s * 0x2545F4914F6CDD1DULL;
    }
    float uniform() { return (float)((next() >> 40) * (1.0 / 16777216.0)) * 2.0f - 1.0f; }
};

bool groupwise(int fmt) { return fmt == QMAT_Q4 || fmt == QMAT_Q5 || fmt == QMAT_Q6 || fmt == QMAT_Q8; }
int code_bits(int fmt) { return fmt == QMAT_Q8 ? 8 : fmt; }
size_t scale_bytes(int fmt, int64_t M, int64_t K) { return groupwise(fmt) ? (size_t)(M * (K / 64)) * 2 : (size_t)M * 4; }

// quantize (exact-size outputs), check the codes, pack twice into exact-size buffers filled
// with different bytes: equal results show a deterministic, complete write
void round_trip(int fmt, int64_t M, int64_t K, int encoder, bool with_importance, uint64_t seed)
{
    Rng rng{seed};
    float *w = (float *)std::malloc(sizeof(float) * M * K);
    for (int64_t i = 0; i < M * K; ++i) w[i] = rng.uniform() * (i % 97 == 0 ? 8.0f : 1.0f);
    for (int64_t j = 0; j < K && M > 1; ++j) w[K + j] = 0.0f;  // an all-zero row (and groups)
    float *imp = nullptr;
    if (with_importance) {
        imp = (float *)std::malloc(sizeof(float) * K);
        for (int64_t j = 0; j < K; ++j) imp[j] = j % 5 == 0 ? 0.0f : 1.0f + rng.uniform();
    }
    void *codes = std::malloc((size_t)(M * K));
    void *scales = std::malloc(scale_bytes(fmt, M, K));
    int st = qmat_quantize(fmt, M, K, w, imp, encoder, codes, scales);
    check(st == QMAT_OK, "qmat_quantize", fmt, M, K);
    if (st == QMAT_OK && groupwise(fmt)) {
        const int lo = -(1 << (code_bits(fmt) - 1)), hi = (1 << (code_bits(fmt) - 1)) - 1;
        bool in_range = true;
        for (int64_t i = 0; i < M * K; ++i) in_range &= ((int8_t *)codes)[i] >= lo && ((int8_t *)codes)[i] <= hi;
        check(in_range, "codes in range", fmt, M, K);
    }
    const size_t nb = qmat_packed_bytes(fmt, M, K);
    check(nb > 0, "qmat_packed_bytes", fmt, M, K);
    uint8_t *a = (uint8_t *)std::malloc(nb), *b = (uint8_t *)std::malloc(nb);
    std::memset(a, 0x00, nb);
    std::memset(b, 0xFF, nb);
    check(qmat_pack(fmt, M, K, codes, scales, a, nb) == QMAT_OK, "qmat_pack", fmt, M, K);
    check(qmat_pack(fmt, M, K, codes, scales, b, nb) == QMAT_OK, "qmat_pack again", fmt, M, K);
    check(std::memcmp(a, b, nb) == 0, "packed output fully written and deterministic", fmt, M, K);
    check(qmat_pack(fmt, M, K, codes, scales, a, nb - 1) == QMAT_ESIZE, "out_bytes one short", fmt, M, K);
    std::free(a);
    std::free(b);
    std::free(codes);
    std::free(scales);
    std::free(imp);
    std::free(w);
}

void error_paths()
{
    const int64_t M = 3, K = 128;
    std::vector<float> w(M * K, 0.5f), imp(K, 1.0f);
    std::vector<int8_t> codes(M * K, 0);
    std::vector<uint16_t> hs(M * (K / 64), 0x3C00);
    std::vector<float> rs(M, 1.0f);
    std::vector<uint8_t> out(qmat_packed_bytes(QMAT_Q8, M, K));
    const size_t nb4 = qmat_packed_bytes(QMAT_Q4, M, K);

    check(qmat_packed_bytes(7, M, K) == 0, "packed_bytes: unknown format", 7, M, K);
    check(qmat_packed_bytes(QMAT_Q4, 0, K) == 0, "packed_bytes: M = 0", 4, 0, K);
    check(qmat_packed_bytes(QMAT_Q4, M, 96) == 0, "packed_bytes: K % 64", 4, M, 96);
    check(qmat_packed_bytes(QMAT_Q4, M, 1 << 21) == 0, "packed_bytes: K too large", 4, M, 1 << 21);

    check(qmat_pack(7, M, K, codes.data(), hs.data(), out.data(), out.size()) == QMAT_EINVAL, "pack: format", 7, M, K);
    check(qmat_pack(QMAT_Q4, M, 32, codes.data(), hs.data(), out.data(), out.size()) == QMAT_ESHAPE, "pack: K < 64", 4, M, 32);
    check(qmat_pack(QMAT_Q4, -1, K, codes.data(), hs.data(), out.data(), out.size()) == QMAT_ESHAPE, "pack: M < 0", 4, -1, K);
    check(qmat_pack(QMAT_Q4, M, K, nullptr, hs.data(), out.data(), out.size()) == QMAT_EINVAL, "pack: null codes", 4, M, K);
    check(qmat_pack(QMAT_Q4, M, K, codes.data(), nullptr, out.data(), out.size()) == QMAT_EINVAL, "pack: null scales", 4, M, K);
    check(qmat_pack(QMAT_Q4, M, K, codes.data(), hs.data(), nullptr, out.size()) == QMAT_EINVAL, "pack: null out", 4, M, K);
    check(qmat_pack(QMAT_Q4, M, K, codes.data(), hs.data(), out.data(), nb4 - 1) == QMAT_ESIZE, "pack: short out", 4, M, K);
    codes[M * K - 1] = 8;  // one past Q4's largest code, at the last index
    check(qmat_pack(QMAT_Q4, M, K, codes.data(), hs.data(), out.data(), out.size()) == QMAT_ERANGE, "pack: Q4 code 8", 4, M, K);
    check(qmat_pack(QMAT_Q5, M, K, codes.data(), hs.data(), out.data(), out.size()) == QMAT_OK, "pack: Q5 code 8", 5, M, K);
    codes[M * K - 1] = -33;
    check(qmat_pack(QMAT_Q6, M, K, codes.data(), hs.data(), out.data(), out.size()) == QMAT_ERANGE, "pack: Q6 code -33", 6, M, K);
    codes[M * K - 1] = -128;
    check(qmat_pack(QMAT_Q8, M, K, codes.data(), hs.data(), out.data(), out.size()) == QMAT_OK, "pack: Q8 code -128", 9, M, K);
    codes[M * K - 1] = 0;
    hs.back() = 0x7C00;  // +infinity
    check(qmat_pack(QMAT_Q4, M, K, codes.data(), hs.data(), out.data(), out.size()) == QMAT_ERANGE, "pack: inf scale", 4, M, K);
    hs.back() = 0xFE00;  // a NaN
    check(qmat_pack(QMAT_Q4, M, K, codes.data(), hs.data(), out.data(), out.size()) == QMAT_ERANGE, "pack: NaN scale", 4, M, K);
    hs.back() = 0xBC00;  // -1: negative scales are allowed
    check(qmat_pack(QMAT_Q4, M, K, codes.data(), hs.data(), out.data(), out.size()) == QMAT_OK, "pack: negative scale", 4, M, K);
    std::vector<uint8_t> bytes(M * K, 0x38);
    bytes[M * K - 1] = 0xFF;
    check(qmat_pack(QMAT_FP8_E4M3_ROW, M, K, bytes.data(), rs.data(), out.data(), out.size()) == QMAT_ERANGE, "pack: NaN E4M3", 8, M, K);
    bytes[M * K - 1] = 0x7E;  // 448, the largest finite value
    check(qmat_pack(QMAT_FP8_E4M3_ROW, M, K, bytes.data(), rs.data(), out.data(), out.size()) == QMAT_OK, "pack: E4M3 448", 8, M, K);
    rs.back() = INFINITY;
    check(qmat_pack(QMAT_FP8_E4M3_ROW, M, K, bytes.data(), rs.data(), out.data(), out.size()) == QMAT_ERANGE, "pack: inf row scale", 8, M, K);

    check(qmat_quantize(7, M, K, w.data(), nullptr, 0, codes.data(), hs.data()) == QMAT_EINVAL, "quantize: format", 7, M, K);
    check(qmat_quantize(QMAT_Q4, 0, K, w.data(), nullptr, 0, codes.data(), hs.data()) == QMAT_ESHAPE, "quantize: M = 0", 4, 0, K);
    check(qmat_quantize(QMAT_Q4, M, 100, w.data(), nullptr, 0, codes.data(), hs.data()) == QMAT_ESHAPE, "quantize: K % 64", 4, M, 100);
    check(qmat_quantize(QMAT_Q4, M, K, nullptr, nullptr, 0, codes.data(), hs.data()) == QMAT_EINVAL, "quantize: null w", 4, M, K);
    check(qmat_quantize(QMAT_Q4, M, K, w.data(), nullptr, 0, nullptr, hs.data()) == QMAT_EINVAL, "quantize: null codes", 4, M, K);
    check(qmat_quantize(QMAT_Q4, M, K, w.data(), nullptr, 2, codes.data(), hs.data()) == QMAT_EINVAL, "quantize: encoder", 4, M, K);
    check(qmat_quantize(QMAT_FP8_E4M3_ROW, M, K, w.data(), nullptr, QMAT_ENCODE_GROUPED_SEARCH, bytes.data(), rs.data()) == QMAT_EINVAL,
          "quantize: FP8 grouped search", 8, M, K);
    imp[K - 1] = -1.0f;
    check(qmat_quantize(QMAT_Q5, M, K, w.data(), imp.data(), QMAT_ENCODE_GROUPED_SEARCH, codes.data(), hs.data()) == QMAT_ERANGE,
          "quantize: negative importance", 5, M, K);
    imp[K - 1] = NAN;
    check(qmat_quantize(QMAT_Q5, M, K, w.data(), imp.data(), QMAT_ENCODE_GROUPED_SEARCH, codes.data(), hs.data()) == QMAT_ERANGE,
          "quantize: NaN importance", 5, M, K);
    check(qmat_quantize(QMAT_Q5, M, K, w.data(), imp.data(), QMAT_ENCODE_RTN, codes.data(), hs.data()) == QMAT_OK,
          "quantize: RTN ignores importance", 5, M, K);
    w[M * K - 1] = INFINITY;
    check(qmat_quantize(QMAT_Q6, M, K, w.data(), nullptr, 0, codes.data(), hs.data()) == QMAT_ERANGE, "quantize: inf weight", 6, M, K);
    check(qmat_quantize(QMAT_FP8_E4M3_ROW, M, K, w.data(), nullptr, 0, bytes.data(), rs.data()) == QMAT_ERANGE, "quantize: FP8 inf weight", 8, M, K);
    w[M * K - 1] = 1.0e6f;  // 1e6 / 7 overflows FP16
    check(qmat_quantize(QMAT_Q4, M, K, w.data(), nullptr, 0, codes.data(), hs.data()) == QMAT_ERANGE, "quantize: FP16 overflow", 4, M, K);
    check(qmat_quantize(QMAT_Q8, M, K, w.data(), nullptr, 0, codes.data(), hs.data()) == QMAT_OK, "quantize: Q8 1e6 fits", 9, M, K);

    const char *e = qmat_last_error();
    check(e != nullptr, "last_error not null", 0, 0, 0);
}

// several threads quantize and pack at once (each also spawns the library's own workers); a
// failing call on one thread must not change another thread's error text
void concurrent_callers()
{
    std::vector<std::thread> th;
    std::vector<int> bad(4, 0);
    for (int t = 0; t < 4; ++t)
        th.emplace_back([t, &bad] {
            const int fmt = t == 3 ? QMAT_FP8_E4M3_ROW : 4 + t;
            const int64_t M = 70 + 13 * t, K = 192;
            std::vector<float> w(M * K);
            Rng rng{0x9E3779B97F4A7C15ULL + (uint64_t)t};
            for (auto &v : w) v = rng.uniform();
            std::vector<uint8_t> codes(M * K), scales(scale_bytes(fmt, M, K));
            std::vector<uint8_t> out(qmat_packed_bytes(fmt, M, K));
            for (int rep = 0; rep < 4; ++rep) {
                if (qmat_quantize(fmt, M, K, w.data(), nullptr, 0, codes.data(), scales.data()) != QMAT_OK) ++bad[t];
                if (qmat_pack(fmt, M, K, codes.data(), scales.data(), out.data(), out.size()) != QMAT_OK) ++bad[t];
                if (t == 0) {
                    qmat_pack(fmt, M, K, codes.data(), scales.data(), out.data(), 1);  // fails on this thread only
                    if (!std::strstr(qmat_last_error(), "out_bytes")) ++bad[t];
                }
            }
        });
    for (auto &x : th) x.join();
    for (int t = 0; t < 4; ++t) check(bad[t] == 0, "concurrent quantize + pack", t, 0, 0);
}

// With "--canary", misstate a buffer's size so that qmat_pack writes one byte past it: under
// AddressSanitizer the run must abort, which shows the library code is instrumented.
int canary()
{
    const int64_t M = 64, K = 128;
    std::vector<int8_t> codes(M * K, 1);
    std::vector<uint16_t> hs(M * (K / 64), 0x3C00);
    const size_t nb = qmat_packed_bytes(QMAT_Q4, M, K);
    uint8_t *out = (uint8_t *)std::malloc(nb - 1);
    const int st = qmat_pack(QMAT_Q4, M, K, codes.data(), hs.data(), out, nb);
    std::free(out);
    std::printf("canary: no sanitizer report (status %d)\n", st);
    return 0;
}

}  // namespace

int main(int argc, char **argv)
{
    if (argc > 1 && std::strcmp(argv[1], "--canary") == 0) return canary();
    const int fmts[] = {QMAT_Q4, QMAT_Q5, QMAT_Q6, QMAT_Q8, QMAT_FP8_E4M3_ROW};
    // one group; a partial tile; an exact tile with a half unit of K; a ragged second tile; and
    // several tiles and units with a half unit left over
    const int64_t shapes[][2] = {{1, 64}, {63, 128}, {64, 192}, {65, 320}, {130, 1088}};
    uint64_t seed = 1;
    for (int fmt : fmts)
        for (auto &s : shapes) {
            round_trip(fmt, s[0], s[1], QMAT_ENCODE_RTN, false, seed++);
            if (groupwise(fmt)) {
                round_trip(fmt, s[0], s[1], QMAT_ENCODE_GROUPED_SEARCH, false, seed++);
                round_trip(fmt, s[0], s[1], QMAT_ENCODE_GROUPED_SEARCH, true, seed++);
            }
        }
    error_paths();
    concurrent_callers();
    if (failures) {
        std::printf("%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("host driver: all checks passed\n");
    return 0;
}
