// gfx950 (CDNA4) prefill GEMM route of the weight-only quantized product y = x . W^T: T > 16
// tokens (any T >= 1 on request), matrix-core tiles of 64 tokens x 256 rows, the same exact
// code conversions as the small-T routes (qmat_device.h).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "qmat_device.h"
#include "qmat_gemm.h"
#include "qmat_kernels.h"
#include "qmat_layout.h"

namespace qmatk {

// Blocks [J0, J1) of a lane's unit slots, plus the scale slot with the last of them (a unit
// fetched in parts), as ordinary cached loads: on the GEMM route every token tile reads the
// same weights, and the workgroups that share them run together on one XCD, so they should
// stay in its L2.
template <int FMT, int J0, int J1, int NB, int XN>
__device__ __forceinline__ void load_weight_blocks(const RunArgs &a, int tile, int u, uint32_t lane,
                                                   Unit<NB, XN> &r)
{
    const int64_t tu = (int64_t)tile * a.NU + u;
    const char *cb = reinterpret_cast<const char *>(a.codes) + tu * (NB * kBlockBytes);
#pragma unroll
    for (int j = J0; j < J1; ++j)
        r.c[j] = *reinterpret_cast<const u32x4_t *>(cb + j * kBlockBytes + 16u * lane);
    if constexpr (FMT != 8 && J1 == NB) {
        const char *sb = reinterpret_cast<const char *>(a.scales) + tu * kScaleBlockBytes;
        r.sc = *reinterpret_cast<const u32x4_t *>(sb + 16u * (lane & 15));
    }
}

// ------------------------------------------------------------------ GEMM route (prefill, T > 16)

// Prefill-sized products: the weights are reused by many tokens, so the MFMA does most of the
// work and each unpacked weight fragment feeds kGemmTB / 16 matrix instructions.  A workgroup
// is 4 waves; wave w owns row tile 4 * rb + w (64 rows), the workgroup a tile of kGemmTB
// tokens.  Per 128-wide k unit the workgroup loads the token tile's activations straight from
// global memory into LDS (shared by its 4 waves, double-buffered, one barrier per unit) while
// each wave streams its tile's packed unit one unit ahead.  Per 64-group and 16-row slice m,
// two MFMAs sum code * x into P and the group scale enters once per (token, row):
// acc += scale * P (exact products, fp32 sums, as on the small-T routes; the signed operands,
// since removing Q4's offset would cost a subtraction per (token, row, group)).  Row-scaled FP8
// has no group scale: the MFMA
// accumulates straight into acc and the row scale is applied at the end.
//
// Two workgroups per CU (at most 256 vector registers per lane) so that one wave's unpack and
// scale arithmetic overlaps the other's matrix instructions and memory waits.
//
// Block order: the hardware deals workgroups to the 8 XCDs in turn (block b to XCD b mod 8).
// Each XCD is given a contiguous range of the work list, which is ordered in patches of 8 row
// blocks x 8 token tiles (then k splits), so the ~64 workgroups one XCD runs at the same time
// share 8 row blocks' weights and 8 token tiles' activations through its L2: a row block's
// weights are fetched once per 8 token tiles and a token tile's activations once per 8 row
// blocks (row-block-major order re-read the activations for every pair of row blocks, plain
// order re-read the weights on every XCD).
//
// Split-K (a.S > 1, when row blocks x token tiles fill the chip's workgroup slots badly):
// split sp takes units [NU sp / S, NU (sp+1) / S).  Split 0 writes its partial to y, split
// sp > 0 stores its 64 x kGemmTB partial tile per wave to workspace region sp - 1 (ntt *
// kGemmTB token rows x NT * 64 floats: no store needs a bounds test); a second kernel, ordered
// after this one on the stream, adds regions 0 .. S-2 to y in split order (deterministic).  The
// partials are megabytes here, so a second launch is cheaper than making them visible to other
// workgroups inside this kernel.
constexpr int kGemmTB = kGemmTokens;      // tokens per workgroup tile
constexpr int kXcds = 8;

template <int FMT>
__global__ __launch_bounds__(256, kGemmTB <= 64 ? 2 : 1) void gemm_kernel(RunArgs a, int nrb, int ntt)
{
    constexpr int NB = Fmt<FMT>::NB, NTB = kGemmTB / 16;
    constexpr int XP = kGemmTB * (kUnitK / 8) / 256;  // 16-byte activation pieces per thread and unit
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][kGemmTB * kUnitK];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // block -> (row block, token tile, k split)
    const int S = a.S;
    const int64_t total = (int64_t)nrb * ntt * S, grid = (int64_t)gridDim.x * gridDim.y;
    const int64_t b = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    const int xcd = (int)(b % kXcds);
    const int64_t per = grid / kXcds, extra = grid % kXcds;
    const int64_t wi = xcd * per + (xcd < extra ? xcd : extra) + b / kXcds;
    if (wi >= total) return;
    // the work list in patches of Pr row blocks x Pt token tiles (x S splits), patch rows
    // outermost: about one patch (64 workgroups) runs on an XCD at a time
    constexpr int Pt = 8, Pr = 8;
    const int64_t prow = (int64_t)Pr * ntt * S;
    const int pr = (int)(wi / prow);
    const int64_t r1 = wi - pr * prow;
    const int R = nrb - pr * Pr < Pr ? nrb - pr * Pr : Pr;  // row blocks in this patch row
    const int pt = (int)(r1 / ((int64_t)R * Pt * S));
    const int64_t r2 = r1 - (int64_t)pt * R * Pt * S;
    const int C = ntt - pt * Pt < Pt ? ntt - pt * Pt : Pt;  // token tiles in this patch
    const int ir = (int)(r2 / ((int64_t)C * S));
    const int64_t r3 = r2 - (int64_t)ir * C * S;
    const int it = (int)(r3 / S), sp = (int)(r3 - (int64_t)it * S);
    const int rb = pr * Pr + ir, tt = pt * Pt + it;
    const int u0 = (int)((int64_t)a.NU * sp / S), u1 = (int)((int64_t)a.NU * (sp + 1) / S);
    const int tile = 4 * rb + w;
    const bool has_tile = tile < a.NT;
    const int tok0 = tt * kGemmTB;

    // activations of unit u for the token tile: thread i stages 16-byte pieces i, i + 256, ...
    // of the kGemmTB x 128 block (token = piece / 16, k octet = piece % 16).  No zero fill:
    // token rows past T are read as row T - 1 (their outputs are never written), and columns
    // past K (the half unit of a K = 64 mod 128 matrix) are read inside the row, where they
    // meet the zero codes of the padding group (x is finite by contract).  The row offsets are
    // fixed for the whole kernel; a unit adds a wave-uniform column.
    // activations of unit u, loaded straight into LDS: wave instruction j of wave w fills LDS
    // pieces 256 j + 64 w + lane (16 bytes each, contiguous); piece p holds token p / 16 and
    // k octet (p % 16) ^ (token % 16), an XOR swizzle that keeps the fragment reads free of
    // bank conflicts without padding.
    const int lane16 = threadIdx.x & 15;
    int64_t xoff[XP];
    int xko[XP];
#pragma unroll
    for (int j = 0; j < XP; ++j) {
        const int tq = (threadIdx.x + 256 * j) >> 4;
        const int t = tok0 + tq;
        xko[j] = lane16 ^ (tq & 15);
        xoff[j] = (int64_t)(t < a.T ? t : a.T - 1) * a.K + 8 * xko[j];
    }
    auto x_dma = [&](int u, int buf) {
        const int kb = u * kUnitK;
#pragma unroll
        for (int j = 0; j < XP; ++j) {
            int64_t off = xoff[j] + kb;
            if (kb + kUnitK > a.K) {
                const int kc = kb + 8 * xko[j] < a.K ? kb : a.K - 8 - 8 * xko[j];
                off = xoff[j] + kc;
            }
            __builtin_amdgcn_global_load_lds(a.x + off, &xs[buf][(256 * j + 64 * w) * 8], 16, 0, 0);
        }
    };

    f32x4_t acc[4][NTB];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < NTB; ++n) acc[m][n] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    const int oct = lane >> 4, tl = lane & 15;

    // group g of a unit: A fragments from LDS, then per row slice m: unpack, 2 MFMAs per
    // token block, scale
    auto compute = [&](const Unit<NB, 1> &cur, const uint16_t *xb, auto gc) {
        constexpr int g = decltype(gc)::value;
        const uint32_t *W = reinterpret_cast<const uint32_t *>(cur.c);
        {
            bf16x8_t A[2][NTB];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int n = 0; n < NTB; ++n)
                    A[ks][n] = *reinterpret_cast<const bf16x8_t *>(
                        &xb[(16 * n + tl) * kUnitK + 8 * ((4 * (2 * g + ks) + oct) ^ tl)]);

#define QMAT_GEMM_SLICE(MM, G)                                                                          \
    {                                                                                                   \
        uint32_t b0[4], b1[4];                                                                          \
        bf16x8_signed<FMT, 2 * (G), MM>(W, b0);                                                         \
        bf16x8_signed<FMT, 2 * (G) + 1, MM>(W, b1);                                                     \
        const bf16x8_t B0 = __builtin_bit_cast(bf16x8_t, (u32x4_t){b0[0], b0[1], b0[2], b0[3]});        \
        const bf16x8_t B1 = __builtin_bit_cast(bf16x8_t, (u32x4_t){b1[0], b1[1], b1[2], b1[3]});        \
        if constexpr (FMT == 8) {                                                                       \
            _Pragma("unroll") for (int n = 0; n < NTB; ++n) {                                           \
                acc[MM][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0][n], B0, acc[MM][n], 0, 0, 0); \
                acc[MM][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1][n], B1, acc[MM][n], 0, 0, 0); \
            }                                                                                           \
        } else {                                                                                        \
            const float sf = group_scale(cur.sc, G, MM);                                                \
            _Pragma("unroll") for (int n = 0; n < NTB; ++n) {                                           \
                f32x4_t P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0][n], B0,                        \
                                                                    (f32x4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0); \
                P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1][n], B1, P, 0, 0, 0);                  \
                _Pragma("unroll") for (int i = 0; i < 4; ++i) acc[MM][n][i] = fmaf(sf, P[i], acc[MM][n][i]); \
            }                                                                                           \
        }                                                                                               \
    }
            if (g == 0) { QMAT_GEMM_SLICE(0, 0) QMAT_GEMM_SLICE(1, 0) QMAT_GEMM_SLICE(2, 0) QMAT_GEMM_SLICE(3, 0) }
            else { QMAT_GEMM_SLICE(0, 1) QMAT_GEMM_SLICE(1, 1) QMAT_GEMM_SLICE(2, 1) QMAT_GEMM_SLICE(3, 1) }
#undef QMAT_GEMM_SLICE
        }
    };

    // unit u: prefetch unit u + 1 (activations to registers, weights to nxt), compute u from
    // cur and LDS buffer u & 1, then stage the prefetched activations in the other buffer.
    // The loop is unrolled by two so that cur and nxt swap roles without register copies.
    // Q8 (8 KB units) fetches the second half of nxt only once group 0 of cur is done with
    // its half (group 0 reads blocks 0-3, group 1 blocks 4-7), keeping 1.5 units live.
    constexpr bool kHalves = FMT == 9;
    auto step = [&](int u, Unit<NB, 1> &cur, Unit<NB, 1> &nxt) {
        const int buf = (u - u0) & 1;
        const bool more = u + 1 < u1;
        if (more) {
            x_dma(u + 1, buf ^ 1);
            if (has_tile) load_weight_blocks<FMT, 0, kHalves ? NB / 2 : NB>(a, tile, u + 1, lane, nxt);
        }
        if (has_tile) {
            compute(cur, xs[buf], std::integral_constant<int, 0>());
            if constexpr (kHalves)
                if (more) load_weight_blocks<FMT, NB / 2, NB>(a, tile, u + 1, lane, nxt);
            compute(cur, xs[buf], std::integral_constant<int, 1>());
        }
        __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this wave's activation loads are in LDS
        __syncthreads();
    };

    Unit<NB, 1> wa, wb;
    x_dma(u0, 0);
    if (has_tile) load_weight_blocks<FMT, 0, NB>(a, tile, u0, lane, wa);
    __builtin_amdgcn_s_waitcnt(0xF70);
    __syncthreads();
    for (int u = u0; u < u1; u += 2) {
        step(u, wa, wb);
        if (u + 1 < u1) step(u + 1, wb, wa);
    }
    if (!has_tile) return;
    constexpr float kF = Fmt<FMT>::kSignedToCode;
    f32x4_t rs = (f32x4_t){kF, kF, kF, kF};
    if constexpr (FMT == 8) rs = reinterpret_cast<const f32x4_t *>(a.scales)[(int64_t)tile * 16 + tl];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < NTB; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[m][n][i] *= rs[m];
    // D[m][n]: lane holds tokens 16n + 4 * oct + i of row 16m + tl
    if (sp == 0) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int row = tile * kTileRows + 16 * m + tl;
            if (row >= a.M) continue;
#pragma unroll
            for (int n = 0; n < NTB; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = tok0 + 16 * n + 4 * oct + i;
                    if (t < a.T) a.y[(int64_t)t * a.ldy + row] = acc[m][n][i];
                }
        }
        return;
    }
    const int64_t ld = (int64_t)a.NT * kTileRows;  // workspace row stride (padded M)
    float *wsp = a.ws + ((int64_t)(sp - 1) * ntt * kGemmTB + tok0) * ld + tile * kTileRows + tl;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < NTB; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) wsp[(int64_t)(16 * n + 4 * oct + i) * ld + 16 * m] = acc[m][n][i];
}

// y[t][r] += ws[0][t][r] + ... + ws[S-2][t][r], added one partial at a time in split order.
// One thread per (token, 4 consecutive padded rows): 16-byte partial loads, up to eight
// partials in flight at a time.
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float *__restrict__ ws, float *__restrict__ y,
                                                         int T, int M, int ldy, int64_t ld, int64_t tpad, int S)
{
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, per_t = ld / 4;
    if (q >= (int64_t)T * per_t) return;
    const int t = (int)(q / per_t);
    const int r = 4 * (int)(q - (int64_t)t * per_t);
    if (r >= M) return;
    float *yr = y + (int64_t)t * ldy + r;
    f32x4_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = r + e < M ? yr[e] : 0.0f;
    const f32x4_t *p = reinterpret_cast<const f32x4_t *>(ws + (int64_t)t * ld + r);
    const int64_t step = tpad * ld / 4;  // one split region, in float4
    const int n = S - 1;
    for (int s0 = 0; s0 < n; s0 += 8) {
        f32x4_t b[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = p[(int64_t)(s0 + j < n ? s0 + j : n - 1) * step];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (s0 + j < n) v += b[j];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (r + e < M) yr[e] = v[e];
}

// ------------------------------------------------------------------ launcher

template <int FMT> static const void *gemm_kernel_ptr() { return reinterpret_cast<const void *>(&gemm_kernel<FMT>); }

hipError_t launch_gemm(int fmt, const RunArgs &a, hipStream_t st)
{
    const void *k = fmt == 4 ? gemm_kernel_ptr<4>() : fmt == 5 ? gemm_kernel_ptr<5>()
                  : fmt == 6 ? gemm_kernel_ptr<6>() : fmt == 8 ? gemm_kernel_ptr<8>()
                  : fmt == 9 ? gemm_kernel_ptr<9>() : nullptr;
    if (!k) return hipErrorInvalidValue;
    RunArgs arg = a;
    int nrb = gemm_row_blocks(a.NT), ntt = gemm_token_tiles(a.T);
    // a 1-D grid while it fits the dispatch limits, else rows of 2^23 blocks (the last row
    // partly idle); either way a multiple of 8 blocks per row keeps b mod 8 the XCD
    const int64_t total = (int64_t)nrb * ntt * a.S, kRow = 1 << 23;
    const unsigned gx = (unsigned)(total < kRow ? total : kRow), gy = (unsigned)((total + gx - 1) / gx);
    void *args[] = {&arg, &nrb, &ntt};
    hipError_t e = hipLaunchKernel(k, dim3(gx, gy), dim3(256), args, 0, st);
    if (e != hipSuccess || a.S == 1) return e;
    const float *ws = a.ws;
    float *y = a.y;
    int T = a.T, M = a.M, ldy = a.ldy, S = a.S;
    int64_t ld = (int64_t)a.NT * kTileRows, tpad = (int64_t)ntt * kGemmTB;
    const int64_t n = (int64_t)T * (ld / 4);
    void *rargs[] = {&ws, &y, &T, &M, &ldy, &ld, &tpad, &S};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemm_reduce_kernel), dim3((unsigned)((n + 255) / 256)),
                           dim3(256), rargs, 0, st);
}

}  // namespace qmatk
