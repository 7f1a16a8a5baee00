// gfx950 (CDNA4) kernels for the weight-only quantized small-T product y = x . W^T (T <= 16)
// and the dequantization checking path.  The code conversions they share with the prefill
// GEMM route are in qmat_device.h.
//
// Weight formats (NInfer model cards): groupwise Q4/Q5/Q6 — FP16 scale per 64 weights along K
// times a two's-complement code ("Qwen3.8-27B for NInfer on the RTX 3090", "What is different
// from the upstream artifact") — groupwise Q8, the same definition with 8-bit codes (the cards'
// format tables: token embedding / output head, attention and other projections) — and
// row-scaled FP8 E4M3 ("Qwen3.8-27B NVFP4 for NInfer", "Artifact").  The packed layout is
// described in qmat_layout.h.  Template parameter FMT is the format id (9 = Q8).
//
// Every code is turned into an exact small float before any product is formed:
//   Q4   v_cvt_off_f32_i4 reads a two's-complement nibble as code/16 (SDWA picks the byte);
//        on request (the offset-operand route, up to 8 tokens) the nibble with its top bit
//        flipped (code + 8) is masked into a byte that v_cvt_scalef32_pk_bf16_fp8 reads as
//        (code + 8) * 2^-9, two per instruction, and each group's product sum then subtracts
//        the same MFMA sum over a constant operand 8 * 2^-9 (q4_group_offset), which is exactly
//        the sum of the offsets for a group of zero codes;
//   Q5/6 the code is assembled in the top bits of a byte and v_cvt_f32_i32 with SDWA sign
//        extension reads it as 8*code or 4*code;
//   Q8   the same SDWA convert reads each stored byte as the code;
//   FP8  v_cvt_scalef32_pk_bf16_fp8 widens two E4M3 bytes to bf16 exactly.
// These values are exact in bf16, so bf16(code) * bf16(x) is an exact product; dot products
// accumulate in fp32 (v_dot2c_f32_bf16 on the vector ALU, or the 16x16x32 bf16 MFMA), and the
// per-group scale (times the power of two of the code encoding) is applied once per 64-group.
// The Q4 offset operands round at the size of the group's sum of activations instead of its
// sum of products, so they are an explicit request and not the automatic route.
//
// Work split: a wave owns one 64-row tile and a contiguous range of 128-wide k units.  NW waves
// of a workgroup split a tile's units and reduce through LDS; S workgroups split further and
// their partial tiles meet over a fixed binary tree of atomic exchanges (see finish):
// deterministic, and no memset (every tree word is empty again when a call ends).
#include <hip/hip_runtime.h>

#include "qmat_device.h"
#include "qmat_kernels.h"
#include "qmat_layout.h"

namespace qmatk {
// ------------------------------------------------------------------ split bookkeeping

// [u0, u1): a contiguous run of the tile's k units for this wave; sl, nsl: the wave's slice
// index and the tile's number of slices (the same share, for kernels that take every nsl-th
// unit from sl).
struct Slice {
    int tile, sp, S, w, nw, u0, u1;
    int sl, nsl;
    int wsrow, wsld;  // the tile's first row and the row count of its tree-node region
    int64_t wsoff;    // start of that region among the tree-node words
};

// Workgroup -> (tile, split, splits of that tile).  The trailing NTt tiles come first in the grid
// so that their shared-tile reductions finish while the other tiles are still streaming.
__device__ __forceinline__ Slice make_slice(const RunArgs &a)
{
    Slice s;
    s.nw = blockDim.x >> 6;
    s.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar loop control
    const int b = blockIdx.x, ntail = a.NTt * a.St;
    const int nlead = a.NT - a.NTt;
    if (b < ntail) {
        const int tt = b / a.St;
        s.tile = nlead + tt;
        s.sp = b - tt * a.St;
        s.S = a.St;
        s.wsrow = tt * kTileRows;
        s.wsld = a.NTt * kTileRows;
        s.wsoff = a.S > 1 ? (int64_t)(a.S - 1) * a.T * nlead * kTileRows : 0;
    } else {
        const int c = b - ntail;
        s.tile = c / a.S;
        s.sp = c - s.tile * a.S;
        s.S = a.S;
        s.wsrow = s.tile * kTileRows;
        s.wsld = nlead * kTileRows;
        s.wsoff = 0;
    }
    const int nsl = s.S * s.nw, sl = s.sp * s.nw + s.w;
    s.sl = sl;
    s.nsl = nsl;
    s.u0 = (int)(((int64_t)a.NU * sl) / nsl);
    s.u1 = (int)(((int64_t)a.NU * (sl + 1)) / nsl);
    return s;
}

// The sum of S partials load(0) + load(1) + ... + load(S - 1), added in index order (so every
// run gives the same bits).  The loads go out eight at a time with clamped, unconditional
// indices, so that a batch is in flight together instead of one memory round trip per partial.
template <typename Load>
__device__ __forceinline__ float ordered_sum(int S, Load load)
{
    float v = 0.0f;
    for (int s0 = 0; s0 < S; s0 += 8) {
        float b[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = load(s0 + j < S ? s0 + j : S - 1);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (s0 + j < S) v = s0 + j == 0 ? b[j] : v + b[j];
    }
    return v;
}

// Combine the waves' and workgroups' partial tiles and write y.  Every wave passes its values
// through put(t, row_in_tile, v) calls made identically by all waves (same (t, row) sets).
// red: dynamic LDS of nw * T * 64 floats (unused when nw == 1 and S == 1).
//
// Tiles shared by S > 1 workgroups are summed over a fixed binary tree of the S splits (pairs
// (0,1), (2,3), ... at the first level; a split without a partner moves up unchanged).  Two
// partial sums meet in one 64-bit word of the tile's tree nodes: each side swaps in {1, bits of
// its value} with one agent-scope atomic exchange.  Exchanges of one location are totally
// ordered, so exactly one side gets back the empty word {0, 0} and is done; the other gets its
// partner's value, adds it (fp32 addition is commutative, so the sum has the same bits
// whichever side arrives second), clears the word for the next call and carries the sum to the
// next level.  Whoever completes the root writes y.  Every element meets independently: no
// counters, barriers or fences, one memory round trip per tree level (a thread with several
// elements sends two up together), and the same bits on every run of the same plan.
template <typename ForEach>
__device__ __forceinline__ void finish(const RunArgs &a, const Slice &s, float *red, ForEach for_each)
{
    const int row0 = s.tile * kTileRows;
    if (s.nw == 1 && s.S == 1) {
        for_each([&](int t, int r, float v) {
            if (row0 + r < a.M) a.y[(int64_t)t * a.ldy + row0 + r] = v;
        });
        return;
    }
    // the waves' partial tiles through LDS (also with one wave when the tile is shared: the tree
    // below walks the tile's elements by thread, not by the lanes that computed them)
    const int n = a.T * kTileRows;
    for_each([&](int t, int r, float v) { red[s.w * n + t * kTileRows + r] = v; });
    __syncthreads();
    const int nthr = blockDim.x;
    if (s.S == 1) {
        for (int e = threadIdx.x; e < n; e += nthr) {
            float v = red[e];
            for (int w = 1; w < s.nw; ++w) v += red[w * n + e];
            const int t = e / kTileRows, r = e - t * kTileRows;
            if (row0 + r < a.M) a.y[(int64_t)t * a.ldy + row0 + r] = v;
        }
        return;
    }
    // the tile's node words: one level slot [node][t][row of the region] per tree node
    uint64_t *nodes = a.nodes + s.wsoff;
    const int64_t nstride = (int64_t)a.T * s.wsld;
    if (n <= nthr) {
        // at most one element per thread
        const int e = threadIdx.x, t = e / kTileRows, r = e - t * kTileRows;
        if (e >= n || row0 + r >= a.M) return;  // padding rows: skipped by every split alike
        float v = red[e];
        for (int w = 1; w < s.nw; ++w) v += red[w * n + e];
        const int64_t wd = (int64_t)t * s.wsld + s.wsrow + r;
        int p = s.sp, m = s.S;
        int64_t base = 0;
        while (m > 1) {
            if ((p ^ 1) < m) {
                uint64_t *slot = nodes + (base + (p >> 1)) * nstride + wd;
                const uint64_t old = __hip_atomic_exchange(slot, (1ull << 32) | __builtin_bit_cast(uint32_t, v),
                                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if ((old >> 32) == 0) return;
                v = __builtin_bit_cast(float, (uint32_t)old) + v;
                __hip_atomic_store(slot, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            base += m >> 1;
            p >>= 1;
            m = (m + 1) >> 1;
        }
        a.y[(int64_t)t * a.ldy + row0 + r] = v;
        return;
    }
    // more elements than threads (T > 8 with 8 waves): a thread takes them two at a time, e and
    // e + nthr, and both go up the tree together (both exchanges of a level in flight at once:
    // one round trip per level for the pair)
    for (int e0 = threadIdx.x; e0 < n; e0 += 2 * nthr) {
        const int e1 = e0 + nthr;
        const int t0 = e0 / kTileRows, r0 = e0 - t0 * kTileRows;
        const int t1 = e1 / kTileRows, r1 = e1 - t1 * kTileRows;
        bool on0 = row0 + r0 < a.M;
        bool on1 = e1 < n && row0 + r1 < a.M;
        float v0 = 0.f, v1 = 0.f;
        if (on0) {
            v0 = red[e0];
            for (int w = 1; w < s.nw; ++w) v0 += red[w * n + e0];
        }
        if (on1) {
            v1 = red[e1];
            for (int w = 1; w < s.nw; ++w) v1 += red[w * n + e1];
        }
        const int64_t wd0 = (int64_t)t0 * s.wsld + s.wsrow + r0;
        const int64_t wd1 = on1 ? (int64_t)t1 * s.wsld + s.wsrow + r1 : wd0;
        int p = s.sp, m = s.S;
        int64_t base = 0;
        while (m > 1) {
            if ((p ^ 1) < m) {
                uint64_t *slot0 = nodes + (base + (p >> 1)) * nstride + wd0;
                uint64_t *slot1 = nodes + (base + (p >> 1)) * nstride + wd1;
                uint64_t o0 = 0, o1 = 0;
                if (on0)
                    o0 = __hip_atomic_exchange(slot0, (1ull << 32) | __builtin_bit_cast(uint32_t, v0), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                if (on1)
                    o1 = __hip_atomic_exchange(slot1, (1ull << 32) | __builtin_bit_cast(uint32_t, v1), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                if (on0) {
                    if ((o0 >> 32) == 0) {
                        on0 = false;
                    } else {
                        v0 = __builtin_bit_cast(float, (uint32_t)o0) + v0;
                        __hip_atomic_store(slot0, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
                if (on1) {
                    if ((o1 >> 32) == 0) {
                        on1 = false;
                    } else {
                        v1 = __builtin_bit_cast(float, (uint32_t)o1) + v1;
                        __hip_atomic_store(slot1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            }
            base += m >> 1;
            p >>= 1;
            m = (m + 1) >> 1;
        }
        if (on0) a.y[(int64_t)t0 * a.ldy + row0 + r0] = v0;
        if (on1) a.y[(int64_t)t1 * a.ldy + row0 + r1] = v1;
    }
}

// ------------------------------------------------------------------ unit loads
// Packed weights are read exactly once per call: nontemporal loads keep them from displacing
// the activations (reused by every row tile) in the caches.
__device__ __forceinline__ u32x4_t stream_load(const u32x4_t *p) { return __builtin_nontemporal_load(p); }

// Every address below is a wave-uniform base (tile, unit, k step: scalar registers) plus a
// per-lane byte offset that is fixed for the whole kernel, so the loads need no vector address
// arithmetic in the loop.
template <int FMT, int NB, int XN>
__device__ __forceinline__ void load_weights(const RunArgs &a, int tile, int u, uint32_t lane, Unit<NB, XN> &r)
{
    const int64_t tu = (int64_t)tile * a.NU + u;
    const char *cb = reinterpret_cast<const char *>(a.codes) + tu * (NB * kBlockBytes);
#pragma unroll
    for (int j = 0; j < NB; ++j)
        r.c[j] = stream_load(reinterpret_cast<const u32x4_t *>(cb + j * kBlockBytes + 16u * lane));
    if constexpr (FMT != 8) {
        const char *sb = reinterpret_cast<const char *>(a.scales) + tu * kScaleBlockBytes;
        r.sc = stream_load(reinterpret_cast<const u32x4_t *>(sb + 16u * (lane & 15)));
    }
}

// 8 bf16 activations for the 32-wide k step starting at column kb (wave-uniform); lane_off is
// the lane's byte offset (token row and k octet).  The step is clamped inside the row: only
// the half unit of a K = 64 (mod 128) matrix is clamped, and its clamped steps meet the zero
// codes of a padding group.
__device__ __forceinline__ u32x4_t load_x8(const RunArgs &a, int kb, uint32_t lane_off)
{
    const int kc = kb < a.K - 32 ? kb : a.K - 32;
    return *reinterpret_cast<const u32x4_t *>(reinterpret_cast<const char *>(a.x) + 2 * (int64_t)kc + lane_off);
}

// The same 8 activations through a raw buffer resource over x (T x K bf16): lane_off past
// the end of the buffer (kPastEnd) returns zeros and makes no memory request.
constexpr uint32_t kRawBufferWord3 = 0x00020000u;  // raw 32-bit data format (gfx9 resource word 3)
constexpr uint32_t kPastEnd = 0x7FFFFFF0u;
__device__ __forceinline__ u32x4_t load_x8_buf(const RunArgs &a, __amdgpu_buffer_rsrc_t xr, int kb, uint32_t lane_off)
{
    const int kc = kb < a.K - 32 ? kb : a.K - 32;
    return __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(lane_off + 2u * (uint32_t)kc), 0, 0);
}

// Software pipeline over iterations [u0, u1) of a wave (each one k unit, which load() maps to
// the unit index): a ring of D units in flight; a slot is refilled with iteration u + D right
// after iteration u has been consumed from it.  mid() runs once after the first loads are
// issued (their latency hides it).  The steady-state loop has no branches inside, so the
// compiler's wait counting sees that only the slot being consumed has to have arrived; the
// guarded tail handles the last units.
template <int D, typename U, typename Load, typename Mid, typename Use>
__device__ __forceinline__ void pipeline(int u0, int u1, U (&buf)[D], Load load, Mid mid, Use use)
{
    if (u1 - u0 >= 2 * D) {
        // every slot is filled and refilled at least once: no guards until the tail.  The
        // slots are issued in order (as the loop refills them) so that the wait counts at the
        // loop head are the same on entry and on the back edge.
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load(buf[d], u0 + d);
            __builtin_amdgcn_sched_barrier(0);
        }
        mid();
        int u = u0;
        do {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                use(buf[d], u + d);
                load(buf[d], u + d + D);
                // keep the refill ahead of the next slot's arithmetic
                __builtin_amdgcn_sched_barrier(0);
            }
            u += D;
        } while (u + 2 * D <= u1);
        // D <= u1 - u < 2D units left; the slots hold units u .. u + D - 1
#pragma unroll
        for (int d = 0; d < D; ++d) {
            use(buf[d], u + d);
            if (u + d + D < u1) load(buf[d], u + d + D);
        }
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (u + D + d < u1) use(buf[d], u + D + d);
    } else {
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (u0 + d < u1) load(buf[d], u0 + d);
        mid();
        for (int u = u0; u < u1; u += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                if (u + d < u1) {
                    use(buf[d], u + d);
                    if (u + d + D < u1) load(buf[d], u + d + D);
                }
            }
        }
    }
}

// ------------------------------------------------------------------ vector-ALU route

template <int FMT, int TT, int KA, int MM, int NB, int XN>
__device__ __forceinline__ void valu_step(const Unit<NB, XN> &U, float (&p)[4][TT])
{
    const uint32_t *W = reinterpret_cast<const uint32_t *>(U.c);
    uint32_t b[4];
    bf16x8_signed<FMT, KA, MM>(W, b);
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int d = 0; d < 4; ++d) p[MM][t] = dot2(b[d], U.x[4 * t + KA][d], p[MM][t]);
}

template <int FMT, int TT, int G, int NB, int XN>
__device__ __forceinline__ void valu_group(const Unit<NB, XN> &U, float (&acc)[4][TT])
{
    float p[4][TT];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int t = 0; t < TT; ++t) p[m][t] = 0.f;
    valu_step<FMT, TT, 2 * G, 0>(U, p); valu_step<FMT, TT, 2 * G, 1>(U, p);
    valu_step<FMT, TT, 2 * G, 2>(U, p); valu_step<FMT, TT, 2 * G, 3>(U, p);
    valu_step<FMT, TT, 2 * G + 1, 0>(U, p); valu_step<FMT, TT, 2 * G + 1, 1>(U, p);
    valu_step<FMT, TT, 2 * G + 1, 2>(U, p); valu_step<FMT, TT, 2 * G + 1, 3>(U, p);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        if constexpr (FMT == 8) {
#pragma unroll
            for (int t = 0; t < TT; ++t) acc[m][t] += p[m][t];
        } else {
            const float sf = group_scale(U.sc, G, m);
#pragma unroll
            for (int t = 0; t < TT; ++t) acc[m][t] = fmaf(sf, p[m][t], acc[m][t]);
        }
    }
}

// Lane L handles rows 16*m + L%16 (m = 0..3) and k octet L/16 of every 32-wide k step, for TT
// tokens; the four lanes sharing L%16 are summed at the end.
template <int FMT, int TT, int D>
__global__ __launch_bounds__(512) void valu_kernel(RunArgs a)
{
    constexpr int NB = Fmt<FMT>::NB, XN = 4 * TT;
    extern __shared__ float red[];
    const Slice s = make_slice(a);
    const uint32_t lane = threadIdx.x & 63, q = lane >> 4;
    float acc[4][TT];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[m][t] = 0.f;

    uint32_t xoff[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) xoff[t] = 2u * (uint32_t)(t * a.K) + 16u * q;
    Unit<NB, XN> buf[D];
    pipeline<D>(s.u0, s.u1, buf,
        [&](Unit<NB, XN> &r, int u) {
            load_weights<FMT>(a, s.tile, u, lane, r);
#pragma unroll
            for (int t = 0; t < TT; ++t)
#pragma unroll
                for (int ka = 0; ka < 4; ++ka) r.x[4 * t + ka] = load_x8(a, u * kUnitK + 32 * ka, xoff[t]);
        },
        [&]() {},
        [&](const Unit<NB, XN> &U, int) {
            valu_group<FMT, TT, 0>(U, acc);
            valu_group<FMT, TT, 1>(U, acc);
        });

    // the code encoding's power of two (groupwise) or the row scale (FP8), once per row
    constexpr float kF = Fmt<FMT>::kSignedToCode;
    f32x4_t rs = (f32x4_t){kF, kF, kF, kF};
    if constexpr (FMT == 8) rs = reinterpret_cast<const f32x4_t *>(a.scales)[(int64_t)s.tile * 16 + (lane & 15)];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[m][t] *= rs[m];
    // the four lanes L, L^16, L^32, L^48 hold the same rows for different k octets
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            acc[m][t] += __shfl_xor(acc[m][t], 16);
            acc[m][t] += __shfl_xor(acc[m][t], 32);
        }
    // lane block q keeps row 16*q + L%16
    float v[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t)
        v[t] = q == 0 ? acc[0][t] : q == 1 ? acc[1][t] : q == 2 ? acc[2][t] : acc[3][t];
    const int r = 16 * q + (lane & 15);
    finish(a, s, red, [&](auto put) {
#pragma unroll
        for (int t = 0; t < TT; ++t) put(t, r, v[t]);
    });
}

// ------------------------------------------------------------------ MFMA route

// One 32-wide k step of a tile: the four 16-row slices' codes (blocks c) times the activation
// fragment xa, accumulated into D.
template <int FMT, int KA, int NB, bool OFF>
__device__ __forceinline__ void mfma_step_w(const u32x4_t (&c)[NB], const u32x4_t &xa, f32x4_t (&D)[4])
{
    const uint32_t *W = reinterpret_cast<const uint32_t *>(c);
    const bf16x8_t A = __builtin_bit_cast(bf16x8_t, xa);
#define QMAT_MFMA_ROW(MM)                                                                       \
    {                                                                                           \
        uint32_t b[4];                                                                          \
        if constexpr (OFF) bf16x8_of<FMT, KA, MM>(W, b);                                        \
        else bf16x8_signed<FMT, KA, MM>(W, b);                                                  \
        const bf16x8_t B = __builtin_bit_cast(bf16x8_t, (u32x4_t){b[0], b[1], b[2], b[3]});     \
        D[MM] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, D[MM], 0, 0, 0);                 \
    }
    QMAT_MFMA_ROW(0) QMAT_MFMA_ROW(1) QMAT_MFMA_ROW(2) QMAT_MFMA_ROW(3)
#undef QMAT_MFMA_ROW
}

template <int FMT, int KA, bool OFF, int NB, int XN>
__device__ __forceinline__ void mfma_step(const Unit<NB, XN> &U, f32x4_t (&D)[4])
{
    mfma_step_w<FMT, KA, NB, OFF>(U.c, U.x[KA], D);
}

// Whether an MFMA kernel with TR token slots per lane uses the offset Q4 operands (two extra
// matrix instructions and TR subtractions per row slice and group, 8 instead of 13 unpack
// instructions per 8 codes): only when the launch asks for them (OFS), and only up to 8 tokens,
// where the shorter unpack pays for the rest.
template <int FMT, int TR, bool OFS> constexpr bool mfma_offset()
{
    return Fmt<FMT>::kOffset != 0.0f && TR < 4 && OFS;
}

// A operand: 16 token slots x 32 k (lane l: slot l % 16, k octet l / 16); B operand: 32 k x 16
// rows of the tile (lane l: row 16*m + l % 16, the same k octet) — exactly the packed layout.
// D[m]: lane l holds slots 4*(l/16) + r (r = 0..3) of row 16*m + l % 16.
//
// Token t sits in slot 4*(t / TR) + t % TR, so that the tokens of a launch fill only the first
// TR of every lane's four D components: TR = 1 up to 4 tokens, 2 up to 8, 4 up to 16.  A lane
// then applies TR group scales per row group and unit instead of four, and keeps TR
// accumulators per row group (the MFMA's other components are computed and dropped).
template <int TR> __device__ __forceinline__ int slot_token(int slot)
{
    return (slot & 3) < TR ? TR * (slot >> 2) + (slot & 3) : 16;  // 16: no token
}

template <int FMT, int D_, int TR, bool OFS>
__global__ __launch_bounds__(512) void mfma_kernel(RunArgs a)
{
    constexpr int NB = Fmt<FMT>::NB, XN = 4;
    extern __shared__ float red[];
    const Slice s = make_slice(a);
    const uint32_t lane = threadIdx.x & 63;
    const int tok = slot_token<TR>(lane & 15), oct = lane >> 4;
    // A rows of slots without a token only feed D rows that are never stored: those lanes read
    // the activations through a buffer resource at an offset past its end, which returns zeros
    // without a memory request (at T = 1, 15 lanes in 16)
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.x), (short)0, 2 * a.T * a.K, kRawBufferWord3);
    const uint32_t xoff = tok < a.T ? 2u * (uint32_t)(tok * a.K) + 16u * oct : kPastEnd;
    constexpr bool OFF = mfma_offset<FMT, TR, OFS>();
    f32x4_t acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    // Depth-2 kernels take every nsl-th unit of the tile from unit sl, so that the waves
    // sharing a tile read neighbouring units at the same time (one moving region per tile
    // instead of one per wave); depth-1 kernels take a contiguous run [u0, u1).
    int ui0 = s.u0, ui1 = s.u1;
    if constexpr (D_ == 2) {
        ui0 = 0;
        ui1 = s.sl < a.NU ? (a.NU - s.sl + s.nsl - 1) / s.nsl : 0;
    }
    Unit<NB, XN> buf[D_];
    pipeline<D_>(ui0, ui1, buf,
        [&](Unit<NB, XN> &r, int u) {
            if constexpr (D_ == 2) u = s.sl + u * s.nsl;
            load_weights<FMT>(a, s.tile, u, lane, r);
#pragma unroll
            for (int ka = 0; ka < 4; ++ka)
                r.x[ka] = load_x8_buf(a, xr, u * kUnitK + 32 * ka, xoff);
        },
        [&]() {},
        [&](const Unit<NB, XN> &U, int) {
            if constexpr (FMT == 8) {
                mfma_step<FMT, 0, OFF>(U, acc);
                mfma_step<FMT, 1, OFF>(U, acc);
                mfma_step<FMT, 2, OFF>(U, acc);
                mfma_step<FMT, 3, OFF>(U, acc);
            } else {
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    f32x4_t P[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) P[m] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
                    if (g == 0) {
                        mfma_step<FMT, 0, OFF>(U, P);
                        mfma_step<FMT, 1, OFF>(U, P);
                    } else {
                        mfma_step<FMT, 2, OFF>(U, P);
                        mfma_step<FMT, 3, OFF>(U, P);
                    }
                    if constexpr (OFF) {
                        const f32x4_t o = q4_group_offset(U.x[2 * g], U.x[2 * g + 1]);
#pragma unroll
                        for (int m = 0; m < 4; ++m)
#pragma unroll
                            for (int r = 0; r < TR; ++r) P[m][r] -= o[r];
                    }
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const float sf = group_scale(U.sc, g, m);
#pragma unroll
                        for (int r = 0; r < TR; ++r) acc[m][r] = fmaf(sf, P[m][r], acc[m][r]);
                    }
                }
            }
        });

    constexpr float kF = OFF ? Fmt<FMT>::kToCode : Fmt<FMT>::kSignedToCode;
    f32x4_t rs = (f32x4_t){kF, kF, kF, kF};
    if constexpr (FMT == 8) rs = reinterpret_cast<const f32x4_t *>(a.scales)[(int64_t)s.tile * 16 + (lane & 15)];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < TR; ++r) acc[m][r] *= rs[m];
    const int t0 = TR * oct, rr = lane & 15;
    finish(a, s, red, [&](auto put) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < TR; ++r)
                if (t0 + r < a.T) put(t0 + r, 16 * m + rr, acc[m][r]);
    });
}

// Two row tiles per wave, one activation fragment: for verify-sized T the activation loads
// (16 tokens x 32 k per step, 1 KB per wave instruction from the L2) cost as much load issue
// as a quarter to a half of the weight stream.  A wave that streams the same k unit of two
// neighbouring tiles loads each fragment once for both.  Only for plans without a trailing-tile
// split: the S workgroups of pair p own tiles 2p and 2p + 1 (the second absent for the last
// pair of an odd tile count; its loads then repeat the first tile and nothing is stored for
// it).  Per tile the arithmetic, the wave and k split of its units and the reduction (through
// that tile's own tree words) are those of mfma_kernel, so both kernels give the same bits.
template <int NB> struct PairUnit {
    u32x4_t c[2][NB];
    u32x4_t sc[2];
    u32x4_t x[4];
};

template <int FMT, int D_, int TR, bool OFS>
__global__ __launch_bounds__(512) void mfma_pair_kernel(RunArgs a)
{
    constexpr int NB = Fmt<FMT>::NB;
    extern __shared__ float red[];
    const Slice s = make_slice(a);  // no trailing tiles: s.tile is the pair index
    const int pair = s.tile;
    const uint32_t lane = threadIdx.x & 63;
    const int tok = slot_token<TR>(lane & 15), oct = lane >> 4;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.x), (short)0, 2 * a.T * a.K, kRawBufferWord3);
    const uint32_t xoff = tok < a.T ? 2u * (uint32_t)(tok * a.K) + 16u * oct : kPastEnd;
    const int tile0 = 2 * pair, tile1 = 2 * pair + 1 < a.NT ? 2 * pair + 1 : 2 * pair;
    constexpr bool OFF = mfma_offset<FMT, TR, OFS>();
    f32x4_t acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[i][m] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    int ui0 = s.u0, ui1 = s.u1;
    if constexpr (D_ == 2) {
        ui0 = 0;
        ui1 = s.sl < a.NU ? (a.NU - s.sl + s.nsl - 1) / s.nsl : 0;
    }
    PairUnit<NB> buf[D_];
    pipeline<D_>(ui0, ui1, buf,
        [&](PairUnit<NB> &r, int u) {
            if constexpr (D_ == 2) u = s.sl + u * s.nsl;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int64_t tu = (int64_t)(i ? tile1 : tile0) * a.NU + u;
                const char *cb = reinterpret_cast<const char *>(a.codes) + tu * (NB * kBlockBytes);
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    r.c[i][j] = stream_load(reinterpret_cast<const u32x4_t *>(cb + j * kBlockBytes + 16u * lane));
                if constexpr (FMT != 8) {
                    const char *sb = reinterpret_cast<const char *>(a.scales) + tu * kScaleBlockBytes;
                    r.sc[i] = stream_load(reinterpret_cast<const u32x4_t *>(sb + 16u * (lane & 15)));
                }
            }
#pragma unroll
            for (int ka = 0; ka < 4; ++ka)
                r.x[ka] = load_x8_buf(a, xr, u * kUnitK + 32 * ka, xoff);
        },
        [&]() {},
        [&](const PairUnit<NB> &U, int) {
            // the Q4 offset sums depend on the activations only: once for both tiles
            f32x4_t o[2] = {(f32x4_t){0.f, 0.f, 0.f, 0.f}, (f32x4_t){0.f, 0.f, 0.f, 0.f}};
            if constexpr (OFF) {
                o[0] = q4_group_offset(U.x[0], U.x[1]);
                o[1] = q4_group_offset(U.x[2], U.x[3]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if constexpr (FMT == 8) {
                    mfma_step_w<FMT, 0, NB, OFF>(U.c[i], U.x[0], acc[i]);
                    mfma_step_w<FMT, 1, NB, OFF>(U.c[i], U.x[1], acc[i]);
                    mfma_step_w<FMT, 2, NB, OFF>(U.c[i], U.x[2], acc[i]);
                    mfma_step_w<FMT, 3, NB, OFF>(U.c[i], U.x[3], acc[i]);
                } else {
#pragma unroll
                    for (int g = 0; g < 2; ++g) {
                        f32x4_t P[4];
#pragma unroll
                        for (int m = 0; m < 4; ++m) P[m] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
                        if (g == 0) {
                            mfma_step_w<FMT, 0, NB, OFF>(U.c[i], U.x[0], P);
                            mfma_step_w<FMT, 1, NB, OFF>(U.c[i], U.x[1], P);
                        } else {
                            mfma_step_w<FMT, 2, NB, OFF>(U.c[i], U.x[2], P);
                            mfma_step_w<FMT, 3, NB, OFF>(U.c[i], U.x[3], P);
                        }
                        if constexpr (OFF) {
#pragma unroll
                            for (int m = 0; m < 4; ++m)
#pragma unroll
                                for (int r = 0; r < TR; ++r) P[m][r] -= o[g][r];
                        }
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            const float sf = group_scale(U.sc[i], g, m);
#pragma unroll
                            for (int r = 0; r < TR; ++r) acc[i][m][r] = fmaf(sf, P[m][r], acc[i][m][r]);
                        }
                    }
                }
            }
        });

    const int t0 = TR * oct, rr = lane & 15;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        Slice si = s;
        si.tile = tile0 + i;
        si.wsrow = si.tile * kTileRows;
        if (si.tile >= a.NT) break;  // uniform over the workgroup
        constexpr float kF = OFF ? Fmt<FMT>::kToCode : Fmt<FMT>::kSignedToCode;
        f32x4_t rs = (f32x4_t){kF, kF, kF, kF};
        if constexpr (FMT == 8) rs = reinterpret_cast<const f32x4_t *>(a.scales)[(int64_t)si.tile * 16 + (lane & 15)];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < TR; ++r) acc[i][m][r] *= rs[m];
        if (i > 0 && s.nw > 1) __syncthreads();  // the first tile's reduction is done with red
        finish(a, si, red, [&](auto put) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int r = 0; r < TR; ++r)
                    if (t0 + r < a.T) put(t0 + r, 16 * m + rr, acc[i][m][r]);
        });
    }
}

// ------------------------------------------------------------------ dequant (checking path)

template <int FMT, int KA, int MM>
__device__ __forceinline__ void dequant_step(const DequantArgs &a, const uint32_t *W, const u32x4_t &sc,
                                             const f32x4_t &rs, int tile, int u, int lane)
{
    const int row = tile * kTileRows + 16 * MM + (lane & 15);
    const int k = u * kUnitK + 32 * KA + 8 * (lane >> 4);
    if (row >= a.M || k >= a.K) return;
    float out[8];
    if constexpr (FMT == 8) {
        uint32_t b[4];
        bf16x8_of<FMT, KA, MM>(W, b);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = rs[MM] * __builtin_bit_cast(float, b[i] << 16);
            out[2 * i + 1] = rs[MM] * __builtin_bit_cast(float, b[i] & 0xFFFF0000u);
        }
    } else {
        // the exact bf16 operands the matrix-core products take, decoded back to the code
        // (u * kToCode - kOffset: both steps exact)
        uint32_t b[4];
        bf16x8_of<FMT, KA, MM>(W, b);
        const float sc_f = group_scale(sc, KA >> 1, MM);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t hb = (i & 1) ? (b[i >> 1] & 0xFFFF0000u) : (b[i >> 1] << 16);
            out[i] = sc_f * (__builtin_bit_cast(float, hb) * Fmt<FMT>::kToCode - Fmt<FMT>::kOffset);
        }
    }
    float *dst = a.w + (int64_t)row * a.K + k;
    reinterpret_cast<f32x4_t *>(dst)[0] = (f32x4_t){out[0], out[1], out[2], out[3]};
    reinterpret_cast<f32x4_t *>(dst)[1] = (f32x4_t){out[4], out[5], out[6], out[7]};
}

template <int FMT>
__global__ __launch_bounds__(64) void dequant_kernel(DequantArgs a)
{
    constexpr int NB = Fmt<FMT>::NB;
    const int lane = threadIdx.x;
    const int tile = blockIdx.x / a.NU, u = blockIdx.x - tile * a.NU;
    u32x4_t c[NB];
    const u32x4_t *cp = reinterpret_cast<const u32x4_t *>(a.codes) + (((int64_t)tile * a.NU + u) * NB) * 64 + lane;
#pragma unroll
    for (int j = 0; j < NB; ++j) c[j] = cp[j * 64];
    u32x4_t sc = (u32x4_t){0u, 0u, 0u, 0u};
    f32x4_t rs = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    if constexpr (FMT == 8)
        rs = reinterpret_cast<const f32x4_t *>(a.scales)[(int64_t)tile * 16 + (lane & 15)];
    else
        sc = reinterpret_cast<const u32x4_t *>(a.scales)[((int64_t)tile * a.NU + u) * 16 + (lane & 15)];
    const uint32_t *W = reinterpret_cast<const uint32_t *>(c);
#define QMAT_DQ(KA)                                          \
    dequant_step<FMT, KA, 0>(a, W, sc, rs, tile, u, lane);   \
    dequant_step<FMT, KA, 1>(a, W, sc, rs, tile, u, lane);   \
    dequant_step<FMT, KA, 2>(a, W, sc, rs, tile, u, lane);   \
    dequant_step<FMT, KA, 3>(a, W, sc, rs, tile, u, lane);
    QMAT_DQ(0) QMAT_DQ(1) QMAT_DQ(2) QMAT_DQ(3)
#undef QMAT_DQ
}

// ------------------------------------------------------------------ launchers

// The MFMA kernel for T tokens: token slots per lane and row group 1 up to 4 tokens, 2 up to 8,
// 4 up to 16; the offset operands (ofs) only change the Q4 kernels up to 8 tokens, so the other
// formats and T share one instantiation.
template <int FMT, int D, int TR> static const void *mfma_kernel_for(int tiles, bool ofs)
{
    constexpr bool kOfsDiffers = mfma_offset<FMT, TR, true>();
    if (ofs && kOfsDiffers)
        return tiles == 2 ? reinterpret_cast<const void *>(&mfma_pair_kernel<FMT, D, TR, kOfsDiffers>)
                          : reinterpret_cast<const void *>(&mfma_kernel<FMT, D, TR, kOfsDiffers>);
    return tiles == 2 ? reinterpret_cast<const void *>(&mfma_pair_kernel<FMT, D, TR, false>)
                      : reinterpret_cast<const void *>(&mfma_kernel<FMT, D, TR, false>);
}

template <int FMT, int D> static const void *run_kernel_d(int route, int T, int tiles, bool ofs)
{
    if (route == kRouteMfma)
        return T <= 4 ? mfma_kernel_for<FMT, D, 1>(tiles, ofs)
             : T <= 8 ? mfma_kernel_for<FMT, D, 2>(tiles, ofs)
                      : mfma_kernel_for<FMT, D, 4>(tiles, ofs);
    if (tiles == 2) return nullptr;
    switch (T) {
    case 1: return reinterpret_cast<const void *>(&valu_kernel<FMT, 1, D>);
    case 2: return reinterpret_cast<const void *>(&valu_kernel<FMT, 2, D>);
    case 3: return reinterpret_cast<const void *>(&valu_kernel<FMT, 3, D>);
    case 4: return reinterpret_cast<const void *>(&valu_kernel<FMT, 4, D>);
    default: return nullptr;
    }
}

template <int FMT> static const void *run_kernel(int route, int T, int depth, int tiles, bool ofs)
{
    switch (depth) {
    case 1: return run_kernel_d<FMT, 1>(route, T, tiles, ofs);
    case 2: return run_kernel_d<FMT, 2>(route, T, tiles, ofs);
    default: return nullptr;
    }
}

static const void *run_kernel_for(int fmt, int route, int T, int depth, int tiles, bool ofs)
{
    switch (fmt) {
    case 4: return run_kernel<4>(route, T, depth, tiles, ofs);
    case 5: return run_kernel<5>(route, T, depth, tiles, ofs);
    case 6: return run_kernel<6>(route, T, depth, tiles, ofs);
    case 8: return run_kernel<8>(route, T, depth, tiles, ofs);
    case 9: return run_kernel<9>(route, T, depth, tiles, ofs);
    default: return nullptr;
    }
}

// dynamic LDS of the small-T kernels: the waves' partial tiles, when a workgroup has several
// waves or its tile is shared with other workgroups
static size_t run_lds_bytes(int waves, int T, bool shared)
{
    return waves > 1 || shared ? (size_t)waves * T * kTileRows * sizeof(float) : 0;
}


hipError_t launch_run(int fmt, int route, int depth, const RunArgs &a, int waves, int tiles, bool offset_ops,
                      hipStream_t st)
{
    if (tiles == 2 && a.NTt != 0) return hipErrorInvalidValue;
    const void *k = run_kernel_for(fmt, route, a.T, depth, tiles, offset_ops);
    if (!k) return hipErrorInvalidValue;
    RunArgs arg = a;
    void *args[] = {&arg};
    const int64_t grid = tiles == 2 ? (int64_t)(a.NT + 1) / 2 * a.S : (int64_t)a.NTt * a.St + (int64_t)(a.NT - a.NTt) * a.S;
    const bool shared = a.S > 1 || (a.NTt > 0 && a.St > 1);
    return hipLaunchKernel(k, dim3((unsigned)grid), dim3((unsigned)(64 * waves)), args, run_lds_bytes(waves, a.T, shared),
                           st);
}

int run_blocks_per_cu(int fmt, int route, int depth, int T, int waves, int S)
{
    const void *k = run_kernel_for(fmt, route, T, depth, 1, false);
    int n = 0;
    if (!k || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, 64 * waves, run_lds_bytes(waves, T, S > 1)) !=
                  hipSuccess)
        return 0;
    return n;
}

template <int FMT> static const void *dequant_kernel_ptr() { return reinterpret_cast<const void *>(&dequant_kernel<FMT>); }

hipError_t launch_dequant(int fmt, const DequantArgs &a, hipStream_t st)
{
    const void *k = fmt == 4 ? dequant_kernel_ptr<4>() : fmt == 5 ? dequant_kernel_ptr<5>()
                  : fmt == 6 ? dequant_kernel_ptr<6>() : fmt == 8 ? dequant_kernel_ptr<8>()
                  : fmt == 9 ? dequant_kernel_ptr<9>() : nullptr;
    if (!k) return hipErrorInvalidValue;
    DequantArgs arg = a;
    void *args[] = {&arg};
    return hipLaunchKernel(k, dim3((unsigned)(a.NT * a.NU)), dim3(64), args, 0, st);
}

}  // namespace qmatk
