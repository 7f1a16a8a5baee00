// gfx950 (CDNA4) kernels for the weight-only quantized small-T product y = x . W^T.
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
//   Q5/6 the code is assembled in the top bits of a byte and v_cvt_f32_i32 with SDWA sign
//        extension reads it as 8*code or 4*code;
//   Q8   the same SDWA convert reads each stored byte as the code;
//   FP8  v_cvt_scalef32_pk_bf16_fp8 widens two E4M3 bytes to bf16 exactly.
// These values are exact in bf16, so bf16(code) * bf16(x) is an exact product; dot products
// accumulate in fp32 (v_dot2c_f32_bf16 on the vector ALU, or the 16x16x32 bf16 MFMA), and the
// per-group scale (times the power of two of the code encoding) is applied once per 64-group.
// No offset-binary tricks: a row with sparse or zero codes has no cancellation error.
//
// Work split: a wave owns one 64-row tile and a contiguous range of 128-wide k units.  NW waves
// of a workgroup split a tile's units and reduce through LDS; S workgroups split further and the
// last-arriving one adds the S partials from the workspace in a fixed order (deterministic, no
// atomics on data, no memset: the arrival counter is reset by the last block).
#include <hip/hip_runtime.h>

#include "qmat_kernels.h"
#include "qmat_layout.h"

namespace qmatk {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

template <int FMT> struct Fmt;
// NB: 1 KB blocks per unit.  kToCode: the unpacked value times kToCode is the code (Q4 reads
// code/16, Q5 8*code, Q6 4*code); the factor is applied once per row at the end.
template <> struct Fmt<4> { static constexpr int NB = 4; static constexpr float kToCode = 16.0f; };
template <> struct Fmt<5> { static constexpr int NB = 5; static constexpr float kToCode = 0.125f; };
template <> struct Fmt<6> { static constexpr int NB = 6; static constexpr float kToCode = 0.25f; };
template <> struct Fmt<8> { static constexpr int NB = 8; static constexpr float kToCode = 1.0f; };
template <> struct Fmt<9> { static constexpr int NB = 8; static constexpr float kToCode = 1.0f; };

// ------------------------------------------------------------------ exact code conversion

// sign-extended nibble in bits [3:0] of byte B of v, as a float equal to nibble / 16
// (v_cvt_off_f32_i4; the byte selection folds into its SDWA operand select).  Plain builtins,
// no inline assembly: the compiler must see these instructions to keep the wait states the
// matrix-core instructions around them need.
template <int B> __device__ __forceinline__ float nib_lo(uint32_t v)
{
    if constexpr (B == 0) return __builtin_amdgcn_cvt_off_f32_i4(v);
    else if constexpr (B == 1) return __builtin_amdgcn_cvt_off_f32_i4((v >> 8) & 0xFFu);
    else if constexpr (B == 2) return __builtin_amdgcn_cvt_off_f32_i4(v >> 16);
    else return __builtin_amdgcn_cvt_off_f32_i4(v >> 24);
}

// byte B of v as a signed integer, converted to float (SDWA sign-extending convert)
template <int B> __device__ __forceinline__ float sbyte(uint32_t v)
{
    return (float)(int8_t)(v >> (8 * B));
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint32_t shift_signed(uint32_t v, int s)
{
    return s >= 0 ? (v << s) : (v >> -s);
}

// The 8 codes of row m in k step KA of a unit, as exact floats equal to code / kToCode.
// W: the lane's 4*NB dwords of the unit (layout in qmat_layout.h).
template <int FMT, int KA, int MM>
__device__ __forceinline__ void codes8(const uint32_t *W, float (&f)[8])
{
    if constexpr (FMT == 4) {
        // nibble e = 2i sits in bits [3:0] of byte i, e = 2i+1 in bits [7:4]; v_cvt_off_f32_i4
        // reads the low four bits of the byte SDWA selects as code/16, so the odd nibbles take
        // one rotate (a rotate rather than a shift keeps h opaque to the compiler, so its bytes
        // are SDWA-selected too instead of being re-extracted from n)
        const uint32_t n = W[4 * KA + MM], h = __builtin_amdgcn_alignbit(n, n, 4);
        f[0] = nib_lo<0>(n); f[1] = nib_lo<0>(h);
        f[2] = nib_lo<1>(n); f[3] = nib_lo<1>(h);
        f[4] = nib_lo<2>(n); f[5] = nib_lo<2>(h);
        f[6] = nib_lo<3>(n); f[7] = nib_lo<3>(h);
    } else {
        uint32_t o[2];
        if constexpr (FMT == 5) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int oi = 2 * MM + hh;
                if (oi < 4) {
                    o[hh] = W[5 * KA + oi] & 0xF8F8F8F8u;
                } else {
                    const int d = oi - 4;
                    o[hh] = ((W[5 * KA + d] << 5) & 0xE0E0E0E0u) |
                            (shift_signed(W[5 * KA + 4], 3 - 2 * d) & 0x18181818u);
                }
            }
        } else if constexpr (FMT == 9) {
            // Q8: the row's 8 codes are the bytes of two dwords, already signed bytes.  The
            // empty asm (no instruction) hides where the dwords come from, so that each byte is
            // converted by one SDWA convert as for the other formats rather than extracted first.
            o[0] = W[8 * KA + 2 * MM];
            o[1] = W[8 * KA + 2 * MM + 1];
            asm("" : "+v"(o[0]), "+v"(o[1]));
        } else {  // FMT == 6
            const uint32_t A = W[6 * KA + 3 * (MM >> 1)], B = W[6 * KA + 3 * (MM >> 1) + 1],
                           C = W[6 * KA + 3 * (MM >> 1) + 2];
            if ((MM & 1) == 0) {
                o[0] = A & 0xFCFCFCFCu;
                o[1] = B & 0xFCFCFCFCu;
            } else {
                o[0] = C & 0xFCFCFCFCu;
                o[1] = ((A << 6) & 0xC0C0C0C0u) | ((B << 4) & 0x30303030u) | ((C << 2) & 0x0C0C0C0Cu);
            }
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            f[4 * hh + 0] = sbyte<0>(o[hh]);
            f[4 * hh + 1] = sbyte<1>(o[hh]);
            f[4 * hh + 2] = sbyte<2>(o[hh]);
            f[4 * hh + 3] = sbyte<3>(o[hh]);
        }
    }
}

// The 8 weights of row m in k step KA as 4 dwords of bf16 pairs (k, k+1), exact: groupwise
// code / kToCode, FP8 the E4M3 value.
template <int FMT, int KA, int MM>
__device__ __forceinline__ void bf16x8_of(const uint32_t *W, uint32_t (&b)[4])
{
    if constexpr (FMT == 8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t w = W[8 * KA + 2 * MM + h];
            b[2 * h + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
            b[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
        }
    } else {
        float f[8];
        codes8<FMT, KA, MM>(W, f);
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = pack_bf16(f[2 * i], f[2 * i + 1]);
    }
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// binary16 scale of group g (0/1 in the unit) for the lane's row m, from the lane's 16-byte
// scale slot (index 4*g + m)
__device__ __forceinline__ float group_scale(const u32x4_t &sc, int g, int m)
{
    const int idx = 4 * g + m;
    const uint32_t w = sc[idx >> 1];
    return half_bits_to_float((idx & 1) ? (w >> 16) : (w & 0xFFFFu));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

// ------------------------------------------------------------------ split bookkeeping

struct Slice {
    int tile, sp, S, w, nw, u0, u1;
    int wsrow, wsld;  // the tile's first row and the row count of its workspace region
    int64_t wsoff;    // start of that region in the workspace (floats)
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
        s.wsoff = a.S > 1 ? (int64_t)a.S * a.T * nlead * kTileRows : 0;
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
    const int n = a.T * kTileRows;
    if (s.nw > 1) {
        for_each([&](int t, int r, float v) { red[s.w * n + t * kTileRows + r] = v; });
        __syncthreads();
    }
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
    // S > 1.  The workgroup's partial tile goes to the workspace through returning agent-scope
    // atomic exchanges: each is performed at the device coherence point before its old value
    // comes back, and every thread consumes its old values before the barrier, so all of the
    // tile's partials are in place before thread 0 bumps the arrival counter.  The last of the
    // S workgroups to arrive reads the S partials with agent-scope atomic loads and adds them
    // in split order (deterministic).  No cache-wide fences, no memset: the last block resets
    // the counter for the next call.
    float *wsr = a.ws + s.wsoff + s.wsrow;
    float *wsp = wsr + (int64_t)s.sp * a.T * s.wsld;
    uint32_t sink = 0;
    auto publish = [&](int t, int r, float v) {
        uint32_t *p = reinterpret_cast<uint32_t *>(wsp + (int64_t)t * s.wsld + r);
        sink |= __hip_atomic_exchange(p, __builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    if (s.nw > 1) {
        for (int e = threadIdx.x; e < n; e += nthr) {
            float v = red[e];
            for (int w = 1; w < s.nw; ++w) v += red[w * n + e];
            const int t = e / kTileRows, r = e - t * kTileRows;
            publish(t, r, v);
        }
    } else {
        for_each(publish);
    }
    asm volatile("" ::"v"(sink));
    __syncthreads();
    __shared__ int last;
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&a.counters[s.tile], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        last = (prev == (uint32_t)(s.S - 1));
    }
    __syncthreads();
    if (!last) return;
    for (int e = threadIdx.x; e < n; e += nthr) {
        const int t = e / kTileRows, r = e - t * kTileRows;
        if (row0 + r >= a.M) continue;
        uint32_t *p = reinterpret_cast<uint32_t *>(wsr + (int64_t)t * s.wsld + r);
        a.y[(int64_t)t * a.ldy + row0 + r] = ordered_sum(s.S, [&](int sp) {
            return __builtin_bit_cast(float, __hip_atomic_load(p + (int64_t)sp * a.T * s.wsld, __ATOMIC_RELAXED,
                                                               __HIP_MEMORY_SCOPE_AGENT));
        });
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&a.counters[s.tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ unit loads

// What one lane needs for one 128-wide k unit: its NB packed code slots, its scale slot and the
// XN vectors of 8 bf16 activations the unit multiplies.
template <int NB, int XN> struct Unit {
    u32x4_t c[NB];
    u32x4_t sc;
    u32x4_t x[XN];
};


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

// 8 bf16 activations for the 32-wide k step starting at column kb (wave-uniform); lane_off is
// the lane's byte offset (token row and k octet).  The step is clamped inside the row: only
// the half unit of a K = 64 (mod 128) matrix is clamped, and its clamped steps meet the zero
// codes of a padding group.
__device__ __forceinline__ u32x4_t load_x8(const RunArgs &a, int kb, uint32_t lane_off)
{
    const int kc = kb < a.K - 32 ? kb : a.K - 32;
    return *reinterpret_cast<const u32x4_t *>(reinterpret_cast<const char *>(a.x) + 2 * (int64_t)kc + lane_off);
}

// Software pipeline over a wave's units [u0, u1): a ring of D units in flight; a slot is
// refilled with unit u + D right after unit u has been consumed from it.  mid() runs once
// after the first loads are issued (their latency hides it).  The steady-state loop has no
// branches inside, so the compiler's wait counting sees that only the slot being consumed
// has to have arrived; the guarded tail handles the last units.
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
    bf16x8_of<FMT, KA, MM>(W, b);
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
    f32x4_t rs = (f32x4_t){Fmt<FMT>::kToCode, Fmt<FMT>::kToCode, Fmt<FMT>::kToCode, Fmt<FMT>::kToCode};
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

template <int FMT, int KA, int NB, int XN>
__device__ __forceinline__ void mfma_step(const Unit<NB, XN> &U, f32x4_t (&D)[4])
{
    const uint32_t *W = reinterpret_cast<const uint32_t *>(U.c);
    const bf16x8_t A = __builtin_bit_cast(bf16x8_t, U.x[KA]);
#define QMAT_MFMA_ROW(MM)                                                                       \
    {                                                                                           \
        uint32_t b[4];                                                                          \
        bf16x8_of<FMT, KA, MM>(W, b);                                                           \
        const bf16x8_t B = __builtin_bit_cast(bf16x8_t, (u32x4_t){b[0], b[1], b[2], b[3]});     \
        D[MM] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, D[MM], 0, 0, 0);                 \
    }
    QMAT_MFMA_ROW(0) QMAT_MFMA_ROW(1) QMAT_MFMA_ROW(2) QMAT_MFMA_ROW(3)
#undef QMAT_MFMA_ROW
}

// A operand: 16 tokens x 32 k (lane l: token l % 16, k octet l / 16); B operand: 32 k x 16 rows
// of the tile (lane l: row 16*m + l % 16, the same k octet) — exactly the packed layout.
// D[m]: lane l holds tokens 4*(l/16) + r (r = 0..3) of row 16*m + l % 16.  TR: how many of the
// four r components can hold a real token (1 when T == 1: only token 0, in lanes 0..15).
template <int FMT, int D_, int TR>
__global__ __launch_bounds__(512) void mfma_kernel(RunArgs a)
{
    constexpr int NB = Fmt<FMT>::NB, XN = 4;
    extern __shared__ float red[];
    const Slice s = make_slice(a);
    const uint32_t lane = threadIdx.x & 63;
    const int tok = lane & 15, oct = lane >> 4;
    // A rows of tokens >= T only feed D rows that are never stored: load a valid token instead
    const int tok_c = tok < a.T ? tok : a.T - 1;
    const uint32_t xoff = 2u * (uint32_t)(tok_c * a.K) + 16u * oct;
    f32x4_t acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    Unit<NB, XN> buf[D_];
    pipeline<D_>(s.u0, s.u1, buf,
        [&](Unit<NB, XN> &r, int u) {
            load_weights<FMT>(a, s.tile, u, lane, r);
#pragma unroll
            for (int ka = 0; ka < 4; ++ka)
                r.x[ka] = load_x8(a, u * kUnitK + 32 * ka, xoff);
        },
        [&]() {},
        [&](const Unit<NB, XN> &U, int) {
            if constexpr (FMT == 8) {
                mfma_step<FMT, 0>(U, acc);
                mfma_step<FMT, 1>(U, acc);
                mfma_step<FMT, 2>(U, acc);
                mfma_step<FMT, 3>(U, acc);
            } else {
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    f32x4_t P[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) P[m] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
                    if (g == 0) {
                        mfma_step<FMT, 0>(U, P);
                        mfma_step<FMT, 1>(U, P);
                    } else {
                        mfma_step<FMT, 2>(U, P);
                        mfma_step<FMT, 3>(U, P);
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

    f32x4_t rs = (f32x4_t){Fmt<FMT>::kToCode, Fmt<FMT>::kToCode, Fmt<FMT>::kToCode, Fmt<FMT>::kToCode};
    if constexpr (FMT == 8) rs = reinterpret_cast<const f32x4_t *>(a.scales)[(int64_t)s.tile * 16 + (lane & 15)];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < TR; ++r) acc[m][r] *= rs[m];
    const int t0 = 4 * oct, rr = lane & 15;
    finish(a, s, red, [&](auto put) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < TR; ++r)
                if (t0 + r < a.T) put(t0 + r, 16 * m + rr, acc[m][r]);
    });
}

// ------------------------------------------------------------------ GEMM route (prefill, T > 16)

// Prefill-sized products: the weights are reused by many tokens, so the MFMA does most of the
// work and each unpacked weight fragment feeds kGemmTB / 16 matrix instructions.  A workgroup
// is 4 waves; wave w owns row tile 4 * rb + w (64 rows), the workgroup a tile of kGemmTB
// tokens.  Per 128-wide k unit the workgroup stages the token tile's activations in LDS (shared
// by its 4 waves, double-buffered, one barrier per unit) while each wave streams its tile's
// packed unit from HBM one unit ahead.  Per 64-group and 16-row slice m, two MFMAs sum
// code * x into P and the group scale enters once per (token, row): acc += scale * P (exact
// products, fp32 sums, as on the small-T routes).  Row-scaled FP8 has no group scale: the MFMA
// accumulates straight into acc and the row scale is applied at the end.
//
// Two workgroups per CU (at most 256 vector registers per lane) so that one wave's unpack and
// scale arithmetic overlaps the other's matrix instructions and memory waits.
//
// Block order: the hardware deals workgroups to the 8 XCDs in turn (block b to XCD b mod 8).
// Each XCD is given a contiguous range of the work list (row block major, then token tile,
// then k split), so the workgroups one XCD runs at the same time share row blocks (their
// weights stay in that XCD's L2) and token tiles (their activations too).
//
// Split-K (a.S > 1, when row blocks x token tiles fill the chip's workgroup slots badly):
// split sp takes units [NU sp / S, NU (sp+1) / S).  Split 0 writes its partial to y, split
// sp > 0 stores its 64 x kGemmTB partial tile per wave to workspace region sp - 1 (ntt *
// kGemmTB token rows x NT * 64 floats: no store needs a bounds test); a second kernel, ordered
// after this one on the stream, adds regions 0 .. S-2 to y in split order (deterministic).  The
// partials are megabytes here, so a second launch is cheaper than making them visible to other
// workgroups inside this kernel.
constexpr int kGemmTB = kGemmTokens;      // tokens per workgroup tile
constexpr int kGemmRS = kUnitK + 8;       // LDS row stride of a staged token (bf16 elements)
constexpr int kXcds = 8;

template <int FMT>
__global__ __launch_bounds__(256, 2) void gemm_kernel(RunArgs a, int nrb, int ntt)
{
    constexpr int NB = Fmt<FMT>::NB, NTB = kGemmTB / 16;
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][kGemmTB * kGemmRS];
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
    const int64_t q = wi / S;
    const int sp = (int)(wi - q * S);
    const int rb = (int)(q / ntt), tt = (int)(q - (int64_t)rb * ntt);
    const int u0 = (int)((int64_t)a.NU * sp / S), u1 = (int)((int64_t)a.NU * (sp + 1) / S);
    const int tile = 4 * rb + w;
    const bool has_tile = tile < a.NT;
    const int tok0 = tt * kGemmTB;

    // activations of unit u for the token tile: thread i stages 16-byte pieces i, i + 256, ...
    // of the kGemmTB x 128 block (token = piece / 16, k octet = piece % 16); rows past T and
    // columns past K are zero
    auto x_fetch = [&](int u, u32x4_t (&xr)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int piece = threadIdx.x + 256 * j, tq = piece >> 4, ko = piece & 15;
            const int t = tok0 + tq, k = u * kUnitK + 8 * ko;
            xr[j] = (t < a.T && k < a.K)
                        ? *reinterpret_cast<const u32x4_t *>(a.x + (int64_t)t * a.K + k)
                        : (u32x4_t){0u, 0u, 0u, 0u};
        }
    };
    auto x_store = [&](int buf, const u32x4_t (&xr)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int piece = threadIdx.x + 256 * j, tq = piece >> 4, ko = piece & 15;
            *reinterpret_cast<u32x4_t *>(&xs[buf][tq * kGemmRS + 8 * ko]) = xr[j];
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
                        &xb[(16 * n + tl) * kGemmRS + 32 * (2 * g + ks) + 8 * oct]);
#define QMAT_GEMM_SLICE(MM, G)                                                                          \
    {                                                                                                   \
        uint32_t b0[4], b1[4];                                                                          \
        bf16x8_of<FMT, 2 * (G), MM>(W, b0);                                                             \
        bf16x8_of<FMT, 2 * (G) + 1, MM>(W, b1);                                                         \
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
    u32x4_t xr[4];
    auto step = [&](int u, Unit<NB, 1> &cur, Unit<NB, 1> &nxt) {
        const int buf = (u - u0) & 1;
        const bool more = u + 1 < u1;
        if (more) {
            x_fetch(u + 1, xr);
            if (has_tile) load_weight_blocks<FMT, 0, kHalves ? NB / 2 : NB>(a, tile, u + 1, lane, nxt);
        }
        if (has_tile) {
            compute(cur, xs[buf], std::integral_constant<int, 0>());
            if constexpr (kHalves)
                if (more) load_weight_blocks<FMT, NB / 2, NB>(a, tile, u + 1, lane, nxt);
            compute(cur, xs[buf], std::integral_constant<int, 1>());
        }
        if (more) x_store(buf ^ 1, xr);
        __syncthreads();
    };

    Unit<NB, 1> wa, wb;
    x_fetch(u0, xr);
    if (has_tile) load_weight_blocks<FMT, 0, NB>(a, tile, u0, lane, wa);
    x_store(0, xr);
    __syncthreads();
    for (int u = u0; u < u1; u += 2) {
        step(u, wa, wb);
        if (u + 1 < u1) step(u + 1, wb, wa);
    }
    if (!has_tile) return;
    f32x4_t rs = (f32x4_t){Fmt<FMT>::kToCode, Fmt<FMT>::kToCode, Fmt<FMT>::kToCode, Fmt<FMT>::kToCode};
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
        // the exact bf16 operands both routes feed to their products, decoded back to the code
        uint32_t b[4];
        bf16x8_of<FMT, KA, MM>(W, b);
        const float sc_f = group_scale(sc, KA >> 1, MM);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t hb = (i & 1) ? (b[i >> 1] & 0xFFFF0000u) : (b[i >> 1] << 16);
            out[i] = sc_f * (__builtin_bit_cast(float, hb) * Fmt<FMT>::kToCode);
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

template <int FMT, int D> static const void *run_kernel_d(int route, int T)
{
    if (route == kRouteMfma)
        return T == 1 ? reinterpret_cast<const void *>(&mfma_kernel<FMT, D, 1>)
                      : reinterpret_cast<const void *>(&mfma_kernel<FMT, D, 4>);
    switch (T) {
    case 1: return reinterpret_cast<const void *>(&valu_kernel<FMT, 1, D>);
    case 2: return reinterpret_cast<const void *>(&valu_kernel<FMT, 2, D>);
    case 3: return reinterpret_cast<const void *>(&valu_kernel<FMT, 3, D>);
    case 4: return reinterpret_cast<const void *>(&valu_kernel<FMT, 4, D>);
    default: return nullptr;
    }
}

template <int FMT> static const void *run_kernel(int route, int T, int depth)
{
    switch (depth) {
    case 1: return run_kernel_d<FMT, 1>(route, T);
    case 2: return run_kernel_d<FMT, 2>(route, T);
    default: return nullptr;
    }
}

static const void *run_kernel_for(int fmt, int route, int T, int depth)
{
    switch (fmt) {
    case 4: return run_kernel<4>(route, T, depth);
    case 5: return run_kernel<5>(route, T, depth);
    case 6: return run_kernel<6>(route, T, depth);
    case 8: return run_kernel<8>(route, T, depth);
    case 9: return run_kernel<9>(route, T, depth);
    default: return nullptr;
    }
}

static size_t run_lds_bytes(int route, int waves, int T, int NU, int S)
{
    (void)route;
    (void)NU;
    (void)S;
    return waves > 1 ? (size_t)waves * T * kTileRows * sizeof(float) : 0;
}

size_t run_lds_bytes_for(int route, int waves, int T, int NU, int S) { return run_lds_bytes(route, waves, T, NU, S); }

hipError_t launch_run(int fmt, int route, int depth, const RunArgs &a, int waves, hipStream_t st)
{
    const void *k = run_kernel_for(fmt, route, a.T, depth);
    if (!k) return hipErrorInvalidValue;
    RunArgs arg = a;
    void *args[] = {&arg};
    const int64_t grid = (int64_t)a.NTt * a.St + (int64_t)(a.NT - a.NTt) * a.S;
    return hipLaunchKernel(k, dim3((unsigned)grid), dim3((unsigned)(64 * waves)), args,
                           run_lds_bytes(route, waves, a.T, a.NU, a.S), st);
}

int run_blocks_per_cu(int fmt, int route, int depth, int T, int waves, int NU, int S)
{
    const void *k = run_kernel_for(fmt, route, T, depth);
    int n = 0;
    if (!k || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, 64 * waves, run_lds_bytes(route, waves, T, NU, S)) !=
                  hipSuccess)
        return 0;
    return n;
}

template <int FMT> static const void *dequant_kernel_ptr() { return reinterpret_cast<const void *>(&dequant_kernel<FMT>); }

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
