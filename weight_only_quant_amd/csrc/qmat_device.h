// Device code shared by the small-T kernels (qmat_kernels.hip) and the prefill GEMM
// (qmat_gemm.hip): vector types, the per-format constants and the exact code -> bf16
// conversions, and the per-lane unit of packed weights.  The conversions are described at the
// top of qmat_kernels.hip; the packed layout in qmat_layout.h.
#pragma once

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
// NB: 1 KB blocks per unit.  bf16x8_of turns each code into an exact bf16 operand u with
// u * kToCode = code + kOffset: Q4 (code + 8) / 512, read by the FP8 converter from an
// offset-binary nibble; Q5 8*code, Q6 4*code, Q8 the code, no offset.  bf16x8_signed (the
// vector-ALU route, and the Q4 kernels where removing the offset costs more than the shorter
// unpack saves) gives u * kSignedToCode = code (Q4 code/16).  The factor is applied once per row
// at the end.
template <> struct Fmt<4> {
    static constexpr int NB = 4;
    static constexpr float kToCode = 512.0f, kOffset = 8.0f, kSignedToCode = 16.0f;
};
template <> struct Fmt<5> {
    static constexpr int NB = 5;
    static constexpr float kToCode = 0.125f, kOffset = 0.0f, kSignedToCode = 0.125f;
};
template <> struct Fmt<6> {
    static constexpr int NB = 6;
    static constexpr float kToCode = 0.25f, kOffset = 0.0f, kSignedToCode = 0.25f;
};
template <> struct Fmt<8> {
    static constexpr int NB = 8;
    static constexpr float kToCode = 1.0f, kOffset = 0.0f, kSignedToCode = 1.0f;
};
template <> struct Fmt<9> {
    static constexpr int NB = 8;
    static constexpr float kToCode = 1.0f, kOffset = 0.0f, kSignedToCode = 1.0f;
};

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

// The 8 codes of row m in k step KA of a unit, as exact floats equal to code / kSignedToCode.
// W: the lane's 4*NB dwords of the unit (layout in qmat_layout.h).
template <int FMT, int KA, int MM>
__device__ __forceinline__ void codes8(const uint32_t *W, float (&f)[8])
{
    if constexpr (FMT == 4) {
        // e = i sits in bits [3:0] of byte i, e = 4 + i in bits [7:4]; v_cvt_off_f32_i4 reads
        // the low four bits of the byte SDWA selects as code/16, so the high nibbles take one
        // rotate (a rotate rather than a shift keeps h opaque to the compiler, so its bytes are
        // SDWA-selected too instead of being re-extracted from n)
        const uint32_t n = W[4 * KA + MM], h = __builtin_amdgcn_alignbit(n, n, 4);
        f[0] = nib_lo<0>(n); f[1] = nib_lo<1>(n);
        f[2] = nib_lo<2>(n); f[3] = nib_lo<3>(n);
        f[4] = nib_lo<0>(h); f[5] = nib_lo<1>(h);
        f[6] = nib_lo<2>(h); f[7] = nib_lo<3>(h);
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

// bf16 pair of E4M3 bytes (SEL ? 2, 3 : 0, 1) of w, exact (every E4M3 value fits in bf16)
template <bool SEL> __device__ __forceinline__ uint32_t e4m3_pair(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, SEL));
}

// The 8 weights of row m in k step KA as 4 dwords of bf16 pairs (k, k+1), exact: groupwise
// (code + kOffset) / kToCode, FP8 the E4M3 value.
//
// Q4: the E4M3 bytes 0..15 are the values v * 2^-9 (0..7 subnormal, 8..15 the first normal
// binade), so a byte holding the offset-binary nibble v = code + 8 (the two's complement nibble
// with its top bit flipped) converts to (code + 8) / 512 with no arithmetic; one XOR and masks
// of the low and the high nibbles of a dword give the 8 bytes, and the converter turns two of
// them into a bf16 pair per instruction: 8 instructions per 8 codes against 13 for signed
// nibble converts and packs.  The +8 is taken out of each group's product sum
// (q4_group_offset).
template <int FMT, int KA, int MM>
__device__ __forceinline__ void bf16x8_of(const uint32_t *W, uint32_t (&b)[4])
{
    if constexpr (FMT == 8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t w = W[8 * KA + 2 * MM + h];
            b[2 * h + 0] = e4m3_pair<false>(w);
            b[2 * h + 1] = e4m3_pair<true>(w);
        }
    } else if constexpr (FMT == 4) {
        const uint32_t n = W[4 * KA + MM] ^ 0x88888888u;
        const uint32_t lo = n & 0x0F0F0F0Fu, hi = (n >> 4) & 0x0F0F0F0Fu;
        b[0] = e4m3_pair<false>(lo);
        b[1] = e4m3_pair<true>(lo);
        b[2] = e4m3_pair<false>(hi);
        b[3] = e4m3_pair<true>(hi);
    } else {
        float f[8];
        codes8<FMT, KA, MM>(W, f);
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = pack_bf16(f[2 * i], f[2 * i + 1]);
    }
}

// The same 8 weights without offset: code / kSignedToCode (FP8: the E4M3 value).
template <int FMT, int KA, int MM>
__device__ __forceinline__ void bf16x8_signed(const uint32_t *W, uint32_t (&b)[4])
{
    if constexpr (FMT == 4) {
        float f[8];
        codes8<FMT, KA, MM>(W, f);
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = pack_bf16(f[2 * i], f[2 * i + 1]);
    } else {
        bf16x8_of<FMT, KA, MM>(W, b);
    }
}

// What Q4's offset adds to a group's product sum: the two 32-wide k steps' activation
// fragments (A operands) against a constant B of 8/512 = 2^-6 (bf16 0x3C80) give, in every D
// component, (8/512) times the token's sum of the group's 64 activations.  The product sum over
// the offset operands minus this value is sum(code * x) / 512.  For a group of zero codes the
// two are the same matrix-core computation on the same bits (every operand 2^-6), so the
// difference is exactly 0: zero and sparse rows keep the accuracy of the signed operands.
__device__ __forceinline__ f32x4_t q4_group_offset(const u32x4_t &x0, const u32x4_t &x1)
{
    static_assert(Fmt<4>::kOffset / Fmt<4>::kToCode == 0.015625f, "offset constant is 2^-6");
    const bf16x8_t c = __builtin_bit_cast(bf16x8_t, (u32x4_t){0x3C803C80u, 0x3C803C80u, 0x3C803C80u, 0x3C803C80u});
    f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x0), c,
                                                         (f32x4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x1), c, d, 0, 0, 0);
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

// What one lane needs for one 128-wide k unit: its NB packed code slots, its scale slot and the
// XN vectors of 8 bf16 activations the unit multiplies.
template <int NB, int XN> struct Unit {
    u32x4_t c[NB];
    u32x4_t sc;
    u32x4_t x[XN];
};

}  // namespace qmatk
