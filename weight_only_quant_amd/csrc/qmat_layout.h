// Packed layout of qmat matrices: constants shared by the host packer and the gfx950 kernels.
//
// A matrix W[M][K] is cut into 64-row tiles (NT = ceil(M/64)) and 128-wide k units
// (NU = ceil(K/128), two 64-weight groups per unit).  Every (tile, unit) owns NB blocks of
// 1024 bytes, one 16-byte slot per lane of a 64-lane wave: block j of unit u of tile t is at
//     codes + ((t * NU + u) * NB + j) * 1024,  lane L's slot at + 16 * L.
// Lane L of the wave that owns a tile covers rows rho(L, m) = 16*m + (L % 16), m = 0..3, and
// inside each 32-wide k step kappa (0..3 in a unit) the 8 columns 32*kappa + 8*(L / 16) + e,
// e = 0..7.  This is the operand layout of the gfx950 16x16x32 bf16 MFMA (lane L supplies
// matrix row L % 16 and k octet L / 16), so the same bytes feed the vector-ALU and the MFMA
// kernels.  Concatenating a lane's slots of one unit gives 4*NB dwords W[0 .. 4*NB-1]
// (W[4*j + d] = dword d of block j):
//
//   Q4  (NB 4): W[4*kappa + m] holds the 8 codes of row m: byte i has e = i in bits [3:0]
//               and e = 4 + i in bits [7:4], two's complement nibbles (flipping every
//               nibble's top bit and masking the low or the high nibbles leaves bytes that read
//               as E4M3 values (code + 8) * 2^-9: the offset-operand route).
//   Q5  (NB 5): W[5*kappa + 0..4] = X0 X1 X2 X3 E.  Output dword o (0..7) carries the codes of
//               row o/2, e = 4*(o%2) + i in byte i, each byte = code << 3 (a signed byte worth
//               8*code).  O_d = X_d & 0xF8F8F8F8 for d < 4; for d < 4 the low 3 bits of each byte
//               of X_d are bits [4:2] of output dword 4+d's code, and E bits [8i+2d+1 : 8i+2d]
//               are its bits [1:0].
//   Q6  (NB 6): W[6*kappa + 3*p + 0..2] = A B C for rows m0 = 2p, m1 = 2p + 1.  A, B, C hold in
//               bits [7:2] of byte i the codes (m0, e=i), (m0, e=4+i), (m1, e=i) (signed byte =
//               4*code); their bits [1:0] hold bits [5:4], [3:2], [1:0] of code (m1, e=4+i).
//   FP8 (NB 8): W[8*kappa + 2*m + h] holds the E4M3 bytes of row m, e = 4h + i in byte i.
//   Q8  (NB 8): the same byte order, each byte an 8-bit two's complement code.
//
// Format ids: 4, 5, 6 groupwise with that many bits; 9 groupwise 8-bit (Q8); 8 row-scaled FP8.
// Scales: groupwise, one 256-byte block per (tile, unit) at scales + (t*NU + u)*256; lane L reads
// 16 bytes at + 16*(L % 16): binary16 of (row rho(L, m), group 2u + g) at index 4*g + m.
// FP8: one 256-byte block per tile at scales + t*256; fp32 of row rho(L, m) at index 4*(L%16) + m.
// Padding rows (>= M) and padding groups (>= K/64) carry code 0 and scale 0.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace qmatk {

constexpr int kTileRows = 64;
constexpr int kUnitK = 128;
constexpr int kGroup = 64;
constexpr int kBlockBytes = 1024;
constexpr int kScaleBlockBytes = 256;
constexpr int kMaxT = 16;

constexpr int kFmtFp8 = 8;  // row-scaled FP8 E4M3
constexpr int kFmtQ8 = 9;   // groupwise 8-bit codes

constexpr int blocks_per_unit(int fmt)
{
    return fmt == 4 ? 4 : fmt == 5 ? 5 : fmt == 6 ? 6 : (fmt == kFmtFp8 || fmt == kFmtQ8) ? 8 : 0;
}

// bits per code of a groupwise format, 0 for FP8
constexpr int group_code_bits(int fmt)
{
    return (fmt == 4 || fmt == 5 || fmt == 6) ? fmt : fmt == kFmtQ8 ? 8 : 0;
}

inline bool format_ok(int fmt) { return blocks_per_unit(fmt) != 0; }

inline int64_t num_tiles(int64_t M) { return (M + kTileRows - 1) / kTileRows; }
inline int64_t num_units(int64_t K) { return (K + kUnitK - 1) / kUnitK; }

inline size_t code_bytes(int fmt, int64_t M, int64_t K)
{
    return (size_t)num_tiles(M) * (size_t)num_units(K) * (size_t)blocks_per_unit(fmt) * kBlockBytes;
}

inline size_t scale_bytes(int fmt, int64_t M, int64_t K)
{
    return fmt == kFmtFp8 ? (size_t)num_tiles(M) * kScaleBlockBytes
                    : (size_t)num_tiles(M) * (size_t)num_units(K) * kScaleBlockBytes;
}

}  // namespace qmatk
