// Host-side interface of the prefill GEMM route (qmat_gemm.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

#include "qmat_kernels.h"

namespace qmatk {

// Prefill GEMM route: any T >= 1 (tiles of 64 tokens x 256 rows), a.S k splits (1..kGemmMaxS).
// With a.S > 1 it needs gemm_workspace_floats(T, NT, S) floats at a.ws and launches a second
// kernel that adds the splits.
hipError_t launch_gemm(int fmt, const RunArgs &a, hipStream_t stream);
// Largest T of one GEMM call (kept to 65535 token tiles).
constexpr int kGemmMaxT = 65535 * 64;
constexpr int kGemmMaxS = 16;
constexpr int kGemmTokens = 64;   // tokens per GEMM workgroup tile
constexpr int kGemmRowTiles = 4;  // 64-row tiles per GEMM workgroup (one per wave)
inline int gemm_row_blocks(int NT) { return (NT + kGemmRowTiles - 1) / kGemmRowTiles; }
inline int gemm_token_tiles(int T) { return (T + kGemmTokens - 1) / kGemmTokens; }
inline size_t gemm_workspace_floats(int T, int NT, int S)
{
    return S > 1 ? (size_t)(S - 1) * gemm_token_tiles(T) * kGemmTokens * NT * 64 : 0;
}

}  // namespace qmatk
