// Kernel launch interface between the host API (qmat_api.cpp) and the gfx950 kernels
// (qmat_kernels.hip).  Internal: not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmatk {

// 64-bit tree-node words one launch needs to sum the partial tiles of tiles shared by several
// workgroups (S - 1 nodes per element of a tile shared S ways; 0 when no tile is shared).
inline size_t run_node_words(int T, int NT, int S, int NTt, int St)
{
    size_t f = 0;
    if (S > 1) f += (size_t)(S - 1) * T * (size_t)(NT - NTt) * 64;
    if (NTt > 0 && St > 1) f += (size_t)(St - 1) * T * (size_t)NTt * 64;
    return f;
}

// One launch of the product kernel: tokens [0, T) of x/y as passed (the caller offsets x and y
// for multi-pass launches), all rows.  The leading NT - NTt row tiles have their k units split
// over S workgroups x NW waves each; the trailing NTt tiles over St workgroups x NW waves.  The
// grid is NTt * St + (NT - NTt) * S workgroups, the trailing tiles' workgroups first.
struct RunArgs {
    const uint8_t *codes;   // packed code blocks
    const uint8_t *scales;  // packed scale blocks
    const uint16_t *x;      // bf16 [T][K]
    float *y;               // fp32 [T][ldy]
    float *ws;              // GEMM route: split-K partials (scratch)
    uint64_t *nodes;        // small-T routes: tree-node words of the shared tiles, all zero between
                            // calls: leading tiles [S-1][T][(NT-NTt)*64] when S > 1, then
                            // trailing tiles [St-1][T][NTt*64] when St > 1
    int64_t ldy;            // row stride of y in elements (M)
    int M, K, T, NT, NU, S;
    int NTt, St;            // trailing tiles and their k splits (NTt == 0: every tile uses S)
};

struct DequantArgs {
    const uint8_t *codes;
    const uint8_t *scales;
    float *w;  // fp32 [M][K]
    int M, K, NT, NU;
};

enum Route { kRouteValu = 1, kRouteMfma = 2, kRouteGemm = 3 };

// Tokens one vector-ALU launch handles; larger T runs as several launches.
constexpr int kValuMaxT = 4;

// depth: k units in flight per wave (1..kMaxDepth).
constexpr int kMaxDepth = 2;
// tiles: row tiles per wave, 1 or 2 (2: MFMA route and a.NTt == 0 only; the grid is then
// ceil(NT / 2) * S workgroups).
// offset_ops: on the MFMA route, Q4 up to 8 tokens takes offset-binary operands (every other
// case, and every case without it, takes two's complement operands).
hipError_t launch_run(int fmt, int route, int depth, const RunArgs &a, int waves, int tiles, bool offset_ops,
                      hipStream_t stream);
hipError_t launch_dequant(int fmt, const DequantArgs &a, hipStream_t stream);


// Workgroups of (64 * waves) threads of the product kernel for (fmt, route, T) that one compute
// unit holds at once (0 on error).
int run_blocks_per_cu(int fmt, int route, int depth, int T, int waves, int S);

}  // namespace qmatk
