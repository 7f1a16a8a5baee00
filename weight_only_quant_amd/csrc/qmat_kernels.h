// Kernel launch interface between the host API (qmat_api.cpp) and the gfx950 kernels
// (qmat_kernels.hip).  Internal: not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmatk {

// One launch of the product kernel: tokens [0, T) of x/y as passed (the caller offsets x and y
// for multi-pass launches), all rows, the k units split over S workgroups x NW waves per tile.
struct RunArgs {
    const uint8_t *codes;   // packed code blocks
    const uint8_t *scales;  // packed scale blocks
    const uint16_t *x;      // bf16 [T][K]
    float *y;               // fp32 [T][ldy]
    float *ws;              // split-K partials [S][T][Mpad] (S > 1 only)
    uint32_t *counters;     // one arrival counter per tile (S > 1 only), zero between launches
    int64_t ldy;            // row stride of y in elements (M)
    int M, K, T, NT, NU, S, Mpad;
};

struct DequantArgs {
    const uint8_t *codes;
    const uint8_t *scales;
    float *w;  // fp32 [M][K]
    int M, K, NT, NU;
};

enum Route { kRouteValu = 1, kRouteMfma = 2 };

// Tokens one vector-ALU launch handles; larger T runs as several launches.
constexpr int kValuMaxT = 4;

// depth: k units in flight per wave (1..kMaxDepth).
constexpr int kMaxDepth = 2;
hipError_t launch_run(int fmt, int route, int depth, const RunArgs &a, int waves, hipStream_t stream);
hipError_t launch_dequant(int fmt, const DequantArgs &a, hipStream_t stream);

// Workgroups of (64 * waves) threads of the product kernel for (fmt, route, T) that one compute
// unit holds at once (0 on error).
int run_blocks_per_cu(int fmt, int route, int depth, int T, int waves, int NU, int S);

// Dynamic LDS bytes of one product launch (activation stage + reduction area).
size_t run_lds_bytes_for(int route, int waves, int T, int NU, int S);

// Dynamic LDS one workgroup may use.
constexpr size_t kMaxLds = 64 * 1024;

}  // namespace qmatk
