// A plain HBM read stream: the bandwidth ceiling the product kernels are compared with.
// Measurement support only (libqmat_probe.so); it shares no code with the product kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qmat_probe.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int64_t kChunkBytes = 1024;  // one 16-byte load per lane of a wave

// MODE kRun: wave w reads chunks [w * per_wave, (w + 1) * per_wave) clipped to the buffer;
// kStride: chunks w, w + nw, w + 2 nw, ... for nw launched waves; kBlockRun: workgroup b reads
// chunks [b * per_wave, (b + 1) * per_wave), its waves taking every wpb-th one in turn (the
// order of a product workgroup streaming one tile).  UNR loads in flight; every chunk index is
// checked against its bound.  Dynamic LDS, if any, is only reserved (it caps the workgroups
// per compute unit).
enum { kRun = 0, kStride = 1, kBlockRun = 2 };

template <int UNR, int MODE>
__global__ __launch_bounds__(512) void read_stream_kernel(const u32x4_t *__restrict__ p, int64_t nchunks,
                                                          int per_wave, uint32_t *out)
{
    const int lane = threadIdx.x & 63;
    const int wpb = blockDim.x >> 6;
    const int64_t wave = (int64_t)blockIdx.x * wpb + (threadIdx.x >> 6);
    uint32_t acc = 0;
    int64_t c0, c1, step;
    if constexpr (MODE == kStride) {
        c0 = wave;
        c1 = nchunks;
        step = (int64_t)gridDim.x * wpb;
    } else if constexpr (MODE == kBlockRun) {
        const int64_t b0 = (int64_t)blockIdx.x * per_wave;
        c0 = b0 + (threadIdx.x >> 6);
        c1 = b0 + per_wave < nchunks ? b0 + per_wave : nchunks;
        step = wpb;
    } else {
        c0 = wave * per_wave;
        c1 = c0 + per_wave < nchunks ? c0 + per_wave : nchunks;
        step = 1;
    }
    for (int64_t c = c0; c < c1; c += UNR * step) {
        u32x4_t v[UNR];
#pragma unroll
        for (int i = 0; i < UNR; ++i)
            v[i] = c + i * step < c1 ? __builtin_nontemporal_load(p + (c + i * step) * 64 + lane)
                                     : (u32x4_t){0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < UNR; ++i) acc ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    }
    out[wave * 64 + lane] = acc;
}

// workgroups of one launch, or -1 if the arguments are out of range
int64_t blocks_for(int64_t nbytes, int per_wave, int wpb, int grid_waves)
{
    if (nbytes <= 0 || nbytes % kChunkBytes || wpb < 1 || wpb > 8 || grid_waves < -1 || grid_waves > (1 << 24))
        return -1;
    const int64_t nchunks = nbytes / kChunkBytes;
    if (grid_waves <= 0 && (per_wave < 1 || per_wave > 65536)) return -1;
    int64_t blocks;
    if (grid_waves > 0) blocks = (grid_waves + wpb - 1) / wpb;
    else if (grid_waves == -1) blocks = (nchunks + per_wave - 1) / per_wave;
    else blocks = ((nchunks + per_wave - 1) / per_wave + wpb - 1) / wpb;
    return blocks <= 0x7FFFFFFFLL ? blocks : -1;
}

template <int MODE>
hipError_t launch(int unroll, dim3 grid, dim3 block, int lds, hipStream_t s, const u32x4_t *p, int64_t n, int pw,
                  uint32_t *out)
{
    switch (unroll) {
    case 1: read_stream_kernel<1, MODE><<<grid, block, lds, s>>>(p, n, pw, out); break;
    case 2: read_stream_kernel<2, MODE><<<grid, block, lds, s>>>(p, n, pw, out); break;
    case 4: read_stream_kernel<4, MODE><<<grid, block, lds, s>>>(p, n, pw, out); break;
    case 8: read_stream_kernel<8, MODE><<<grid, block, lds, s>>>(p, n, pw, out); break;
    case 16: read_stream_kernel<16, MODE><<<grid, block, lds, s>>>(p, n, pw, out); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

extern "C" {

int64_t qmat_probe_read_out_words(int64_t nbytes, int per_wave, int waves_per_block, int grid_waves)
{
    const int64_t blocks = blocks_for(nbytes, per_wave, waves_per_block, grid_waves);
    return blocks < 0 ? 0 : blocks * waves_per_block * 64;
}

int qmat_probe_read(const void *buf, int64_t nbytes, int per_wave, int grid_waves, int unroll, int waves_per_block,
                    int lds_bytes, uint32_t *out, int64_t out_words, void *stream)
{
    if (!buf || reinterpret_cast<uintptr_t>(buf) % 16 || !out) return 1;
    if (!(unroll == 1 || unroll == 2 || unroll == 4 || unroll == 8 || unroll == 16)) return 1;
    if (lds_bytes < 0 || lds_bytes > 65536) return 1;
    const int64_t blocks = blocks_for(nbytes, per_wave, waves_per_block, grid_waves);
    if (blocks < 0 || out_words < blocks * waves_per_block * 64) return 1;
    const u32x4_t *p = static_cast<const u32x4_t *>(buf);
    const dim3 grid((unsigned)blocks), block(64 * waves_per_block);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t n = nbytes / kChunkBytes;
    const hipError_t e = grid_waves > 0    ? launch<kStride>(unroll, grid, block, lds_bytes, s, p, n, per_wave, out)
                         : grid_waves == -1 ? launch<kBlockRun>(unroll, grid, block, lds_bytes, s, p, n, per_wave, out)
                                            : launch<kRun>(unroll, grid, block, lds_bytes, s, p, n, per_wave, out);
    return e == hipSuccess ? 0 : 5;
}

}  // extern "C"
