/*
 * qmat_probe — a plain HBM read stream for AMD MI355X (gfx950), the practical bandwidth
 * ceiling that the product kernels of qmat.h are measured against.  Measurement support
 * only: it is not part of the product path and shares no code with it.
 *
 * The kernel reads a device buffer once, in 1 KB chunks (one 16-byte nontemporal load per
 * lane of a 64-lane wave), each wave keeping `unroll` loads in flight, and folds what it read
 * into one 32-bit word per lane so the loads cannot be dropped.  Waves take consecutive runs of
 * chunks, or every grid_waves-th chunk, or workgroups take runs that their waves interleave
 * (the order of a product workgroup streaming a tile), and the workgroup size and an LDS
 * reservation set how many waves a compute unit runs at once.  The best launch shape over a
 * small sweep on a buffer much larger than the last-level caches is the practical ceiling of
 * a streaming kernel on this GPU.
 *
 * Conventions as in qmat.h: status return (0 on success, never throws), device pointers of
 * the current device, stream = hipStream_t as void* (NULL = null stream), asynchronous,
 * no allocation.  Built as its own library (libqmat_probe.so).
 */
#ifndef QMAT_PROBE_H
#define QMAT_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Words of `out` that qmat_probe_read needs for these arguments: one per lane of every launched
 * wave.  0 if the arguments are invalid (as qmat_probe_read checks them). */
int64_t qmat_probe_read_out_words(int64_t nbytes, int per_wave, int waves_per_block, int grid_waves);

/* Read nbytes of buf (device, 16-byte aligned) once.
 *   nbytes:          > 0, a multiple of 1024.
 *   per_wave:        with grid_waves == 0, each wave reads per_wave consecutive 1 KB chunks
 *                    (1 .. 65536) and the grid covers the buffer.
 *   grid_waves:      if > 0 (at most 2^24), that many waves instead, wave w reading chunks
 *                    w, w + grid_waves, w + 2 grid_waves, ... (per_wave is not read);
 *                    if -1, each workgroup reads per_wave consecutive chunks, its waves
 *                    taking every waves_per_block-th chunk of the run in turn.
 *   unroll:          loads in flight per wave: 1, 2, 4, 8 or 16.
 *   waves_per_block: waves per workgroup, 1 .. 8.
 *   lds_bytes:       dynamic LDS per workgroup, 0 .. 65536: unused memory whose only effect is
 *                    to cap how many workgroups a compute unit holds at once.
 *   out:             device uint32 [out_words], out_words >= qmat_probe_read_out_words(...);
 *                    receives the fold of the data (a value with no meaning beyond keeping
 *                    the loads live).
 * Returns 0, 1 (invalid argument: a null or misaligned pointer, a size or count outside its
 * range, out too small, a grid beyond 2^31 - 1 workgroups) or 5 (launch failure). */
int qmat_probe_read(const void *buf, int64_t nbytes, int per_wave, int grid_waves, int unroll,
                    int waves_per_block, int lds_bytes, uint32_t *out, int64_t out_words,
                    void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QMAT_PROBE_H */
