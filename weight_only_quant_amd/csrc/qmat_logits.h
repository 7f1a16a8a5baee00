// Launch interface of the output-head epilogue kernel (qmat_logits.hip).  Internal: the public
// contract is qmat_logits_* in include/qmat.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmatk {

struct LogitsArgs {
    const float *y;         // fp32 logits, row t at y + t * ldy, M entries
    int64_t ldy;
    int M, T, k;            // rows, tokens, entries of the top-k (0 = log-sum-exp only)
    const int32_t *index;   // row -> id map [M], or null (ids are rows)
    float *lse;             // [T] or null
    float *vals;            // [T][k]
    int32_t *ids;           // [T][k]
    float *part_f;          // per (token, block): max, sum, k best values   [T][B][2 + k]
    int32_t *part_i;        // per (token, block): rows of the k best        [T][B][k]
    uint32_t *counter;      // per token arrival counter, zero between launches
    int B, rpb;             // blocks per token, rows per block
};

// Blocks per token for M rows (each block of 16 waves streams about 4096 rows: one round of
// four 64-row loads per wave).
inline int logits_blocks(int64_t M)
{
    int64_t b = (M + 4095) / 4096;
    return (int)(b < 1 ? 1 : b > 512 ? 512 : b);
}

// Workgroups of the epilogue kernel one compute unit holds at once (0 if unknown).
int logits_blocks_per_cu();

hipError_t launch_logits(const LogitsArgs &a, hipStream_t stream);

}  // namespace qmatk
