// Launch interface of the output-head epilogue kernels (qmat_logits.hip).  Internal: the public
// contract is qmat_logits_* in include/qmat.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmatk {

constexpr int kMaxBlocks = 512;  // row blocks per token at most
constexpr int kLogitsWaves = 4;  // waves per block of the first kernel, one (max, sum) state each

struct LogitsArgs {
    const float *y;         // fp32 logits, row t at y + t * ldy, M entries
    int64_t ldy;
    int M, T, k;            // rows, tokens, entries of the top-k (0 = log-sum-exp only)
    const int32_t *index;   // row -> id map [M], or null (ids are rows)
    float *lse;             // [T] or null
    float *vals;            // [T][k]
    int32_t *ids;           // [T][k]
    float2 *part_lse;       // per (token, block, wave): (max, sum of exp(y - max))   [T][B][kLogitsWaves]
    uint64_t *part_list;    // per (token, block): the k best keys, best first  [T][B][k]
    uint64_t *part_kth;     // per (token, block): the k-th best key (0: none)  [T][B]
    int B, rpb;             // blocks per token (<= kMaxBlocks), rows per block (B * rpb >= M)
};

// Blocks per token for M rows: one round of 8 rows per lane of a 256-thread block (2048 rows) per
// block, at most kMaxBlocks.  A block costs about the same with fewer rows (a round takes 8
// slots per lane), and every block adds a list to the merge, so no more blocks than the rows
// fill, whatever T is.
inline int logits_blocks(int64_t M)
{
    const int64_t b = (M + 2047) / 2048;
    return (int)(b < 1 ? 1 : b > kMaxBlocks ? kMaxBlocks : b);
}

// Both kernels of the epilogue: the blocks' partials, then their merge, one block per token.
hipError_t launch_logits(const LogitsArgs &a, hipStream_t stream);

struct MergeArgs {
    const float2 *lse_part;  // [T][G][kLogitsWaves]
    const uint64_t *kth;     // [T][G]
    const uint64_t *list;    // [T][G][k]
    int G, k;
    const int32_t *index;    // row -> id map [M], or null
    float *lse;              // [T] or null
    float *vals;             // [T][k]
    int32_t *ids;            // [T][k]
};

}  // namespace qmatk
