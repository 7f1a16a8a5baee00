/*
 * qmat — weight-only quantized small-T matrix-activation product for AMD MI355X (gfx950).
 *
 *     y[T][M] = x[T][K] . W^T          1 <= T <= 16, bf16 x, fp32 y
 *
 * W is stored in one of two weight-only formats described on the NInfer model cards:
 *
 *  - Groupwise Q4 / Q5 / Q6 ("Qwen3.8-27B for NInfer on the RTX 3090", section "What is
 *    different from the upstream artifact"): every run of 64 weights along a row (along
 *    K) shares one IEEE binary16 scale; each weight is that scale times a b-bit two's
 *    complement code c in [-2^(b-1), 2^(b-1)-1].  A negative scale is legal; it lets a group
 *    whose largest weight is positive map it to -2^(b-1), the code without a positive twin.
 *        w[i][j] = fp32(scale[i][j/64]) * code[i][j]            (exact in fp32)
 *    Groupwise Q8 is the same definition with 8-bit codes in [-128, 127]: the cards' format
 *    tables store the token embedding, the upstream output head and several projections so.
 *  - Row-scaled FP8 ("Qwen3.8-27B NVFP4 for NInfer", introduction and "Artifact"): one
 *    scale per row times an FP8 value.  The FP8 encoding is OCP E4M3 ("FN": bias 7, no
 *    infinities, S.1111.111 is NaN, largest finite 448) and the row scale is fp32.
 *        w[i][j] = fl32(r[i] * e4m3(b[i][j]))
 *
 * The library packs W once on the host (qmat_pack) into a layout made for gfx950 wave64
 * loads, then streams it from HBM once per call (qmat_run).  qmat_dequant expands the
 * packed matrix back to fp32 for bit-exact checking.
 *
 * Conventions for every function:
 *  - Return value: qmat_status (0 on success).  Nothing throws across this boundary.
 *    After a failure, qmat_last_error() returns a message for the calling thread.
 *  - "host" pointers are ordinary CPU memory; "device" pointers are HIP device memory of
 *    the current device.  The library never frees caller memory.
 *  - A handle (qmat_t, qmat_logits_t) belongs to the device that was current when it was
 *    created; a call on it, or a view of it, made while another device is current returns
 *    QMAT_EINVAL.
 *  - stream: a hipStream_t passed as void* (NULL = the null stream).  qmat_run and
 *    qmat_dequant are asynchronous on that stream, allocate nothing, never synchronize,
 *    and may be captured into a HIP graph.
 *  - Row-major everywhere: x is [T][K] bf16 (K contiguous), y is [T][M] fp32.
 */
#ifndef QMAT_H
#define QMAT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QMAT_OK = 0,
    QMAT_EINVAL = 1, /* bad format, null pointer, bad handle, bad route */
    QMAT_ESHAPE = 2, /* M < 1, K < 64, K % 64 != 0; T < 0, or T above the route's limit (16 on
                        the small-T routes, 4194240 on the GEMM route that qmat_run takes for
                        T > 16) */
    QMAT_ERANGE = 3, /* code outside the format's range, NaN FP8 byte, non-finite scale */
    QMAT_ESIZE = 4,  /* a buffer is smaller than required, or a launch shape exceeds the workspace */
    QMAT_EHIP = 5,   /* a HIP runtime call or kernel launch failed */
    QMAT_ENOMEM = 6  /* host or device allocation failed */
} qmat_status;

typedef enum {
    QMAT_Q4 = 4,           /* groupwise 4-bit codes, FP16 scale per 64 weights */
    QMAT_Q5 = 5,           /* groupwise 5-bit */
    QMAT_Q6 = 6,           /* groupwise 6-bit */
    QMAT_FP8_E4M3_ROW = 8, /* OCP E4M3 bytes, fp32 scale per row */
    QMAT_Q8 = 9            /* groupwise 8-bit (the value is not the bit width: 8 is FP8) */
} qmat_format;

typedef enum {
    QMAT_ROUTE_AUTO = 0, /* the library's choice for (format, shape, T) */
    QMAT_ROUTE_VALU = 1, /* vector-ALU dot products; T > 4 runs as several passes */
    QMAT_ROUTE_MFMA = 2, /* bf16 matrix-core tiles (16 tokens x 16 rows x 32 k) */
    QMAT_ROUTE_GEMM = 3, /* prefill-sized T: 64-token x 256-row matrix-core tiles, activations
                            staged in LDS; the automatic route for T > 16 */
    QMAT_ROUTE_MFMA_OFFSET = 4 /* QMAT_ROUTE_MFMA, except that Q4 codes up to 8 tokens reach
                            the matrix cores as offset-binary operands (code + 8) read by the FP8
                            converter, and each group's sum over a constant operand takes the
                            offset out again: 3-5% faster on Q4 at T <= 8 (every other format
                            and T runs the same kernels as QMAT_ROUTE_MFMA).  Groups of zero codes
                            stay exact, but the fp32 rounding scales with the sum of |x| over a
                            group instead of the sum of |code * x|, so the error bound
                            1e-4 * sum|w x| + 1e-6 holds only while a row's products are not
                            dwarfed by activations that meet zero codes (measured 15-48x over the
                            bound on rows of half zero codes with 2^18x larger activations on
                            them).  Explicit requests only. */
} qmat_route;

typedef struct qmat *qmat_t;

/* Size in bytes of the packed blob for an M x K matrix, or 0 if (fmt, M, K) is invalid.
 * Layout (all offsets from the start of the blob; 64-row tiles, NT = ceil(M/64);
 * 128-wide k units, NU = ceil(K/128)):
 *   codes:  NT * NU * NB blocks of 1024 bytes, NB = 4 (Q4), 5 (Q5), 6 (Q6), 8 (Q8, FP8);
 *   scales: groupwise NT * NU * 256 bytes (fp16 [tile][unit][row%16][group in unit][row/16]);
 *           FP8 NT * 256 bytes (fp32 [tile][row%16][row/16]).
 * The byte order inside a block is documented in the repository's design notes.
 * Rows past M and groups past K/64 are zero-filled. */
size_t qmat_packed_bytes(int fmt, int64_t M, int64_t K);

/* Pack a matrix into the layout above.  Host only; pure; thread-safe.
 * What is stored is exactly the information of the formats' definitions: the b-bit two's
 * complement codes and one FP16 scale per 64-weight group along K ("Qwen3.8-27B for NInfer on
 * the RTX 3090", "What is different from the upstream artifact"), or the E4M3 bytes and one
 * scale per row of the row-scaled FP8 tensors ("Qwen3.8-27B NVFP4 for NInfer", "Artifact"); the
 * engine on those pages likewise re-encodes tensors once, at load ("Qwen3.8-27B for NInfer on
 * the RTX 3090", "Measurements": the embedding transcoded to 4 bits at load).
 *   codes:  groupwise: int8 [M][K], each in [-2^(b-1), 2^(b-1)-1] (b = 4, 5, 6, or 8 for Q8);
 *           FP8: uint8 [M][K] E4M3 bytes (0x7F / 0xFF, the NaNs, are rejected).
 *   scales: groupwise: uint16 [M][K/64] binary16 bit patterns, finite, any sign;
 *           FP8: float [M], finite.
 *   out:    host buffer of out_bytes >= qmat_packed_bytes(fmt, M, K); fully written.
 * Errors: QMAT_EINVAL (fmt, null), QMAT_ESHAPE (M, K), QMAT_ERANGE (code or scale value,
 * with the first offending index in the message), QMAT_ESIZE (out_bytes). */
int qmat_pack(int fmt, int64_t M, int64_t K, const void *codes, const void *scales, void *out,
              size_t out_bytes);

typedef enum {
    QMAT_ENCODE_RTN = 0,            /* upstream: scale = max|w| / qmax, nearest codes (FP8: the
                                       row maximum maps to 448) */
    QMAT_ENCODE_GROUPED_SEARCH = 1  /* groupwise only: FP16 scale searched over 50 candidates of
                                       both signs for the least importance-weighted error */
} qmat_encoder;

/* Quantize fp32 weights w [M][K] (host) into the logical arrays qmat_pack takes.  Host only;
 * pure; thread-safe.
 *  Groupwise (Q4, Q5, Q6, Q8), per 64-weight group along K, a = max |w| of the group:
 *   - QMAT_ENCODE_RTN, upstream's encoder ("Qwen3.8-27B for NInfer on the RTX 3090", "What is
 *     different from the upstream artifact"): scale = FP16(a / qmax), code = nearest integer
 *     to w / scale, clamped to [-2^(b-1), qmax] (qmax = 2^(b-1) - 1).
 *   - QMAT_ENCODE_GROUPED_SEARCH, that artifact's encoder (same section): the FP16 scale is the
 *     candidate with the least sum_j importance[k_j] * (w_j - scale * code_j)^2 among the 50
 *     candidates +-a / (qmax + i/24), i = 0..24 (ordered +, - for each i; the first of equal
 *     errors wins), with codes taken against each candidate as for RTN.  Negative scales let a
 *     group reach the most negative code.  importance: float [K] per input channel (the mean
 *     squared activation of that channel, an imatrix), finite and >= 0; NULL means all 1.
 *   Every FP16 scale is rounded once (nearest-even) from the double quotient; codes round half
 *   to even.  An all-zero group gets scale +0 and codes 0.
 *   Outputs: codes int8 [M][K], scales uint16 binary16 bits [M][K/64].
 *  Row-scaled FP8: QMAT_ENCODE_RTN only.  r = fl32(a / 448) with a the row's max |w|; each byte
 *   is the E4M3 value nearest (even ties, saturating at +-448) to fl32(w / r); an all-zero row
 *   gets r = 0 and zero bytes.  Outputs: codes uint8 [M][K], scales float [M].
 * Errors: QMAT_EINVAL (format, encoder, null pointer, FP8 with the grouped search),
 * QMAT_ESHAPE (M, K), QMAT_ERANGE (non-finite weight or importance, negative importance, a
 * group whose a / qmax overflows FP16). */
int qmat_quantize(int fmt, int64_t M, int64_t K, const float *w, const float *importance, int encoder,
                  void *codes_out, void *scales_out);

/* Create a handle over a packed matrix already in device memory: the weight operand of the
 * decode and verify products whose speed the pages measure ("Qwen3.8-27B for NInfer on the
 * RTX 3090", "Measurements": the 6-bit output head under an 8-token verify).
 *   packed_dev: device pointer to qmat_pack's output (bytes == qmat_packed_bytes, 16-byte
 *               aligned).  Borrowed: it must outlive the handle and is never written.
 * The handle owns a device workspace that it allocates and zero-fills here: the tree words
 * that sum the partial results of row tiles whose K range is split across workgroups (every
 * call leaves them zero again), and, for matrices of fewer than 1024 rows per CU, up to 32 MB
 * for the GEMM route's k splits.  Calls that share one handle must therefore be ordered (one
 * stream, or synchronized streams).
 * Errors: QMAT_EINVAL, QMAT_ESHAPE, QMAT_ESIZE (bytes mismatch), QMAT_ENOMEM, QMAT_EHIP. */
int qmat_create(qmat_t *handle, int fmt, int64_t M, int64_t K, const void *packed_dev, size_t bytes);

/* A handle over rows [row0, row0 + rows) of an existing handle's matrix, sharing its packed
 * device memory (no copy): for example the gate and the up halves of a gate+up matrix packed
 * as one (the giveen/ninfer-ext README, "Flash-Next speed", "How it got here": projection splits
 * taken as views of one weight instead of device copies).
 *   row0: a multiple of 64 (a tile boundary); rows >= 1; row0 + rows <= the parent's M.
 * The view behaves as an M = rows matrix in every call (y is [T][rows]).  It borrows the packed
 * memory the parent borrows (which must outlive both) but not the parent handle itself, which
 * may be destroyed first; it owns its own split-K workspace, allocated here.
 * Errors: QMAT_EINVAL (null pointers), QMAT_ESHAPE (row range), QMAT_ENOMEM, QMAT_EHIP. */
int qmat_create_view(qmat_t *view, qmat_t parent, int64_t row0, int64_t rows);

/* y = x . W^T, with W as the format defines it (w = fp32(scale) * code per 64-weight group,
 * "Qwen3.8-27B for NInfer on the RTX 3090", "What is different from the upstream artifact";
 * w = fl32(r * e4m3) per row, "Qwen3.8-27B NVFP4 for NInfer", "Artifact") applied to T tokens:
 * T = 1 is decode, T <= 16 a speculative verify of up to 15 drafts (the NVFP4 card's "Artifact"
 * section; the RTX 3090 card's "Measurements" times the head's 8-token verify).  y is computed
 * with fp32 accumulation of exact bf16 products; it agrees with the exact sum to within
 * 1e-4 * sum_j |w_ij x_tj| + 1e-6 per element.
 * x: device bf16 [T][K] (16-byte aligned); y: device fp32 [T][M], fully overwritten.  T == 0 is a no-op.  Decode and verify sizes (T <= 16) take the small-T routes;
 * prefill sizes (17 <= T <= 4194240) the GEMM route, where each unpacked weight feeds the
 * matrix cores for 64 tokens (the pages' prefill, where the groupwise route is capped by the
 * 4-bit -> bf16 decoding: "Qwen3.6-35B-A3B NVFP4" / "Qwen3.8-27B EXL3" speed notes).  When a
 * narrow matrix at a small prefill T gives too few tiles to fill the GPU, the GEMM route splits
 * K and sums the splits through the workspace in a fixed order (deterministic).
 * Asynchronous on stream; no allocation, no sync.
 * Errors: QMAT_EINVAL (null handle/pointers, misaligned x), QMAT_ESHAPE (T < 0 or too large),
 * QMAT_EHIP (launch failure). */
int qmat_run(qmat_t handle, const void *x_dev, float *y_dev, int T, void *stream);

/* qmat_run for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same product, the same automatic
 * plan and the same kernels as qmat_create + qmat_run, without a handle and without any
 * allocation.  The library plans the launch on the host and keeps what the kernels need beyond
 * x, y and the packed matrix in one static device array per GPU (32 MiB, held by each GPU the
 * library runs on until the process ends): 8 MiB of tree words that sum a row tile's partial
 * results when K is split across workgroups (zero from the moment the code loads, and left
 * zero by every call), and 24 MiB for the GEMM route's split-K partial sums (T > 16; its
 * automatic splits are limited to what fits).  Every call on a GPU shares that GPU's array:
 * calls that overlap on one GPU (different streams without synchronization, or several host
 * threads at once) race and give wrong results; calls ordered on one stream are safe.
 *   fmt, M, K, packed_dev, bytes: as for qmat_create (the packed matrix is only read);
 *   x_dev, y_dev, T, stream: as for qmat_run.
 * Errors: as qmat_create and qmat_run, plus QMAT_ESIZE when the launch plan would need more
 * scratch than the array holds, QMAT_EINVAL on a device index of 64 or more. */
int qmat_run_static(int fmt, int64_t M, int64_t K, const void *packed_dev, size_t bytes,
                    const void *x_dev, float *y_dev, int T, void *stream);

/* A launch shape of the product kernel.  The matrix is cut into NT = ceil(M/64) row tiles;
 * a workgroup of `waves` waves works on one tile (or on two neighbouring tiles, see `tiles`)
 * and splits the tile's 128-wide k units among its waves.  The leading NT - tail_tiles tiles
 * are each shared by `splits` workgroups along K, the trailing tail_tiles tiles by
 * `tail_splits` workgroups (a way to spread a few leftover tiles over the whole GPU when NT is
 * not a multiple of the compute-unit count).  Tiles shared by several workgroups are summed
 * over a fixed binary tree of the splits in the handle's workspace, so every plan gives the
 * same y for the same inputs run after run (different plans may differ in the last bits: the
 * summation order differs). */
typedef struct {
    int route;       /* QMAT_ROUTE_VALU, QMAT_ROUTE_MFMA, QMAT_ROUTE_MFMA_OFFSET or QMAT_ROUTE_GEMM
                        (then only splits is
                        read: the k splits of every 64-token x 256-row tile, 1..16) */
    int depth;       /* 128-wide k units each wave keeps in flight: 1 or 2 */
    int waves;       /* waves per workgroup: 1, 2, 4 or 8 */
    int splits;      /* workgroups per leading tile: >= 1 */
    int tail_tiles;  /* trailing tiles using tail_splits: 0 .. ceil(M/64) */
    int tail_splits; /* workgroups per trailing tile: >= 1 (not read when tail_tiles == 0) */
    int tiles;       /* row tiles per wave: 0 or 1 (one), or 2 (a wave streams the same k units
                        of two neighbouring tiles and loads each activation fragment once for
                        both; the MFMA routes with tail_tiles == 0 only) */
} qmat_plan;

/* qmat_run with the automatic plan for (route, T) changed by the nonzero arguments, for tests
 * and tuning.
 *   route:  qmat_route.
 *   depth:  replaces plan.depth (0 = keep).
 *   waves:  replaces plan.waves (0 = keep).
 *   splits: replaces plan.splits and removes the trailing-tile split, so every tile is shared
 *           by `splits` workgroups (0 = keep the automatic plan's splits and tail); on the GEMM
 *           route the k splits, 1..16 (0 = automatic).
 * Errors: as qmat_run, plus QMAT_EINVAL (route, depth, waves) and QMAT_ESIZE (the splits at
 * this T need more workspace than was reserved at create time). */
int qmat_run_ex(qmat_t handle, const void *x_dev, float *y_dev, int T, int route, int depth,
                int waves, int splits, void *stream);

/* qmat_run with an explicit launch shape (all fields read as documented on qmat_plan).
 * Errors: as qmat_run, plus QMAT_EINVAL (null plan, a field outside its range) and QMAT_ESIZE
 * (more splits than the handle's workspace holds at this T, or a grid beyond 2^31-1). */
int qmat_run_plan(qmat_t handle, const void *x_dev, float *y_dev, int T, const qmat_plan *plan,
                  void *stream);

/* The plan qmat_run (route QMAT_ROUTE_AUTO) or qmat_run_ex with only a route would use for T
 * tokens; plan->route is the route taken.  Host only.
 * Errors: QMAT_EINVAL (null argument, bad route), QMAT_ESHAPE (T outside [1, 16] on the
 * small-T routes, outside [1, 4194240] on the GEMM route). */
int qmat_get_plan(qmat_t handle, int T, int route, qmat_plan *plan);

/* Expand the packed matrix to fp32 w [M][K] (device), bit-exact: groupwise fp32(scale) * code
 * ("Qwen3.8-27B for NInfer on the RTX 3090", "What is different from the upstream artifact"),
 * FP8 fl32(r * e4m3) ("Qwen3.8-27B NVFP4 for NInfer", "Artifact").  Asynchronous on stream, no
 * allocation.  w must be 16-byte aligned and hold M * K floats.  For checking; not a fast path.
 * Errors: QMAT_EINVAL (null handle or w, misaligned w, another device current), QMAT_EHIP. */
int qmat_dequant(qmat_t handle, float *w_dev, void *stream);

/* Device workspace of a handle, in bytes.
 *   T >= 1: what qmat_run with T tokens uses of it under the automatic plan: the tree words
 *           that sum a row tile's partial results when K is split across workgroups (small T),
 *           or the GEMM route's split-K partial sums (T > 16); 0 when that plan splits nothing.
 *   T == 0: everything the handle holds (allocated by qmat_create / qmat_create_view for every
 *           T and every launch shape qmat_run_ex / qmat_run_plan accept).
 * Returns 0 for a NULL handle or T outside [0, 4194240].  Host only; no device calls. */
size_t qmat_workspace_bytes(qmat_t handle, int T);

/* Release the handle and its workspace (not the packed matrix).  NULL is ignored. */
void qmat_destroy(qmat_t handle);

/* ---------------------------------------------------------------- output-head epilogue
 *
 * Per token, over fp32 logits y [T][M] (for example what qmat_run wrote for an output head):
 *   lse[t]        = log sum_i exp(y[t][i])                        (the fork's "single-pass
 *                   logsumexp": giveen/ninfer-ext README, upstream pull requests merged ahead)
 *   top_vals[t][] = the k largest y[t][i], largest first; equal values by ascending row i
 *   top_ids[t][]  = their rows i, or index[i] when an index map is given (the indexed 131,072-row
 *                   proposal head whose rows stand for vocabulary ids; the candidate top-k reads
 *                   either it or the full head: "Qwen3.8-27B for NInfer on the RTX 3090", run
 *                   notes).  Slots beyond M hold (-inf, -1).  -0 is returned as +0.
 * Two kernels: one pass over y by row blocks, then one merge per token; the result is
 * deterministic.  y must be finite. */
typedef struct qmat_logits *qmat_logits_t;

/* An epilogue handle for M rows, up to max_T tokens (1..16) and top-k up to max_k (0..64).  It
 * owns a device workspace, allocated here: per token and row block (blocks of 2048 rows, at most
 * 512: beyond 2^20 rows the blocks grow) four (max, sum) states, max_k (value, row) keys and the
 * k-th key, and max_T * M floats of logits for qmat_run_logits called without y.  Nothing in it
 * needs resetting between calls; calls sharing a handle must be ordered.
 * Errors: QMAT_EINVAL (null pointer), QMAT_ESHAPE (M outside [1, 2^30], max_T, max_k),
 * QMAT_ENOMEM, QMAT_EHIP. */
int qmat_logits_create(qmat_logits_t *handle, int64_t M, int max_T, int max_k);

/* Run the epilogue on the stream (asynchronous, no allocation, graph-capturable).
 *   y_dev:        device fp32, row t at y_dev + t * ldy (ldy >= M), 4-byte aligned.
 *   k:            0..max_k; 0 computes only lse.
 *   index_dev:    device int32 [M] row -> id map, or NULL (ids are rows).
 *   lse_dev:      device fp32 [T], or NULL (not computed).
 *   top_vals_dev: device fp32 [T][k]; top_ids_dev: device int32 [T][k] (both required if k > 0).
 * T == 0, or k == 0 with no lse output, is a no-op.
 * Errors: QMAT_EINVAL (null handle / y / outputs, misaligned y), QMAT_ESHAPE (T, k, ldy),
 * QMAT_EHIP (launch). */
int qmat_logits_run(qmat_logits_t handle, const float *y_dev, int64_t ldy, int T, int k,
                    const int32_t *index_dev, float *lse_dev, float *top_vals_dev,
                    int32_t *top_ids_dev, void *stream);

/* The product and the epilogue in one call, on one stream: y = x . W^T exactly as qmat_run
 * computes it, then per token the log-sum-exp and the top k of y exactly as qmat_logits_run
 * computes them.  With y NULL the logits go to the handle's own buffer and are not returned.
 *   handle:  the product matrix; epilogue: created for the same M (max_T, max_k as needed).
 *   x_dev, T, stream: as for qmat_run (T <= the epilogue's max_T);  y_dev: as for qmat_run, or
 *   NULL;  k, index_dev, lse_dev, top_vals_dev, top_ids_dev: as for qmat_logits_run.
 * Asynchronous, no allocation, graph-capturable.  Calls sharing an epilogue handle must be
 * ordered.
 * Errors: QMAT_EINVAL (null handle, x or top-k outputs), QMAT_ESHAPE (M differs, T, k), and
 * those of qmat_run. */
int qmat_run_logits(qmat_t handle, qmat_logits_t epilogue, const void *x_dev, float *y_dev, int T,
                    int k, const int32_t *index_dev, float *lse_dev, float *top_vals_dev,
                    int32_t *top_ids_dev, void *stream);

/* Release the handle and its workspace.  NULL is ignored. */
void qmat_logits_destroy(qmat_logits_t handle);

/* Message describing the calling thread's most recent error ("" if none). */
const char *qmat_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QMAT_H */
