// Device side of the qmat C ABI: handles and their workspaces, launch planning, the product,
// dequant and epilogue calls.  The public contract is in include/qmat.h; the packer and the
// host helpers are in qmat_pack.cpp and qmat_host.cpp (no HIP there).
#include <hip/hip_runtime.h>

#include <mutex>
#include <new>

#include "../../include/qmat.h"
#include "qmat_host.h"
#include "qmat_gemm.h"
#include "qmat_kernels.h"
#include "qmat_layout.h"
#include "qmat_logits.h"

using namespace qmatk;

using qmath::fail;
using qmath::ok;
using qmath::shape_ok;

namespace {

// ------------------------------------------------------------------ planning

struct Plan {
    int route, depth, waves, splits, tail_tiles, tail_splits;
    int tiles = 1;            // row tiles per wave (2: mfma_pair_kernel)
    bool offset_ops = false;  // MFMA route: Q4 up to 8 tokens as offset-binary operands
};

// Launch shape for one (route, tokens-per-launch), from graph-timed sweeps of depth x waves x
// splits x trailing-tile splits over the benchmark shapes on MI355X.
//
// MFMA kernel.
//  - Matrices of at least 2048 row tiles: one tile per workgroup, never split; 4 waves share a
//    tile's k units at T = 1 (a single token leaves registers for two units in flight), 1 wave
//    otherwise.  From a format's crossover a wave streams two neighbouring tiles with one unit
//    in flight, loading each activation fragment once for both.  With at least 3072 tiles:
//    FP8 from T = 2, Q8 and Q5 from 9, Q4 and Q6 from 10 (measured on 248320 x 5120 heads,
//    pair against one tile per wave: FP8 0-3% faster at T = 2-8; Q8 2-3% slower at T = 6-8
//    since tokens up to 8 fill only two accumulator slots per lane; Q5 2% faster at T = 9; Q4
//    and Q6 0.3-9% slower up to T = 9; every format slower at T = 1; above the crossovers
//    1-14% faster, the most at T = 16).  Fewer tiles (the 131072-row proposal head: pairs 1.6%
//    slower at T = 8): the 8-bit formats from T = 9, the others from 10.
//  - At least one tile per compute unit: 4 waves per workgroup, two units in flight up to T = 8
//    and one above.  Up to 8 tokens a lane keeps at most two accumulators per row group; from
//    T = 9 it keeps four, and a two-unit ring then leaves too few resident waves (25-30% slower
//    at T = 12-16).  Gate+up, ring against one unit: 3% faster at T = 4, 4-5% at T = 6-8.  When
//    the tile count is not a multiple of the compute-unit count, the leftover tiles would form a
//    second, nearly empty round of workgroups on a few compute units (measured: 34816 rows take
//    4 us longer than 32768).  Those trailing tiles are instead split along K over up to 8
//    workgroups each at T = 1, up to 4 from T = 2, and dispatched first (34816 rows: 8 splits
//    best at T = 1, 4 splits 1.3% faster at T = 4 and 8, where each piece's tree carries
//    several tokens).  The short trailing workgroups may run beyond one round of resident
//    workgroups, as long as the whole tiles themselves fit in one round.
//  - Fewer tiles than compute units: every tile split along K across workgroups until about 8
//    waves per compute unit exist, at most 3 ways (every split adds a round of partial-sum
//    traffic and a level of the reduction tree at the end of the kernel; 4 and more splits
//    measured slower on every shape).  4 waves per workgroup with two units in flight up to
//    T = 8 (Q5 down at T = 6 / 8: 6% / 3% faster than 8 waves with one unit), 8 waves with one
//    unit beyond (a two-unit ring in 8-wave workgroups would leave room for only one workgroup
//    per compute unit); but when 4 waves would get fewer than 8 units each (short K, e.g.
//    5120), 8 waves with one unit in flight at every T (2-3% faster at T = 1-4, 10% at 8).  A
//    wave's k units are a contiguous slice of the tile's NU units cut into splits x waves slices,
//    and the longest slice sets the tile's time: on very short K the splits go as far as one
//    unit per slice, some slices left empty (5120 x 2176, 17 units: 3 splits x 8 waves 7% faster
//    than 2 x 8, whose one two-unit slice doubles the longest; 4 x 8 slower again).
//
// Vector-ALU kernel (explicit requests only): two units in flight while they fit in registers
// (below), 4 waves per workgroup, single-wave workgroups for wide matrices, splits up to about
// 4 waves per compute unit.
Plan make_plan(int fmt, int route, int Tl, int64_t NT, int64_t NU, int cus)
{
    if (route == kRouteMfma) {
        Plan p{route, 2, 1, 1, 0, 1};
        if (NT >= 2048) {
            p.waves = Tl == 1 ? 4 : 1;
            // two tiles per wave from the token count where sharing the activation fragments
            // outweighs having half as many workgroups (sweeps on 248320 x 5120 heads; a
            // 2048-tile head keeps more workgroups up to T = 8)
            const bool many = NT >= 3072;
            const int pair_from = fmt == kFmtFp8 ? (many ? 2 : 9)
                                  : fmt == kFmtQ8 ? 9
                                  : fmt == 5      ? (many ? 9 : 10)
                                                  : 10;
            if (Tl >= pair_from) {
                p.tiles = 2;
                p.depth = 1;
            }
        } else if (NT >= cus) {
            p.waves = 4;
            p.depth = Tl <= 8 ? 2 : 1;
            while (p.waves > 1 && NU < (int64_t)p.waves) p.waves /= 2;
            const int64_t rem = NT % cus;
            if (rem > 0) {
                const int64_t resident = (int64_t)run_blocks_per_cu(fmt, kRouteMfma, p.depth, Tl, p.waves, 1) * cus;
                int64_t st = cus / rem;
                if (st > (Tl == 1 ? 8 : 4)) st = Tl == 1 ? 8 : 4;
                if (st > NU) st = NU;
                if (NT - rem > resident) st = 1;
                if (st > 1) {
                    p.tail_tiles = (int)rem;
                    p.tail_splits = (int)st;
                }
            }
        } else {
            const bool short_k = NU < 8LL * 4 * 3;  // < 8 units per wave with 4 waves and 3 splits
            p.waves = Tl <= 8 && !short_k ? 4 : 8;
            const int64_t target_waves = 8LL * cus;
            int64_t splits = (target_waves + NT * p.waves - 1) / (NT * p.waves);
            if (splits > 3) splits = 3;
            // a tile's longest slice (k units of one wave) is ceil(NU / (splits * waves)): allow
            // the split that brings it to one unit even when some slices are then empty
            if (splits > (NU + p.waves - 1) / p.waves) splits = (NU + p.waves - 1) / p.waves;
            if (splits < 1) splits = 1;
            p.splits = (int)splits;
            // fewer waves while that keeps every slice at one unit at most
            while (p.waves > 1 && 2 * NU <= (int64_t)p.waves * p.splits) p.waves /= 2;
            if (p.waves == 8) p.depth = 1;
        }
        return p;
    }
    Plan p{route, 2, NT >= 2048 ? 1 : 4, 1, 0, 1};
    // two units in flight only while they fit in registers: from 3 tokens per pass (2 for the
    // 8-bit formats) a second unit spills 32-477 VGPRs and one unit in flight ran 10-40% faster
    // (Q4 gate+up, Q6 and FP8 heads); Q6 at 2 tokens spills 8 and keeps two (4% faster)
    if (Tl >= 3 || (Tl == 2 && (fmt == kFmtFp8 || fmt == kFmtQ8))) p.depth = 1;
    while (p.waves > 1 && NU < 2 * p.waves) p.waves /= 2;
    const int64_t target_waves = 4LL * cus;
    int64_t splits = (target_waves + (NT * p.waves) / 2) / (NT * p.waves);  // rounded
    const int64_t cap = (2 * NU) / (5 * p.waves);                          // >= 2.5 units per wave
    if (splits > cap) splits = cap;
    if (splits < 1) splits = 1;
    p.splits = (int)splits;
    return p;
}

}  // namespace

struct qmat {
    int fmt;
    int64_t M, K, NT, NU, Mpad;
    const uint8_t *codes;   // first code block of the handle's first tile (borrowed)
    const uint8_t *scales;  // its first scale block (borrowed)
    float *ws;          // GEMM route: split-K partial sums (scratch)
    size_t ws_floats;
    uint64_t *nodes;    // small-T routes: tree-node words of shared tiles (all zero between calls)
    size_t node_words;
    int device;
    int cus;
    Plan plan[2][kMaxT + 1];  // [route - 1][tokens per launch]
};

namespace {

// A handle's device memory belongs to the device that was current when it was created; every
// call on it must find that device current again (its kernels launch on the current device).
int device_ok(int device, const char *who)
{
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return fail(QMAT_EHIP, "%s: hipGetDevice failed", who);
    if (cur != device)
        return fail(QMAT_EINVAL, "%s: the handle belongs to device %d but device %d is current", who, device, cur);
    return QMAT_OK;
}

// tokens one launch of a route handles when the call has T tokens
int launch_tokens(int route, int T) { return route == kRouteValu ? (T < kValuMaxT ? T : kValuMaxT) : T; }

// The automatic route is the MFMA kernel for every T.  Both routes unpack each code to bf16
// with the vector ALU; the MFMA kernel then spends one matrix-core instruction per 8 weights
// per lane where the vector-ALU kernel spends four v_dot2c_f32_bf16, and the vector ALU is what
// keeps these kernels from the HBM roofline (measured on MI355X: the MFMA kernel is 2-13%
// faster at T = 1 on the benchmark shapes, and far faster from T = 2).
int auto_route(int fmt, int T)
{
    (void)fmt;
    (void)T;
    return kRouteMfma;
}

}  // namespace

extern "C" {

namespace {

// The GEMM route's share of a handle's workspace is capped (a model holds hundreds of narrow
// matrices); automatic k splits are limited to what fits.
constexpr size_t kGemmSplitWsFloats = (size_t)8 << 20;  // 32 MB

// k splits of the GEMM route: the workgroups (row blocks x token tiles x S) run in waves of
// two per CU, so the time goes as ceil(workgroups / slots) / S in units of one whole-K
// workgroup, plus about 1% of that per split for the partial sums' second pass.  The
// cheapest S with >= 4 units per split, at most kGemmMaxS, whose partials fit ws_cap floats.
int gemm_auto_splits(int64_t NT, int64_t NU, int T, int cus, size_t ws_cap = kGemmSplitWsFloats)
{
    const int64_t slots = 2LL * cus, w0 = (int64_t)gemm_row_blocks((int)NT) * gemm_token_tiles(T);
    int best = 1;
    double best_cost = (double)((w0 + slots - 1) / slots);
    for (int S = 2; S <= kGemmMaxS && NU / S >= 4; ++S) {
        if (gemm_workspace_floats(T, (int)NT, S) > ws_cap) break;
        const double cost = (double)((w0 * S + slots - 1) / slots) / S + 0.01 * S;
        if (cost < best_cost - 1e-9) {
            best = S;
            best_cost = cost;
        }
    }
    return best;
}

// A handle over M x K rows whose packed tiles start at (codes, scales): plans for every route
// and T, and the split-K workspace they need.
int make_handle(qmat_t *handle, int fmt, int64_t M, int64_t K, const uint8_t *codes, const uint8_t *scales,
                const char *who)
{
    qmat *h = new (std::nothrow) qmat;
    if (!h) return fail(QMAT_ENOMEM, "%s: out of host memory", who);
    h->fmt = fmt;
    h->M = M;
    h->K = K;
    h->NT = num_tiles(M);
    h->NU = num_units(K);
    h->Mpad = h->NT * kTileRows;
    h->codes = codes;
    h->scales = scales;
    h->ws = nullptr;
    h->nodes = nullptr;
    h->ws_floats = 0;
    h->node_words = 0;
    if (hipGetDevice(&h->device) != hipSuccess) {
        delete h;
        return fail(QMAT_EHIP, "%s: hipGetDevice failed", who);
    }
    if (hipDeviceGetAttribute(&h->cus, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess || h->cus < 1) {
        delete h;
        return fail(QMAT_EHIP, "%s: cannot read the compute unit count", who);
    }
    // launch plans for both routes and every tokens-per-launch; the tree nodes cover the largest
    // split among them, and at least 8 splits at T = 16 for matrices of up to 16384 rows (explicit
    // launch shapes in tests and tuning)
    size_t need_nodes = 0;
    for (int r = kRouteValu; r <= kRouteMfma; ++r)
        for (int T = 1; T <= kMaxT; ++T) {
            const int Tl = launch_tokens(r, T);
            const Plan p = make_plan(fmt, r, Tl, h->NT, h->NU, h->cus);
            h->plan[r - 1][T] = p;
            const size_t f = run_node_words(Tl, (int)h->NT, p.splits, p.tail_tiles, p.tail_splits);
            if (f > need_nodes) need_nodes = f;
        }
    if (h->Mpad <= 16384 && need_nodes < (size_t)7 * kMaxT * h->Mpad) need_nodes = (size_t)7 * kMaxT * h->Mpad;
    size_t need_ws = 0;
    // the GEMM route's automatic k splits (each within the cap by construction); beyond
    // 2 workgroup waves of row blocks x token tiles no split pays
    for (int ntt = 1; gemm_row_blocks((int)h->NT) * (int64_t)ntt <= 4LL * h->cus; ++ntt) {
        const int T = ntt * kGemmTokens;
        const size_t f = gemm_workspace_floats(T, (int)h->NT, gemm_auto_splits(h->NT, h->NU, T, h->cus));
        if (f > need_ws) need_ws = f;
    }
    if (need_ws > 0) {
        h->ws_floats = need_ws;
        if (hipMalloc(&h->ws, h->ws_floats * sizeof(float)) != hipSuccess) {
            (void)hipGetLastError();
            delete h;
            return fail(QMAT_ENOMEM, "%s: workspace allocation failed", who);
        }
    }
    if (need_nodes > 0) {
        h->node_words = need_nodes;
        if (hipMalloc(&h->nodes, h->node_words * sizeof(uint64_t)) != hipSuccess) {
            (void)hipGetLastError();
            if (h->ws) (void)hipFree(h->ws);
            delete h;
            return fail(QMAT_ENOMEM, "%s: workspace allocation failed", who);
        }
        // the tree nodes start empty; every call leaves them empty again
        if (hipMemset(h->nodes, 0, h->node_words * sizeof(uint64_t)) != hipSuccess ||
            hipDeviceSynchronize() != hipSuccess) {
            (void)hipGetLastError();
            if (h->ws) (void)hipFree(h->ws);
            (void)hipFree(h->nodes);
            delete h;
            return fail(QMAT_EHIP, "%s: workspace initialisation failed", who);
        }
    }
    *handle = h;
    return ok();
}

}  // namespace

int qmat_create(qmat_t *handle, int fmt, int64_t M, int64_t K, const void *packed_dev, size_t bytes)
{
    if (!handle) return fail(QMAT_EINVAL, "qmat_create: null handle pointer");
    *handle = nullptr;
    if (!format_ok(fmt)) return fail(QMAT_EINVAL, "qmat_create: unknown format %d", fmt);
    if (!shape_ok(M, K)) return fail(QMAT_ESHAPE, "qmat_create: bad shape M=%lld K=%lld", (long long)M, (long long)K);
    if (!packed_dev) return fail(QMAT_EINVAL, "qmat_create: null packed pointer");
    if (reinterpret_cast<uintptr_t>(packed_dev) % 16) return fail(QMAT_EINVAL, "qmat_create: packed pointer not 16-byte aligned");
    const size_t need = qmat_packed_bytes(fmt, M, K);
    if (bytes != need) return fail(QMAT_ESIZE, "qmat_create: bytes %zu != packed size %zu", bytes, need);
    const uint8_t *codes = static_cast<const uint8_t *>(packed_dev);
    return make_handle(handle, fmt, M, K, codes, codes + code_bytes(fmt, M, K), "qmat_create");
}

int qmat_create_view(qmat_t *view, qmat_t parent, int64_t row0, int64_t rows)
{
    if (!view) return fail(QMAT_EINVAL, "qmat_create_view: null view pointer");
    *view = nullptr;
    if (!parent) return fail(QMAT_EINVAL, "qmat_create_view: null parent");
    if (const int st = device_ok(parent->device, "qmat_create_view")) return st;
    if (row0 < 0 || rows < 1 || row0 % kTileRows || row0 + rows > parent->M)
        return fail(QMAT_ESHAPE, "qmat_create_view: rows [%lld, %lld) not a 64-aligned range of the parent's %lld rows",
                    (long long)row0, (long long)(row0 + rows), (long long)parent->M);
    const int64_t t0 = row0 / kTileRows;
    const size_t cstep = (size_t)parent->NU * blocks_per_unit(parent->fmt) * kBlockBytes;
    const size_t sstep = parent->fmt == kFmtFp8 ? (size_t)kScaleBlockBytes : (size_t)parent->NU * kScaleBlockBytes;
    return make_handle(view, parent->fmt, rows, parent->K, parent->codes + t0 * cstep, parent->scales + t0 * sstep,
                       "qmat_create_view");
}

namespace {

// The prefill GEMM route (any T >= 1; the automatic choice above the small-T limit) with
// S k splits (0: automatic).
int run_gemm(qmat_t h, const void *x_dev, float *y_dev, int T, int S, void *stream)
{
    if (T < 0 || T > kGemmMaxT) return fail(QMAT_ESHAPE, "qmat_run: T=%d outside [0,%d]", T, kGemmMaxT);
    if (S < 0 || S > kGemmMaxS || S > h->NU)
        return fail(QMAT_EINVAL, "qmat_run: GEMM splits %d outside [0, min(%d, units %lld)]", S, kGemmMaxS,
                    (long long)h->NU);
    if (T == 0) return ok();
    if (!x_dev || !y_dev) return fail(QMAT_EINVAL, "qmat_run: null x or y");
    if (reinterpret_cast<uintptr_t>(x_dev) % 16) return fail(QMAT_EINVAL, "qmat_run: x not 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(y_dev) % 4) return fail(QMAT_EINVAL, "qmat_run: y not 4-byte aligned");
    if (const int st = device_ok(h->device, "qmat_run")) return st;
    if (S == 0) S = gemm_auto_splits(h->NT, h->NU, T, h->cus, h->ws_floats);
    if (S > 1 && gemm_workspace_floats(T, (int)h->NT, S) > h->ws_floats)
        return fail(QMAT_ESIZE, "qmat_run: %d GEMM splits at T=%d exceed the workspace", S, T);
    RunArgs a{};
    a.ws = h->ws;
    a.nodes = nullptr;
    a.codes = h->codes;
    a.scales = h->scales;
    a.x = static_cast<const uint16_t *>(x_dev);
    a.y = y_dev;
    a.ldy = h->M;
    a.M = (int)h->M;
    a.K = (int)h->K;
    a.T = T;
    a.NT = (int)h->NT;
    a.NU = (int)h->NU;
    a.S = S;
    const hipError_t e = launch_gemm(h->fmt, a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(QMAT_EHIP, "qmat_run: launch failed: %s", hipGetErrorString(e));
    return ok();
}

int run_plan(qmat_t h, const void *x_dev, float *y_dev, int T, const Plan &p, void *stream)
{
    if (p.route == kRouteGemm) return run_gemm(h, x_dev, y_dev, T, p.splits, stream);
    if (T < 0 || T > kMaxT) return fail(QMAT_ESHAPE, "qmat_run: T=%d outside [0,%d]", T, kMaxT);
    if (T == 0) return ok();
    if (!x_dev || !y_dev) return fail(QMAT_EINVAL, "qmat_run: null x or y");
    if (reinterpret_cast<uintptr_t>(x_dev) % 16) return fail(QMAT_EINVAL, "qmat_run: x not 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(y_dev) % 4) return fail(QMAT_EINVAL, "qmat_run: y not 4-byte aligned");
    if (p.route != kRouteValu && p.route != kRouteMfma) return fail(QMAT_EINVAL, "qmat_run: bad route");
    if (p.tiles != 1 && p.tiles != 2) return fail(QMAT_EINVAL, "qmat_run: tiles must be 1 or 2");
    if (p.tiles == 2 && (p.route != kRouteMfma || p.tail_tiles != 0))
        return fail(QMAT_EINVAL, "qmat_run: two tiles per wave need the MFMA route and no trailing split");
    if (const int st = device_ok(h->device, "qmat_run")) return st;
    if (!(p.waves == 1 || p.waves == 2 || p.waves == 4 || p.waves == 8))
        return fail(QMAT_EINVAL, "qmat_run: waves must be 1, 2, 4 or 8");
    if (p.depth < 1 || p.depth > kMaxDepth) return fail(QMAT_EINVAL, "qmat_run: depth must be 1..%d", kMaxDepth);
    if (p.splits < 1) return fail(QMAT_EINVAL, "qmat_run: splits must be >= 1");
    if (p.tail_tiles < 0 || p.tail_tiles > h->NT)
        return fail(QMAT_EINVAL, "qmat_run: tail_tiles %d outside [0,%lld]", p.tail_tiles, (long long)h->NT);
    const int tail_splits = p.tail_tiles > 0 ? p.tail_splits : 1;
    if (tail_splits < 1) return fail(QMAT_EINVAL, "qmat_run: tail_splits must be >= 1");
    if ((int64_t)p.splits * p.waves > h->NU * 64 || (int64_t)tail_splits * p.waves > h->NU * 64)
        return fail(QMAT_ESIZE, "qmat_run: too many splits");
    const int64_t grid = (int64_t)p.tail_tiles * tail_splits + (h->NT - p.tail_tiles) * (int64_t)p.splits;
    if (grid > 0x7FFFFFFFLL) return fail(QMAT_ESIZE, "qmat_run: grid of %lld workgroups too large", (long long)grid);
    const int Tl = launch_tokens(p.route, T);
    if (run_node_words(Tl, (int)h->NT, p.splits, p.tail_tiles, tail_splits) > h->node_words)
        return fail(QMAT_ESIZE, "qmat_run: splits %d / tail %d x %d at %d tokens exceed the workspace", p.splits,
                    p.tail_tiles, tail_splits, Tl);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint16_t *x = static_cast<const uint16_t *>(x_dev);
    const uint8_t *codes = h->codes;
    const uint8_t *scales = h->scales;
    for (int t0 = 0; t0 < T; t0 += Tl) {
        RunArgs a{};
        a.codes = codes;
        a.scales = scales;
        a.x = x + (int64_t)t0 * h->K;
        a.y = y_dev + (int64_t)t0 * h->M;
        a.ws = nullptr;
        a.nodes = h->nodes;
        a.ldy = h->M;
        a.M = (int)h->M;
        a.K = (int)h->K;
        a.T = (T - t0 < Tl) ? (T - t0) : Tl;
        a.NT = (int)h->NT;
        a.NU = (int)h->NU;
        a.S = p.splits;
        a.NTt = p.tail_tiles;
        a.St = tail_splits;
        const hipError_t e = launch_run(h->fmt, p.route, p.depth, a, p.waves, p.tiles, p.offset_ops, st);
        if (e != hipSuccess) return fail(QMAT_EHIP, "qmat_run: launch failed: %s", hipGetErrorString(e));
    }
    return ok();
}

}  // namespace

int qmat_run_ex(qmat_t h, const void *x_dev, float *y_dev, int T, int route, int depth, int waves, int splits,
                void *stream)
{
    if (!h) return fail(QMAT_EINVAL, "qmat_run: null handle");
    if (route < QMAT_ROUTE_AUTO || route > QMAT_ROUTE_MFMA_OFFSET)
        return fail(QMAT_EINVAL, "qmat_run: bad route %d", route);
    if (route == QMAT_ROUTE_GEMM || (route == QMAT_ROUTE_AUTO && T > kMaxT))
        return run_gemm(h, x_dev, y_dev, T, splits, stream);
    if (T < 0 || T > kMaxT) return fail(QMAT_ESHAPE, "qmat_run: T=%d outside [0,%d] on this route", T, kMaxT);
    if (T == 0) return ok();
    if (!(waves == 0 || waves == 1 || waves == 2 || waves == 4 || waves == 8))
        return fail(QMAT_EINVAL, "qmat_run: waves must be 0, 1, 2, 4 or 8");
    if (splits < 0) return fail(QMAT_EINVAL, "qmat_run: splits must be >= 0");
    if (depth < 0 || depth > kMaxDepth) return fail(QMAT_EINVAL, "qmat_run: depth must be 0..%d", kMaxDepth);
    const int r = route == QMAT_ROUTE_AUTO ? auto_route(h->fmt, T) : route == QMAT_ROUTE_VALU ? kRouteValu : kRouteMfma;
    Plan p = h->plan[r - 1][T];
    p.offset_ops = route == QMAT_ROUTE_MFMA_OFFSET;
    if (depth) p.depth = depth;
    if (waves) p.waves = waves;
    if (splits) {
        p.splits = splits;
        p.tail_tiles = 0;
        p.tail_splits = 1;
    }
    return run_plan(h, x_dev, y_dev, T, p, stream);
}

int qmat_run_plan(qmat_t h, const void *x_dev, float *y_dev, int T, const qmat_plan *plan, void *stream)
{
    if (!h) return fail(QMAT_EINVAL, "qmat_run_plan: null handle");
    if (!plan) return fail(QMAT_EINVAL, "qmat_run_plan: null plan");
    if (plan->route == QMAT_ROUTE_GEMM) {
        if (plan->splits < 1) return fail(QMAT_EINVAL, "qmat_run_plan: splits must be >= 1");
        return run_gemm(h, x_dev, y_dev, T, plan->splits, stream);
    }
    if (plan->route != QMAT_ROUTE_VALU && plan->route != QMAT_ROUTE_MFMA && plan->route != QMAT_ROUTE_MFMA_OFFSET)
        return fail(QMAT_EINVAL,
                    "qmat_run_plan: route must be QMAT_ROUTE_VALU, QMAT_ROUTE_MFMA, QMAT_ROUTE_MFMA_OFFSET or QMAT_ROUTE_GEMM");
    const Plan p{plan->route == QMAT_ROUTE_VALU ? kRouteValu : kRouteMfma, plan->depth, plan->waves, plan->splits,
                 plan->tail_tiles, plan->tail_splits, plan->tiles == 0 ? 1 : plan->tiles,
                 plan->route == QMAT_ROUTE_MFMA_OFFSET};
    return run_plan(h, x_dev, y_dev, T, p, stream);
}

int qmat_get_plan(qmat_t h, int T, int route, qmat_plan *plan)
{
    if (!h || !plan) return fail(QMAT_EINVAL, "qmat_get_plan: null argument");
    if (route < QMAT_ROUTE_AUTO || route > QMAT_ROUTE_MFMA_OFFSET)
        return fail(QMAT_EINVAL, "qmat_get_plan: bad route %d", route);
    if (route == QMAT_ROUTE_GEMM || (route == QMAT_ROUTE_AUTO && T > kMaxT)) {
        if (T < 1 || T > kGemmMaxT) return fail(QMAT_ESHAPE, "qmat_get_plan: T=%d outside [1,%d]", T, kGemmMaxT);
        *plan = qmat_plan{QMAT_ROUTE_GEMM, 1, 4, gemm_auto_splits(h->NT, h->NU, T, h->cus, h->ws_floats), 0, 1, 1};
        return ok();
    }
    if (T < 1 || T > kMaxT) return fail(QMAT_ESHAPE, "qmat_get_plan: T=%d outside [1,%d]", T, kMaxT);
    const int r = route == QMAT_ROUTE_AUTO ? auto_route(h->fmt, T) : route == QMAT_ROUTE_VALU ? kRouteValu : kRouteMfma;
    const Plan &p = h->plan[r - 1][T];
    plan->route = r == kRouteValu ? QMAT_ROUTE_VALU : route == QMAT_ROUTE_MFMA_OFFSET ? QMAT_ROUTE_MFMA_OFFSET : QMAT_ROUTE_MFMA;
    plan->depth = p.depth;
    plan->waves = p.waves;
    plan->splits = p.splits;
    plan->tail_tiles = p.tail_tiles;
    plan->tail_splits = p.tail_tiles > 0 ? p.tail_splits : 1;
    plan->tiles = p.tiles;
    return ok();
}

int qmat_run(qmat_t h, const void *x_dev, float *y_dev, int T, void *stream)
{
    return qmat_run_ex(h, x_dev, y_dev, T, QMAT_ROUTE_AUTO, 0, 0, 0, stream);
}

int qmat_dequant(qmat_t h, float *w_dev, void *stream)
{
    if (!h) return fail(QMAT_EINVAL, "qmat_dequant: null handle");
    if (!w_dev) return fail(QMAT_EINVAL, "qmat_dequant: null output");
    if (reinterpret_cast<uintptr_t>(w_dev) % 16) return fail(QMAT_EINVAL, "qmat_dequant: output not 16-byte aligned");
    if (const int st = device_ok(h->device, "qmat_dequant")) return st;
    DequantArgs a;
    a.codes = h->codes;
    a.scales = h->scales;
    a.w = w_dev;
    a.M = (int)h->M;
    a.K = (int)h->K;
    a.NT = (int)h->NT;
    a.NU = (int)h->NU;
    const hipError_t e = launch_dequant(h->fmt, a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(QMAT_EHIP, "qmat_dequant: launch failed: %s", hipGetErrorString(e));
    return ok();
}

size_t qmat_workspace_bytes(qmat_t h, int T)
{
    if (!h || T < 0 || T > kGemmMaxT) return 0;
    if (T == 0) return h->ws_floats * sizeof(float) + h->node_words * sizeof(uint64_t);
    if (T > kMaxT) {  // the GEMM route with its automatic k splits
        const int S = gemm_auto_splits(h->NT, h->NU, T, h->cus, h->ws_floats);
        return S > 1 ? gemm_workspace_floats(T, (int)h->NT, S) * sizeof(float) : 0;
    }
    const int r = auto_route(h->fmt, T);
    const Plan &p = h->plan[r - 1][T];
    return run_node_words(launch_tokens(r, T), (int)h->NT, p.splits, p.tail_tiles, p.tail_tiles > 0 ? p.tail_splits : 1) *
           sizeof(uint64_t);
}

}  // extern "C"

// ------------------------------------------------------------------ allocation-free entry point

namespace {

// The scratch of qmat_run_static: one array per GPU (each device holds its own copy, at its own
// address, until the process ends), shared by every such call on that GPU.
//   words [0, kStaticNodeWords): the tree words that sum shared row tiles (small T).  Static
//       storage starts zeroed when the code object is loaded, and every call leaves the words
//       it used zero again.
//   words [kStaticNodeWords, kStaticWords): the GEMM route's split-K partial sums (fp32 scratch).
constexpr size_t kStaticNodeWords = (size_t)1 << 20;   // 8 MiB: every automatic small-T plan on
                                                       // a 256-CU GPU needs at most 512 Ki words
constexpr size_t kStaticGemmFloats = (size_t)6 << 20;  // 24 MiB
constexpr size_t kStaticWords = kStaticNodeWords + kStaticGemmFloats / 2;
static __device__ __align__(256) uint64_t scratch[kStaticWords];

constexpr int kStaticMaxDevices = 64;
std::mutex g_static_mu;
uint64_t *g_static_ptr[kStaticMaxDevices];  // device address of scratch on each device
int g_static_cus[kStaticMaxDevices];

// The device address of the current device's scratch and its compute-unit count, looked up once
// per device.  The array's name is only a host-side stand-in: kernels get this address.
int static_scratch(int dev, uint64_t **ptr, int *cus)
{
    if (dev < 0 || dev >= kStaticMaxDevices)
        return fail(QMAT_EINVAL, "qmat_run_static: device %d beyond the %d devices supported", dev, kStaticMaxDevices);
    std::lock_guard<std::mutex> lock(g_static_mu);
    if (!g_static_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(QMAT_EHIP, "qmat_run_static: cannot locate the scratch array on device %d", dev);
        }
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
            return fail(QMAT_EHIP, "qmat_run_static: cannot read the compute unit count of device %d", dev);
        g_static_cus[dev] = n;
        g_static_ptr[dev] = static_cast<uint64_t *>(p);
    }
    *ptr = g_static_ptr[dev];
    *cus = g_static_cus[dev];
    return QMAT_OK;
}

}  // namespace

extern "C" {

int qmat_run_static(int fmt, int64_t M, int64_t K, const void *packed_dev, size_t bytes, const void *x_dev,
                    float *y_dev, int T, void *stream)
{
    if (!format_ok(fmt)) return fail(QMAT_EINVAL, "qmat_run_static: unknown format %d", fmt);
    if (!shape_ok(M, K))
        return fail(QMAT_ESHAPE, "qmat_run_static: bad shape M=%lld K=%lld", (long long)M, (long long)K);
    if (T < 0 || T > kGemmMaxT) return fail(QMAT_ESHAPE, "qmat_run_static: T=%d outside [0,%d]", T, kGemmMaxT);
    if (!packed_dev) return fail(QMAT_EINVAL, "qmat_run_static: null packed pointer");
    if (reinterpret_cast<uintptr_t>(packed_dev) % 16)
        return fail(QMAT_EINVAL, "qmat_run_static: packed pointer not 16-byte aligned");
    const size_t need = qmat_packed_bytes(fmt, M, K);
    if (bytes != need) return fail(QMAT_ESIZE, "qmat_run_static: bytes %zu != packed size %zu", bytes, need);
    if (T == 0) return ok();
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(QMAT_EHIP, "qmat_run_static: hipGetDevice failed");
    uint64_t *scr = nullptr;
    int cus = 0;
    if (const int st = static_scratch(dev, &scr, &cus)) return st;
    // a handle on the stack over the caller's packed matrix and the scratch: nothing allocated
    qmat h;
    h.fmt = fmt;
    h.M = M;
    h.K = K;
    h.NT = num_tiles(M);
    h.NU = num_units(K);
    h.Mpad = h.NT * kTileRows;
    h.codes = static_cast<const uint8_t *>(packed_dev);
    h.scales = h.codes + code_bytes(fmt, M, K);
    h.nodes = scr;
    h.node_words = kStaticNodeWords;
    h.ws = reinterpret_cast<float *>(scr + kStaticNodeWords);
    h.ws_floats = kStaticGemmFloats;
    h.device = dev;
    h.cus = cus;
    if (T > kMaxT) return run_gemm(&h, x_dev, y_dev, T, 0, stream);
    const int r = auto_route(fmt, T);
    const int Tl = launch_tokens(r, T);
    const Plan p = make_plan(fmt, r, Tl, h.NT, h.NU, cus);
    const size_t words = run_node_words(Tl, (int)h.NT, p.splits, p.tail_tiles, p.tail_tiles > 0 ? p.tail_splits : 1);
    if (words > kStaticNodeWords)
        return fail(QMAT_ESIZE, "qmat_run_static: the plan for M=%lld at T=%d needs %zu scratch words, above the %zu "
                    "the library reserves", (long long)M, T, words, kStaticNodeWords);
    return run_plan(&h, x_dev, y_dev, T, p, stream);
}

void qmat_destroy(qmat_t h)
{
    if (!h) return;
    if (h->ws) (void)hipFree(h->ws);
    if (h->nodes) (void)hipFree(h->nodes);
    delete h;
}


// ------------------------------------------------------------------ head epilogue

}  // extern "C"

struct qmat_logits {
    int64_t M;
    int max_T, max_k;
    int B;                // row blocks per token
    float2 *part_lse;     // [max_T][B][kLogitsWaves] wave states
    uint64_t *part_list;  // [max_T][B][max(max_k, 1)] block lists
    uint64_t *part_kth;   // [max_T][B] blocks' k-th keys
    float *ybuf;          // [max_T][M] logits for qmat_run_logits without y
    int device;
};

extern "C" {

int qmat_logits_create(qmat_logits_t *e, int64_t M, int max_T, int max_k)
{
    if (!e) return fail(QMAT_EINVAL, "qmat_logits_create: null handle pointer");
    *e = nullptr;
    if (M < 1 || M > (1LL << 30)) return fail(QMAT_ESHAPE, "qmat_logits_create: M=%lld outside [1, 2^30]", (long long)M);
    if (max_T < 1 || max_T > kMaxT) return fail(QMAT_ESHAPE, "qmat_logits_create: max_T=%d outside [1,%d]", max_T, kMaxT);
    if (max_k < 0 || max_k > 64) return fail(QMAT_ESHAPE, "qmat_logits_create: max_k=%d outside [0,64]", max_k);
    qmat_logits *h = new (std::nothrow) qmat_logits;
    if (!h) return fail(QMAT_ENOMEM, "qmat_logits_create: out of host memory");
    h->M = M;
    h->max_T = max_T;
    h->max_k = max_k;
    h->part_lse = nullptr;
    h->part_list = nullptr;
    h->part_kth = nullptr;
    h->ybuf = nullptr;
    if (hipGetDevice(&h->device) != hipSuccess) {
        delete h;
        return fail(QMAT_EHIP, "qmat_logits_create: hipGetDevice failed");
    }
    h->B = logits_blocks(M);
    const size_t nt = (size_t)max_T;
    if (hipMalloc(&h->part_lse, nt * h->B * kLogitsWaves * sizeof(float2)) != hipSuccess ||
        hipMalloc(&h->part_list, nt * h->B * (max_k > 0 ? max_k : 1) * sizeof(uint64_t)) != hipSuccess ||
        hipMalloc(&h->part_kth, nt * h->B * sizeof(uint64_t)) != hipSuccess ||
        hipMalloc(&h->ybuf, nt * M * sizeof(float)) != hipSuccess) {
        (void)hipGetLastError();
        for (void *p : {(void *)h->part_lse, (void *)h->part_list, (void *)h->part_kth, (void *)h->ybuf})
            if (p) (void)hipFree(p);
        delete h;
        return fail(QMAT_ENOMEM, "qmat_logits_create: workspace allocation failed");
    }
    *e = h;
    return ok();
}

int qmat_logits_run(qmat_logits_t e, const float *y_dev, int64_t ldy, int T, int k, const int32_t *index_dev,
                    float *lse_dev, float *top_vals_dev, int32_t *top_ids_dev, void *stream)
{
    if (!e) return fail(QMAT_EINVAL, "qmat_logits_run: null handle");
    if (T < 0 || T > e->max_T) return fail(QMAT_ESHAPE, "qmat_logits_run: T=%d outside [0,%d]", T, e->max_T);
    if (k < 0 || k > e->max_k) return fail(QMAT_ESHAPE, "qmat_logits_run: k=%d outside [0,%d]", k, e->max_k);
    if (T == 0 || (k == 0 && !lse_dev)) return ok();
    if (!y_dev) return fail(QMAT_EINVAL, "qmat_logits_run: null y");
    if (reinterpret_cast<uintptr_t>(y_dev) % 4) return fail(QMAT_EINVAL, "qmat_logits_run: y not 4-byte aligned");
    if (ldy < e->M) return fail(QMAT_ESHAPE, "qmat_logits_run: ldy=%lld < M=%lld", (long long)ldy, (long long)e->M);
    if (k > 0 && (!top_vals_dev || !top_ids_dev)) return fail(QMAT_EINVAL, "qmat_logits_run: null top-k output");
    if (const int st = device_ok(e->device, "qmat_logits_run")) return st;
    LogitsArgs a;
    a.y = y_dev;
    a.ldy = ldy;
    a.M = (int)e->M;
    a.T = T;
    a.k = k;
    a.index = index_dev;
    a.lse = lse_dev;
    a.vals = top_vals_dev;
    a.ids = top_ids_dev;
    a.part_lse = e->part_lse;
    a.part_list = e->part_list;
    a.part_kth = e->part_kth;
    a.B = e->B;
    a.rpb = (int)((e->M + a.B - 1) / a.B);
    const hipError_t err = launch_logits(a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(QMAT_EHIP, "qmat_logits_run: launch failed: %s", hipGetErrorString(err));
    return ok();
}

void qmat_logits_destroy(qmat_logits_t e)
{
    if (!e) return;
    for (void *p : {(void *)e->part_lse, (void *)e->part_list, (void *)e->part_kth, (void *)e->ybuf})
        if (p) (void)hipFree(p);
    delete e;
}

int qmat_run_logits(qmat_t h, qmat_logits_t e, const void *x_dev, float *y_dev, int T, int k, const int32_t *index_dev,
                    float *lse_dev, float *top_vals_dev, int32_t *top_ids_dev, void *stream)
{
    if (!h || !e) return fail(QMAT_EINVAL, "qmat_run_logits: null handle");
    if (e->M != h->M)
        return fail(QMAT_ESHAPE, "qmat_run_logits: epilogue handle for M=%lld, matrix has M=%lld", (long long)e->M,
                    (long long)h->M);
    if (T < 0 || T > e->max_T) return fail(QMAT_ESHAPE, "qmat_run_logits: T=%d outside [0,%d]", T, e->max_T);
    if (k < 0 || k > e->max_k) return fail(QMAT_ESHAPE, "qmat_run_logits: k=%d outside [0,%d]", k, e->max_k);
    if (T == 0) return ok();
    if (!x_dev) return fail(QMAT_EINVAL, "qmat_run_logits: null x");
    if (k > 0 && (!top_vals_dev || !top_ids_dev)) return fail(QMAT_EINVAL, "qmat_run_logits: null top-k output");
    if (const int st = device_ok(e->device, "qmat_run_logits")) return st;
    float *y = y_dev ? y_dev : e->ybuf;
    if (const int st = qmat_run(h, x_dev, y, T, stream)) return st;
    if (k == 0 && !lse_dev) return ok();
    return qmat_logits_run(e, y, h->M, T, k, index_dev, lse_dev, top_vals_dev, top_ids_dev, stream);
}

}  // extern "C"
