// gfx950 kernel for the output-head epilogue: per token, the log-sum-exp of the fp32 logits and
// their k largest values with row ids, in one pass over y.
//
// The pages describe both steps next to the head product: the fork merges a "single-pass
// logsumexp" (giveen/ninfer-ext README, upstream pull requests merged ahead of upstream), and
// its speculative drafting takes a candidate top-k that reads either the full head or the
// indexed 131,072-row proposal head ("Qwen3.8-27B for NInfer on the RTX 3090", run notes;
// "Qwen3.8-27B EXL3", the indexed proposal head).  Here the epilogue is format-independent: it
// reads the logits any qmat product wrote, and maps rows through an optional index.
//
// Work split: grid (B, T); block b of token t streams rows [b*rpb, (b+1)*rpb) with 16 waves.
// Each lane keeps an online (max, sum of exp(y - max)); each wave keeps its 64 best (value, row)
// pairs sorted across its lanes (lane i holds the i-th best).  Each lane first orders its four
// rows of a round; the round then enters the list as four 64-pair chunks (every lane's best, then
// every lane's second, ...), each costing one compare against the current k-th best and a wave
// vote, and only when some lane beats it a bitonic sort (DPP / swizzle / half-swap lane
// exchanges) and merge.  Comparisons are branch-free selects.  The block's 16 lists merge in a
// fixed pairwise tree; the block publishes (max, sum, k best) to the workspace, and the last
// block of the token to arrive (arrival counter, reset by that block) merges the B partials
// the same way, with the log-sum-exp states combined in double in a fixed order:
// deterministic output, no memset between calls.
//
// Order: value descending, equal values by ascending row.  Empty slots are (-inf, INT_MAX).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "qmat_logits.h"

namespace qmatk {

namespace {

constexpr int kRowEmpty = 0x7FFFFFFF;

// (v1, r1) ranks before (v2, r2).  Bitwise, not short-circuit, operators: the comparisons
// stay lane masks and selects instead of becoming divergent branches.
__device__ __forceinline__ bool better(float v1, int r1, float v2, int r2)
{
    return (v1 > v2) | ((v1 == v2) & (r1 < r2));
}

// value of lane ^ S, by the cheapest cross-lane route for each distance: DPP within a quad
// (1, 2) or a row of 16 (8), LDS-unit swizzle within 32 lanes (4, 16), and the gfx950 swap of
// the wave's halves (32).  None of these goes through the LDS crossbar's address path.
template <int S> __device__ __forceinline__ int lane_xor(int v)
{
    if constexpr (S == 1) return __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
    else if constexpr (S == 2) return __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
    else if constexpr (S == 4) return __builtin_amdgcn_ds_swizzle(v, 0x101F);                  // xor 4 in 32
    else if constexpr (S == 8) return __builtin_amdgcn_update_dpp(v, v, 0x128, 0xF, 0xF, false); // row_ror 8
    else if constexpr (S == 16) return __builtin_amdgcn_ds_swizzle(v, 0x401F);                 // xor 16 in 32
    else {
        static_assert(S == 32, "lane distance");
        const auto p = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
        return (int)((__lane_id() < 32) ? p[1] : p[0]);
    }
}

template <int S> __device__ __forceinline__ float lane_xor(float v)
{
    return __builtin_bit_cast(float, lane_xor<S>(__builtin_bit_cast(int, v)));
}

// one compare-exchange step between lanes `lane` and `lane ^ S`; keep_better selects which of
// the two this lane keeps
template <int S> __device__ __forceinline__ void cmpx(float &v, int &r, bool keep_better)
{
    const float pv = lane_xor<S>(v);
    const int pr = lane_xor<S>(r);
    // rows are distinct except empty slots, which are identical, so "mine is better" is
    // "partner is not better" (swapping two identical empty slots changes nothing)
    const bool take = keep_better == better(pv, pr, v, r);
    v = take ? pv : v;
    r = take ? pr : r;
}

// bitonic sort of the wave's 64 (v, r) pairs, worst first (lane 63 holds the best: the order
// a sorted list merges against without reversing it)
template <int SIZE, int S> __device__ __forceinline__ void sort_stage(float &v, int &r, int lane)
{
    if constexpr (S > 0) {
        cmpx<S>(v, r, ((lane & S) == 0) != ((lane & SIZE) == 0));
        sort_stage<SIZE, S / 2>(v, r, lane);
    }
}

template <int SIZE = 2> __device__ __forceinline__ void wave_sort(float &v, int &r, int lane)
{
    if constexpr (SIZE <= 64) {
        sort_stage<SIZE, SIZE / 2>(v, r, lane);
        wave_sort<SIZE * 2>(v, r, lane);
    }
}

// bitonic clean of a bitonic 64-sequence into best-first order
template <int S = 32> __device__ __forceinline__ void wave_clean(float &v, int &r, int lane)
{
    if constexpr (S > 0) {
        cmpx<S>(v, r, (lane & S) == 0);
        wave_clean<S / 2>(v, r, lane);
    }
}

// L (sorted, best first) := the 64 best of L and Q, with Q sorted worst first: lane by lane
// the better of the two is the upper half of a bitonic sequence, which one clean sorts.
__device__ __forceinline__ void wave_merge(float &lv, int &lr, float qv, int qr, int lane)
{
    const bool qb = better(qv, qr, lv, lr);
    lv = qb ? qv : lv;
    lr = qb ? qr : lr;
    wave_clean(lv, lr, lane);
}

// Merge the wave's 64 (v, r) pairs, one per lane, into the sorted list.  Only pairs that beat
// the current k-th best can end in the top k: when none does (one compare and a wave vote), the
// chunk costs nothing more; otherwise it is sorted worst first (unless SORTED: then it already
// is) and merged.  (Inserting a few
// candidates one at a time measured slower than the sort: each insertion is a chain of
// vector-to-scalar round trips.)
template <bool SORTED>
__device__ __forceinline__ void wave_take(float &lv, int &lr, float v, int r, int k, int lane)
{
    const float tv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lv), k - 1));
    const int tr = __builtin_amdgcn_readlane(lr, k - 1);
    if (!__ballot(better(v, r, tv, tr))) return;
    if constexpr (!SORTED) wave_sort(v, r, lane);
    wave_merge(lv, lr, v, r, lane);
}

// sort one lane's pairs a, b into best-first order
__device__ __forceinline__ void lane_cswap(float &va, int &ra, float &vb, int &rb)
{
    const bool sw = better(vb, rb, va, ra);
    const float tv = va;
    const int tr = ra;
    va = sw ? vb : va;
    ra = sw ? rb : ra;
    vb = sw ? tv : vb;
    rb = sw ? tr : rb;
}

// The log-sum-exp state (max, sum of exp(v - max)) of the whole wave from the lanes' states:
// the wave max, one exponential per lane to rescale its sum, then a sum over the lanes, all
// through the lane exchanges above.  Every lane ends with the max; lane 0's sum is the one
// used (its order of additions is the same every run).
template <int S> __device__ __forceinline__ double lane_xor(double v)
{
    const int lo = lane_xor<S>(__double2loint(v)), hi = lane_xor<S>(__double2hiint(v));
    return __hiloint2double(hi, lo);
}

template <typename F> __device__ __forceinline__ F wave_max(F v)
{
    v = fmax(v, lane_xor<1>(v));
    v = fmax(v, lane_xor<2>(v));
    v = fmax(v, lane_xor<4>(v));
    v = fmax(v, lane_xor<8>(v));
    v = fmax(v, lane_xor<16>(v));
    return fmax(v, lane_xor<32>(v));
}

template <typename F> __device__ __forceinline__ F wave_sum(F v)
{
    v += lane_xor<1>(v);
    v += lane_xor<2>(v);
    v += lane_xor<4>(v);
    v += lane_xor<8>(v);
    v += lane_xor<16>(v);
    return v + lane_xor<32>(v);
}

template <typename F> __device__ __forceinline__ void wave_lse(F &m, F &s)
{
    const F mx = wave_max(m);
    s = wave_sum(m == -INFINITY ? F(0) : s * exp(m - mx));
    m = mx;
}

__device__ __forceinline__ float ld_agent(const float *p)
{
    return __builtin_bit_cast(float, __hip_atomic_load(reinterpret_cast<const uint32_t *>(p), __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT));
}

__device__ __forceinline__ int ld_agent(const int32_t *p)
{
    return (int)__hip_atomic_load(reinterpret_cast<const uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t publish(float *p, float v)
{
    return __hip_atomic_exchange(reinterpret_cast<uint32_t *>(p), __builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t publish(int32_t *p, int v)
{
    return __hip_atomic_exchange(reinterpret_cast<uint32_t *>(p), (uint32_t)v, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kWaves = 16;        // waves per block
constexpr int kThreads = 64 * kWaves;
constexpr int kStageWords = 8192;  // LDS words staging block partials in the final merge (32 KB)
constexpr int kBurst = 16;         // loads each thread issues before using the first

// (m, s) := combination of two online log-sum-exp states, in double
__device__ __forceinline__ void lse_combine_d(double &m, double &s, double pm, double ps)
{
    if (pm == -INFINITY) return;
    if (m == -INFINITY) {
        m = pm;
        s = ps;
        return;
    }
    const double mx = fmax(m, pm);
    s = s * exp(m - mx) + ps * exp(pm - mx);
    m = mx;
}


// The sorted lists of the block's 16 waves (in s_v / s_r) merge pairwise in a fixed tree
// (wave w takes wave w + step); wave 0 ends with the block's list in (lv, lr).
__device__ __forceinline__ void block_tree_merge(float (*s_v)[64], int (*s_r)[64], float &lv, int &lr, int w,
                                                 int lane)
{
    for (int step = kWaves / 2; step > 0; step >>= 1) {
        __syncthreads();
        if (w < step) {
            wave_merge(lv, lr, s_v[w + step][63 - lane], s_r[w + step][63 - lane], lane);
            s_v[w][lane] = lv;
            s_r[w][lane] = lr;
        }
    }
}

__global__ __launch_bounds__(kThreads) void logits_kernel(LogitsArgs a)
{
    __shared__ float s_v[kWaves][64];
    __shared__ int s_r[kWaves][64];
    __shared__ float s_m[kWaves], s_s[kWaves];
    __shared__ int32_t s_stage[kStageWords];
    __shared__ int s_last;

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int b = blockIdx.x, t = blockIdx.y;
    const int k = a.k, kc = a.k;
    const float *yt = a.y + (int64_t)t * a.ldy;
    const int r0 = b * a.rpb;
    const int r1 = r0 + a.rpb < a.M ? r0 + a.rpb : a.M;

    // ---- stream the block's rows: 4 chunks of 64 rows per wave in flight,
    //      rows r0 + 64 * (kWaves * (4i + j) + w) + lane
    float lv = -INFINITY, m = -INFINITY, s = 0.f;
    int lr = kRowEmpty;
    for (int base = r0; base < r1; base += 4 * kThreads) {
        float v[4];
        int row[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            row[j] = base + kThreads * j + 64 * w + lane;
            v[j] = row[j] < r1 ? yt[row[j]] : -INFINITY;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (row[j] < r1) {
                if (v[j] > m) {
                    s = s * expf(m - v[j]) + 1.f;
                    m = v[j];
                } else {
                    s += expf(v[j] - m);
                }
            } else {
                row[j] = kRowEmpty;
            }
        }
        if (k > 0) {
            // each lane orders its four rows first: chunk j then holds every lane's j-th best, so
            // once the lane maxima are in the list the later chunks rarely have a candidate
            lane_cswap(v[0], row[0], v[1], row[1]);
            lane_cswap(v[2], row[2], v[3], row[3]);
            lane_cswap(v[0], row[0], v[2], row[2]);
            lane_cswap(v[1], row[1], v[3], row[3]);
            lane_cswap(v[1], row[1], v[2], row[2]);
#pragma unroll
            for (int j = 0; j < 4; ++j) wave_take<false>(lv, lr, v[j], row[j], k, lane);
        }
    }
    wave_lse(m, s);
    s_v[w][lane] = lv;
    s_r[w][lane] = lr;
    if (lane == 0) {
        s_m[w] = m;
        s_s[w] = s;
    }
    if (k > 0) block_tree_merge(s_v, s_r, lv, lr, w, lane);
    __syncthreads();

    // ---- block partial (wave 0): publish (max, sum, k best) with returning exchanges
    float *pf = a.part_f + ((int64_t)t * a.B + b) * (2 + kc);
    int32_t *pi = a.part_i + ((int64_t)t * a.B + b) * kc;
    uint32_t sink = 0;
    if (w == 0) {
        // the 16 wave states: lanes 0..15 hold them, lane 0 ends with the block's state
        m = lane < kWaves ? s_m[lane] : -INFINITY;
        s = lane < kWaves ? s_s[lane] : 0.f;
        wave_lse(m, s);
        if (lane < kc) {
            sink |= publish(pf + 2 + lane, lv);
            sink |= publish(pi + lane, lr);
        }
        if (lane == 0) {
            sink |= publish(pf, m);
            sink |= publish(pf + 1, s);
        }
    }
    asm volatile("" ::"v"(sink));
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&a.counter[t], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (uint32_t)(a.B - 1);
    }
    __syncthreads();
    if (!s_last) return;

    // ---- last block of token t: merge the B partials.  They are staged through LDS in chunks
    //      of cb blocks; each thread issues kBurst independent loads before using the first.
    const float *tf = a.part_f + (int64_t)t * a.B * (2 + kc);
    const int32_t *ti = a.part_i + (int64_t)t * a.B * kc;
    const int stride_f = 2 + kc, per = 2 + 2 * kc;
    const int cb = kStageWords / per < a.B ? kStageWords / per : a.B;
    float *st_f = reinterpret_cast<float *>(s_stage);
    int32_t *st_i = s_stage + cb * stride_f;
    double tm = -INFINITY, ts = 0.0;  // wave 0 lane l: blocks l, l + 64, ... in order
    lv = -INFINITY;
    lr = kRowEmpty;
    for (int c0 = 0; c0 < a.B; c0 += cb) {
        const int n = a.B - c0 < cb ? a.B - c0 : cb;
        const int nf = n * stride_f, ni = n * kc;
        __syncthreads();  // the previous chunk's readers are done
        for (int e0 = threadIdx.x; e0 < nf; e0 += kBurst * kThreads) {
            float v[kBurst];
#pragma unroll
            for (int i = 0; i < kBurst; ++i) {
                const int e = e0 + kThreads * i;
                v[i] = e < nf ? ld_agent(tf + (int64_t)c0 * stride_f + e) : 0.f;
            }
#pragma unroll
            for (int i = 0; i < kBurst; ++i)
                if (e0 + kThreads * i < nf) st_f[e0 + kThreads * i] = v[i];
        }
        for (int e0 = threadIdx.x; e0 < ni; e0 += kBurst * kThreads) {
            int v[kBurst];
#pragma unroll
            for (int i = 0; i < kBurst; ++i) {
                const int e = e0 + kThreads * i;
                v[i] = e < ni ? ld_agent(ti + (int64_t)c0 * kc + e) : 0;
            }
#pragma unroll
            for (int i = 0; i < kBurst; ++i)
                if (e0 + kThreads * i < ni) st_i[e0 + kThreads * i] = v[i];
        }
        __syncthreads();
        if (w == 0)
            for (int e = lane; e < n; e += 64)
                lse_combine_d(tm, ts, (double)st_f[e * stride_f], (double)st_f[e * stride_f + 1]);
        // top-k: wave w takes the block lists w, w + 16, ... of the chunk (lane i reads entry i)
        if (k > 0)
            for (int e = w; e < n; e += kWaves) {
                // the block's list, read worst first (empty slots, then entry kc - 1 ... 0)
                const int q = 63 - lane;
                const float cv = q < kc ? st_f[e * stride_f + 2 + q] : -INFINITY;
                const int cr = q < kc ? st_i[e * kc + q] : kRowEmpty;
                wave_take<true>(lv, lr, cv, cr, k, lane);
            }
    }
    if (k > 0) {
        __syncthreads();  // the stage is free; s_v / s_r take the wave lists
        s_v[w][lane] = lv;
        s_r[w][lane] = lr;
        block_tree_merge(s_v, s_r, lv, lr, w, lane);
    }
    if (w == 0) {
        if (lane < kc) {
            a.vals[(int64_t)t * kc + lane] = lv;
            a.ids[(int64_t)t * kc + lane] = lr == kRowEmpty ? -1 : (a.index ? a.index[lr] : lr);
        }
        // the 64 lane states (in double), lane 0 ends with the token's
        wave_lse(tm, ts);
        if (lane == 0 && a.lse) a.lse[t] = (float)(tm + log(ts));
        if (lane == 0) __hip_atomic_store(&a.counter[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace

int logits_blocks_per_cu()
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(&logits_kernel), kThreads, 0) !=
        hipSuccess)
        return 0;
    return n;
}

hipError_t launch_logits(const LogitsArgs &a, hipStream_t st)
{
    LogitsArgs arg = a;
    void *args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void *>(&logits_kernel), dim3((unsigned)a.B, (unsigned)a.T),
                           dim3(kThreads), args, 0, st);
}

}  // namespace qmatk
