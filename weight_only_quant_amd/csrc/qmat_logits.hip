// gfx950 kernels for the output-head epilogue: per token, the log-sum-exp of the fp32 logits and
// their k largest values with row ids.
//
// The pages describe both steps next to the head product: the fork merges a "single-pass
// logsumexp" (giveen/ninfer-ext README, upstream pull requests merged ahead of upstream), and
// its speculative drafting takes a candidate top-k that reads either the full head or the
// indexed 131,072-row proposal head ("Qwen3.8-27B for NInfer on the RTX 3090", run notes;
// "Qwen3.8-27B EXL3", the indexed proposal head).  Here the epilogue is format-independent: it
// reads the logits any qmat product wrote, and maps rows through an optional index.
//
// Order: a (value, row) pair is one 64-bit key, the value's bits made unsigned-monotone above
// the row's complement, so "better" (larger value, equal values by smaller row) is one unsigned
// compare and every step of a sort is one compare and two selects.  -0 ranks as +0 (it is
// returned as +0); key 0 is an empty slot and ranks below every pair, -inf included.
//
// Kernel 1, grid (B, T), 4 waves: block b of token t streams rows [b*rpb, (b+1)*rpb) in rounds
// of 8 rows per lane, the next round's loads in flight while one round is processed.  Each lane
// keeps an online (max, sum of exp(y - max)), the sum across rounds in double.  For the top k
// the block keeps its k best keys in LDS and theta, the k-th of them: a key below theta cannot
// reach the top k.  The first round seeds theta: per wave the largest value that k of its lane
// maxima reach (for k > 32, k of all its keys), found by a binary search over the value's bits
// with one vote per bit and key; the largest over the waves (k distinct rows reach it).  Each
// round the list and the keys at or above theta
// (usually a few dozen) go to LDS, and each candidate's rank among them, counted from LDS
// broadcast reads, is its place in the new list: independent compares instead of the dependent
// steps of a sort.  Rounds with more than 256 candidates (adversarial orders) take them with
// wave sorting networks and a merge of the waves' lists.  Each wave writes its (max, sum); the
// block writes its k best keys and its k-th key.
//
// Kernel 2, one block per token, after kernel 1 (the kernel boundary makes its stores visible):
// tau is the larger of two keys that k distinct rows reach, the largest k-th key of a block and
// a key that k of the blocks' best keys reach (their k-th best, or for k <= 32 the largest over
// the waves of the value k of a wave's best keys reach), so every key of the token's top k is at
// or above it.
// Every block's list is loaded in one round of loads; the keys at or above tau (usually about
// k) are ranked the same way.  The waves' states combine in double in a fixed order.  The
// candidate set is exact and the order total, so the output is deterministic: no atomics on
// global memory, nothing to reset between calls.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "qmat_logits.h"

namespace qmatk {

namespace {

// ---------------------------------------------------------------------------- keys

__device__ __forceinline__ uint64_t make_key(float v, int row)
{
    uint32_t u = __builtin_bit_cast(uint32_t, v);
    u = u == 0x80000000u ? 0u : u;
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)o << 32) | (uint32_t)~(uint32_t)row;
}

__device__ __forceinline__ float key_value(uint64_t key)
{
    const uint32_t o = (uint32_t)(key >> 32);
    return __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ int key_row(uint64_t key) { return (int)~(uint32_t)key; }

// ---------------------------------------------------------------------------- lane exchanges

// value of lane ^ S: DPP within a quad (1, 2) or a row of 16 (8), the LDS unit's swizzle within
// 32 lanes (4, 16: no VALU issue slot), and the gfx950 swap of the wave's halves (32)
template <int S> __device__ __forceinline__ int lane_xor(int v)
{
    if constexpr (S == 1) return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);   // quad_perm 1,0,3,2
    else if constexpr (S == 2) return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);  // quad_perm 2,3,0,1
    else if constexpr (S == 4) return __builtin_amdgcn_ds_swizzle(v, 0x101F);             // xor 4 in 32
    else if constexpr (S == 8) return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true); // row_ror 8
    else if constexpr (S == 16) return __builtin_amdgcn_ds_swizzle(v, 0x401F);            // xor 16 in 32
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

template <int S> __device__ __forceinline__ uint64_t lane_xor(uint64_t v)
{
    const uint32_t lo = (uint32_t)lane_xor<S>((int)(uint32_t)v), hi = (uint32_t)lane_xor<S>((int)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

template <int S> __device__ __forceinline__ double lane_xor(double v)
{
    const int lo = lane_xor<S>(__double2loint(v)), hi = lane_xor<S>(__double2hiint(v));
    return __hiloint2double(hi, lo);
}

__device__ __forceinline__ uint64_t readlane(uint64_t v, int l)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// ---------------------------------------------------------------------------- wave sort / merge

// one compare-exchange between lanes `lane` and `lane ^ S`; keep_better says which one this lane
// keeps (keys are distinct except empty slots, which are equal, so either choice is right then)
template <int S> __device__ __forceinline__ void cmpx(uint64_t &key, bool keep_better)
{
    const uint64_t p = lane_xor<S>(key);
    key = keep_better == (p > key) ? p : key;
}

template <int SIZE, int S> __device__ __forceinline__ void sort_stage(uint64_t &key, int lane)
{
    if constexpr (S > 0) {
        cmpx<S>(key, ((lane & S) == 0) != ((lane & SIZE) == 0));
        sort_stage<SIZE, S / 2>(key, lane);
    }
}

// bitonic sort of the wave's 64 keys, worst first (lane 63 holds the best: the order a sorted
// list merges against without reversing it)
template <int SIZE = 2, int LAST = 64> __device__ __forceinline__ void wave_sort(uint64_t &key, int lane)
{
    if constexpr (SIZE <= LAST) {
        sort_stage<SIZE, SIZE / 2>(key, lane);
        wave_sort<SIZE * 2, LAST>(key, lane);
    }
}

// bitonic clean of a bitonic 64-sequence into best-first order
template <int S = 32> __device__ __forceinline__ void wave_clean(uint64_t &key, int lane)
{
    if constexpr (S > 0) {
        cmpx<S>(key, (lane & S) == 0);
        wave_clean<S / 2>(key, lane);
    }
}

// L (sorted, best first) := the 64 best of L and Q, with Q sorted worst first: lane by lane the
// better of the two is the upper half of a bitonic sequence, which one clean sorts
__device__ __forceinline__ void wave_merge(uint64_t &list, uint64_t q, int lane)
{
    list = q > list ? q : list;
    wave_clean(list, lane);
}

// Take the wave's 64 keys (one per lane, 0 = none) into the sorted list, keeping its k best:
// when no key beats the list's k-th (one compare and a wave vote) nothing more is done,
// otherwise the keys are sorted and merged.
__device__ __forceinline__ void wave_take(uint64_t &list, uint64_t key, int k, int lane)
{
    if (!__ballot(key > readlane(list, k - 1))) return;
    wave_sort(key, lane);
    wave_merge(list, key, lane);
}

// ---------------------------------------------------------------------------- exp

// e^x for x <= 0 (or -inf): 2^(x log2 e) with x log2 e carried in two parts, the hardware 2^h of
// the rounded part times the first-order term of the rest, within a few ulp.  x is clamped at
// -200 (e^-200 and below flush to zero, which no sum of terms up to 1 can tell apart; -inf
// would make the residual NaN).
__device__ __forceinline__ float exp_nonpos(float x)
{
    constexpr float kL = 1.44269502f;         // log2 e rounded to float
    constexpr float kLlo = 1.92596299e-8f;    // log2 e - kL
    constexpr float kLn2 = 0.693147182f;
    x = fmaxf(x, -200.f);
    const float h = x * kL;
    const float l = fmaf(x, kL, -h) + x * kLlo;
    const float e = __builtin_amdgcn_exp2f(h);
    return fmaf(e, l * kLn2, e);
}

// ---------------------------------------------------------------------------- reductions

template <int S, typename F> __device__ __forceinline__ F max_step(F v)
{
    const F o = lane_xor<S>(v);
    return o > v ? o : v;
}

template <typename F> __device__ __forceinline__ F wave_max(F v)
{
    v = max_step<1>(v);
    v = max_step<2>(v);
    v = max_step<4>(v);
    v = max_step<8>(v);
    v = max_step<16>(v);
    return max_step<32>(v);
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

// The log-sum-exp state (max, sum of exp(v - max)) of the whole wave from the lanes' states: the
// wave max, one exponential per lane to rescale its sum, then a sum over the lanes, in a fixed
// order.  Every lane ends with the wave's state.
__device__ __forceinline__ void wave_lse(float &m, float &s)
{
    const float mx = wave_max(m);
    s = wave_sum(m == -INFINITY ? 0.f : s * exp_nonpos(m - mx));
    m = mx;
}

// ---------------------------------------------------------------------------- rank selection

// The number of keys in s[0..n) above `key`: LDS broadcast reads of two keys each, eight in
// flight, counted into four independent sums (the compares do not wait on each other, unlike
// the steps of a sort, and the sums do not form one long chain).
__device__ __forceinline__ int rank_in(const uint64_t *s, int n, uint64_t key)
{
    const ulonglong2 *p = reinterpret_cast<const ulonglong2 *>(s);
    const int np = n >> 1;
    int r0 = 0, r1 = 0, r2 = 0, r3 = 0, i = 0;
#pragma unroll 2
    for (; i + 4 <= np; i += 4) {
        const ulonglong2 q0 = p[i], q1 = p[i + 1], q2 = p[i + 2], q3 = p[i + 3];
        r0 += (int)(q0.x > key) + (int)(q0.y > key);
        r1 += (int)(q1.x > key) + (int)(q1.y > key);
        r2 += (int)(q2.x > key) + (int)(q2.y > key);
        r3 += (int)(q3.x > key) + (int)(q3.y > key);
    }
    for (; i < np; ++i) {
        const ulonglong2 q = p[i];
        r0 += (int)(q.x > key) + (int)(q.y > key);
    }
    if (n & 1) r0 += (int)(s[n - 1] > key);
    return (r0 + r1) + (r2 + r3);
}

// Each thread appends its keys at or above th (and non-zero) to s_cand at offset `at0` +
// its place from one atomic on s_count: one LDS atomic per thread that has any.
template <int N>
__device__ __forceinline__ void append_at_or_above(const uint64_t (&key)[N], uint64_t th, uint64_t *s_cand, int cap,
                                                   int *s_count, int at0)
{
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) cnt += (int)(key[j] != 0 && key[j] >= th);
    if (cnt == 0) return;
    int at = at0 + atomicAdd(s_count, cnt);
#pragma unroll
    for (int j = 0; j < N; ++j) {
        if (key[j] != 0 && key[j] >= th) {
            if (at < cap) s_cand[at] = key[j];
            ++at;
        }
    }
}

// ---------------------------------------------------------------------------- kernel 1

constexpr int kWaves = kLogitsWaves;         // waves per block
constexpr int kThreads = 64 * kWaves;
constexpr int kPerLane = 8;                  // rows per lane per round
constexpr int kRound = kPerLane * kThreads;  // rows per round
constexpr int kCand = kThreads;              // candidates ranked at once: one per thread

// The sorted lists of the block's waves (in s_list and in registers, best first) merge pairwise
// in a fixed tree (wave w takes wave w + step, read worst first); wave 0 ends with the block's.
template <int NW>
__device__ __forceinline__ void block_tree_merge(uint64_t (*s_list)[64], uint64_t &list, int w, int lane)
{
    for (int step = NW / 2; step > 0; step >>= 1) {
        __syncthreads();
        if (w < step) {
            wave_merge(list, s_list[w + step][63 - lane], lane);
            s_list[w][lane] = list;
        }
    }
}

// BIG_K (k > 32): the seed counts all of a wave's keys (below)
template <bool BIG_K>
__global__ __launch_bounds__(kThreads) void logits_kernel(LogitsArgs a)
{
    __shared__ __align__(16) uint64_t s_cand[kCand];
    __shared__ uint64_t s_top[64];
    __shared__ __align__(16) uint64_t s_lm[kWaves][64];
    __shared__ uint64_t s_thw[kWaves];
    __shared__ int s_count[3];  // round r counts in s_count[r % 3]
    __shared__ int s_ntop;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int b = blockIdx.x, t = blockIdx.y;
    const int k = a.k;
    const float *yt = a.y + (int64_t)t * a.ldy;
    const int r0 = b * a.rpb;
    const int r1 = r0 + a.rpb < a.M ? r0 + a.rpb : a.M;
    if (threadIdx.x == 0) s_count[0] = 0;

    float m = -INFINITY;  // the lane's running max
    double s = 0.0;       // sum of exp(y - m) over the lane's rows: in double, so that blocks of
                          // many rounds (large M) add no fp32 rounding per round
    int ntop = 0;        // entries in s_top, the block's best keys so far (best first)
    uint64_t theta = 0;  // the k-th of them (0 while there are fewer)
    int rr = 0;  // round index mod 3
    float nv[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        const int row = r0 + kThreads * j + threadIdx.x;
        nv[j] = row < r1 ? yt[row] : -INFINITY;
    }
    for (int base = r0; base < r1; base += kRound) {
        float v[kPerLane];
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) v[j] = nv[j];
        if (base + kRound < r1) {
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) {
                const int row = base + kRound + kThreads * j + threadIdx.x;
                nv[j] = row < r1 ? yt[row] : -INFINITY;
            }
        }
        // online log-sum-exp: rows past the end load as -inf and add exp(-inf) = 0
        float mr = v[0];
#pragma unroll
        for (int j = 1; j < kPerLane; ++j) mr = fmaxf(mr, v[j]);
        if (mr > -INFINITY) {
            const float mn = fmaxf(m, mr);
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) acc += exp_nonpos(v[j] - mn);
            s = (m == -INFINITY ? 0.0 : s * (double)exp_nonpos(m - mn)) + (double)acc;
            m = mn;
        }
        if (k == 0) continue;
        uint64_t key[kPerLane];
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int row = base + kThreads * j + threadIdx.x;
            key[j] = row < r1 ? make_key(v[j], row) : 0ull;
        }
        if (base == r0) {
            // theta := over the waves, the largest value part that at least k lane maxima of the
            // wave reach (a binary search over its 32 bits, one compare and vote per bit), as
            // the smallest key with that value part: k distinct rows reach it
            uint64_t mx = key[0];
#pragma unroll
            for (int j = 1; j < kPerLane; ++j) mx = key[j] > mx ? key[j] : mx;
            const uint32_t mv = (uint32_t)(mx >> 32);  // 0 for an empty lane
            uint32_t tv = 0;
            if constexpr (!BIG_K) {
#pragma unroll
                for (int bit = 31; bit >= 0; --bit) {
                    const uint32_t c = tv | (1u << bit);
                    if (__popcll(__ballot(mv >= c)) >= k) tv = c;
                }
            } else {
                // for large k the lane maxima alone give a loose bound (at k = 64 their
                // smallest): count all of the wave's keys instead
                uint32_t kv[kPerLane];
#pragma unroll
                for (int j = 0; j < kPerLane; ++j) kv[j] = (uint32_t)(key[j] >> 32);
#pragma unroll
                for (int bit = 31; bit >= 0; --bit) {
                    const uint32_t c = tv | (1u << bit);
                    int n = 0;
#pragma unroll
                    for (int j = 0; j < kPerLane; ++j) n += __popcll(__ballot(kv[j] >= c));
                    if (n >= k) tv = c;
                }
            }
            if (lane == 0) s_thw[w] = (uint64_t)tv << 32;
            __syncthreads();
            theta = s_thw[0];
#pragma unroll
            for (int i = 1; i < kWaves; ++i) theta = s_thw[i] > theta ? s_thw[i] : theta;
        }
        // candidates: the list so far, then this round's keys at or above theta.  The next
        // round's counter is cleared before this round's barrier: its last readers (two rounds
        // ago) are past the previous barrier, and the next round counts after this one.
        const int rn = rr == 2 ? 0 : rr + 1;
        if (threadIdx.x == 0) s_count[rn] = 0;
        if ((int)threadIdx.x < ntop) s_cand[threadIdx.x] = s_top[threadIdx.x];
        append_at_or_above(key, theta, s_cand, kCand, &s_count[rr], ntop);
        __syncthreads();
        const int C = ntop + s_count[rr];
        rr = rn;
        if (C == ntop) continue;  // nothing new; s_cand and s_top were only read
        if (C <= kCand) {
            if ((int)threadIdx.x < C) {
                const uint64_t c = s_cand[threadIdx.x];
                const int r = rank_in(s_cand, C, c);
                if (r < k) s_top[r] = c;
            }
            ntop = C < k ? C : k;
        } else {
            // rare: every wave takes its keys at or above theta (wave 0 the list too) by sorts,
            // and the waves' lists merge
            uint64_t wl = 0;
            if (w == 0) wave_take(wl, lane < ntop ? s_top[lane] : 0ull, k, lane);
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) wave_take(wl, key[j] >= theta ? key[j] : 0ull, k, lane);
            __syncthreads();  // every reader of s_top is done
            s_lm[w][lane] = wl;
            block_tree_merge<kWaves>(s_lm, wl, w, lane);
            if (w == 0) {
                if (lane < k) s_top[lane] = wl;
                const int nz = __popcll(__ballot(lane < k && wl != 0));
                if (lane == 0) s_ntop = nz;
            }
            __syncthreads();
            ntop = s_ntop;
        }
        __syncthreads();
        theta = ntop == k ? s_top[k - 1] : 0ull;
    }

    // block partial: each wave's (max, sum), the k best keys and the k-th (s_top was last
    // written before a barrier)
    float sf = (float)s;
    wave_lse(m, sf);
    const int64_t tb = (int64_t)t * a.B + b;
    if (lane == 0) a.part_lse[tb * kWaves + w] = make_float2(m, sf);
    if (w == 0 && k > 0) {
        if (lane < k) a.part_list[tb * k + lane] = lane < ntop ? s_top[lane] : 0ull;
        if (lane == 0) a.part_kth[tb] = ntop == k ? s_top[k - 1] : 0ull;
    }
}

// ---------------------------------------------------------------------------- kernel 2

constexpr int kMWaves = 4;
constexpr int kMThreads = 64 * kMWaves;
constexpr int kMPer = 16;                               // list entries per thread per round of loads
constexpr int kMPerBlock = kMaxBlocks / kMThreads;      // blocks (heads, k-th keys) per thread at most
constexpr int kMPerState = kMPerBlock * kWaves;         // wave states per thread at most
constexpr int kMCand = 1024;                            // candidates ranked at once

__global__ __launch_bounds__(kMThreads) void logits_merge_kernel(MergeArgs a)
{
    __shared__ __align__(16) uint64_t s_cand[kMCand];
    __shared__ __align__(16) uint64_t s_h[kMaxBlocks];   // the lists' best keys
    __shared__ __align__(16) uint64_t s_hc[kMaxBlocks];  // those among the k best of their group of 64
    __shared__ uint64_t s_list[kMWaves][64];
    __shared__ float s_mx[kMWaves];
    __shared__ double s_sum[kMWaves];
    __shared__ uint64_t s_kth[kMWaves];
    __shared__ uint64_t s_th;
    __shared__ uint64_t s_hw[kMWaves];
    __shared__ int s_count, s_hcount;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int t = blockIdx.x;
    const int k = a.k, G = a.G;
    const int n = G * k;
    const int i0 = threadIdx.x;
    if (i0 == 0) {
        s_count = 0;
        s_hcount = 0;
        s_th = 0;
    }

    // every load at once: the block states, k-th keys and best keys (thread i0 takes blocks
    // i0, i0 + 256), and the first kMPer entries of the lists per thread
    float2 p[kMPerState];
    uint64_t kth = 0, head[kMPerBlock];
    const uint64_t *lists = a.list + (int64_t)t * n;
    const int ns = G * kWaves;
#pragma unroll
    for (int q = 0; q < kMPerState; ++q) {
        const int i = i0 + kMThreads * q;
        p[q] = i < ns ? a.lse_part[(int64_t)t * ns + i] : make_float2(-INFINITY, 0.f);
    }
#pragma unroll
    for (int q = 0; q < kMPerBlock; ++q) {
        const int i = i0 + kMThreads * q;
        const uint64_t kq = k > 0 && i < G ? a.kth[(int64_t)t * G + i] : 0ull;
        kth = kq > kth ? kq : kth;
        head[q] = k > 0 && i < G ? lists[(int64_t)i * k] : 0ull;
    }
    uint64_t e[kMPer];
#pragma unroll
    for (int j = 0; j < kMPer; ++j) {
        const int idx = i0 + kMThreads * j;
        e[j] = idx < n ? lists[idx] : 0ull;
    }

    // log-sum-exp: the largest block max, then the blocks' sums rescaled to it (fp32 exponent of
    // a difference, summed in double in a fixed order)
    float mt = p[0].x;
#pragma unroll
    for (int q = 1; q < kMPerState; ++q) mt = fmaxf(mt, p[q].x);
    mt = wave_max(mt);
    kth = wave_max(kth);
    if (lane == 0) {
        s_mx[w] = mt;
        s_kth[w] = kth;
    }
#pragma unroll
    for (int q = 0; q < kMPerBlock; ++q)
        if (i0 + kMThreads * q < G) s_h[i0 + kMThreads * q] = head[q];
    __syncthreads();
    float mstar = s_mx[0];
    uint64_t tau = s_kth[0];
#pragma unroll
    for (int i = 1; i < kMWaves; ++i) {
        mstar = fmaxf(mstar, s_mx[i]);
        tau = s_kth[i] > tau ? s_kth[i] : tau;
    }
    double term = 0.0;
#pragma unroll
    for (int q = 0; q < kMPerState; ++q)
        term += p[q].x == -INFINITY ? 0.0 : (double)p[q].y * (double)expf(p[q].x - mstar);
    const double sw = wave_sum(term);
    if (lane == 0) s_sum[w] = sw;

    if (k > 0) {
        // tau: the larger of two keys that k distinct rows reach, the largest k-th entry of a
        // list and a key that k of the lists' best keys reach (tight when the lists are many):
        // up to 256 lists and k <= 32 a search per wave; up to 256 lists otherwise each best
        // key is ranked among all of them; beyond, among its group of 64 first, and the group
        // winners among each other
        if (G <= kMThreads && k <= 32) {
            // per wave, the largest value part that k of its lists' best keys reach (a binary
            // search over the 32 bits, one compare and vote per bit); the largest over the waves.
            // With up to 64 lists per wave this stays tight for k up to about half of them (at
            // k = 64 a wave's bound would be its smallest best key).
            const uint32_t hv = (uint32_t)(head[0] >> 32);  // 0: no list here, or an empty one
            uint32_t tv = 0;
#pragma unroll
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t c = tv | (1u << bit);
                if (__popcll(__ballot(hv >= c)) >= k) tv = c;
            }
            if (lane == 0) s_hw[w] = (uint64_t)tv << 32;
            __syncthreads();
            if (i0 == 0) {
                uint64_t th = s_hw[0];
#pragma unroll
                for (int i = 1; i < kMWaves; ++i) th = s_hw[i] > th ? s_hw[i] : th;
                s_th = th;
            }
        } else if (G <= kMThreads) {
            if (i0 < G && head[0] != 0 && rank_in(s_h, G, head[0]) == k - 1) s_th = head[0];
        } else {
#pragma unroll
            for (int q = 0; q < kMPerBlock; ++q) {
                const int i = i0 + kMThreads * q;
                if (i < G && head[q] != 0) {
                    const int g0 = i & ~63, gn = G - g0 < 64 ? G - g0 : 64;
                    if (rank_in(s_h + g0, gn, head[q]) < k) s_hc[atomicAdd(&s_hcount, 1)] = head[q];
                }
            }
            __syncthreads();
            const int Ch = s_hcount;
            for (int c = i0; c < Ch; c += kMThreads)
                if (rank_in(s_hc, Ch, s_hc[c]) == k - 1) s_th = s_hc[c];
        }
        __syncthreads();
        tau = s_th > tau ? s_th : tau;
        // candidates: the entries at or above tau
        append_at_or_above(e, tau, s_cand, kMCand, &s_count, 0);
        for (int c0 = kMThreads * kMPer; c0 < n; c0 += kMThreads * kMPer) {
#pragma unroll
            for (int j = 0; j < kMPer; ++j) {
                const int idx = c0 + i0 + kMThreads * j;
                e[j] = idx < n ? lists[idx] : 0ull;
            }
            append_at_or_above(e, tau, s_cand, kMCand, &s_count, 0);
        }
        __syncthreads();
        const int C = s_count;
        float *vals = a.vals + (int64_t)t * k;
        int32_t *ids = a.ids + (int64_t)t * k;
        if (C <= kMCand) {
            for (int c = i0; c < C; c += kMThreads) {
                const uint64_t key = s_cand[c];
                const int r = rank_in(s_cand, C, key);
                if (r < k) {
                    vals[r] = key_value(key);
                    ids[r] = a.index ? a.index[key_row(key)] : key_row(key);
                }
            }
            if (i0 >= C && i0 < k) {
                vals[i0] = -INFINITY;
                ids[i0] = -1;
            }
        } else {
            // rare: every wave takes its threads' candidates by sorts, read again
            uint64_t list = 0;
#pragma unroll 1
            for (int idx = i0; idx - lane < n; idx += kMThreads) {
                const uint64_t c = idx < n ? lists[idx] : 0ull;
                wave_take(list, c >= tau ? c : 0ull, k, lane);
            }
            s_list[w][lane] = list;
            block_tree_merge<kMWaves>(s_list, list, w, lane);
            if (w == 0 && lane < k) {
                vals[lane] = list ? key_value(list) : -INFINITY;
                ids[lane] = list ? (a.index ? a.index[key_row(list)] : key_row(list)) : -1;
            }
        }
    }
    __syncthreads();
    if (w == 0 && a.lse) {
        double ss = lane < kMWaves ? s_sum[lane] : 0.0;
        ss = wave_sum(ss);
        if (lane == 0) a.lse[t] = (float)((double)mstar + log(ss));
    }
}

}  // namespace

hipError_t launch_logits(const LogitsArgs &a, hipStream_t st)
{
    if (a.B < 1 || a.B > kMaxBlocks || a.T < 1 || a.k < 0 || a.k > 64 || a.M < 1 || a.rpb < 1 ||
        (int64_t)a.B * a.rpb < a.M)
        return hipErrorInvalidValue;
    LogitsArgs arg = a;
    void *args[] = {&arg};
    const void *k1 = a.k > 32 ? reinterpret_cast<const void *>(&logits_kernel<true>)
                              : reinterpret_cast<const void *>(&logits_kernel<false>);
    hipError_t e = hipLaunchKernel(k1, dim3((unsigned)a.B, (unsigned)a.T),
                                   dim3(kThreads), args, 0, st);
    if (e != hipSuccess) return e;
    MergeArgs m;
    m.lse_part = a.part_lse;
    m.kth = a.part_kth;
    m.list = a.part_list;
    m.G = a.B;
    m.k = a.k;
    m.index = a.index;
    m.lse = a.lse;
    m.vals = a.vals;
    m.ids = a.ids;
    void *margs[] = {&m};
    return hipLaunchKernel(reinterpret_cast<const void *>(&logits_merge_kernel), dim3((unsigned)a.T),
                           dim3(kMThreads), margs, 0, st);
}

}  // namespace qmatk
