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
// Work split: grid (B, T); block b of token t streams rows [b*rpb, (b+1)*rpb) with 4 waves.
// Each lane keeps an online (max, sum of exp(y - max)); each wave keeps its 64 best (value, row)
// pairs sorted across its lanes (lane i holds the i-th best) and merges a 64-row chunk into that
// list only when some lane beats the current k-th best (a bitonic sort of the chunk and a
// bitonic merge, all in registers through lane shuffles).  The block's four waves combine in
// LDS; the block publishes (max, sum, k best) to the workspace, and the last block of the token
// to arrive (arrival counter, reset by that block) merges the B partials in block order:
// deterministic output, no memset between calls.
//
// Order: value descending, equal values by ascending row.  Empty slots are (-inf, INT_MAX).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "qmat_logits.h"

namespace qmatk {

namespace {

constexpr int kRowEmpty = 0x7FFFFFFF;

__device__ __forceinline__ bool better(float v1, int r1, float v2, int r2)
{
    return v1 > v2 || (v1 == v2 && r1 < r2);
}

// one compare-exchange step between lanes `lane` and `lane ^ stride`; keep_better selects
// which of the two this lane keeps
__device__ __forceinline__ void cmpx(float &v, int &r, int stride, bool keep_better)
{
    const float pv = __shfl_xor(v, stride);
    const int pr = __shfl_xor(r, stride);
    const bool take = keep_better ? better(pv, pr, v, r) : better(v, r, pv, pr);
    if (take) {
        v = pv;
        r = pr;
    }
}

// bitonic sort of the wave's 64 (v, r) pairs, best first
__device__ __forceinline__ void wave_sort(float &v, int &r, int lane)
{
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const bool lower = (lane & stride) == 0, first_half_desc = (lane & size) == 0;
            cmpx(v, r, stride, lower == first_half_desc);
        }
}

// L (sorted, best first) := the 64 best of L and S (both sorted, best first)
__device__ __forceinline__ void wave_merge(float &lv, int &lr, float sv, int sr, int lane)
{
    const float qv = __shfl(sv, 63 - lane);
    const int qr = __shfl(sr, 63 - lane);
    if (better(qv, qr, lv, lr)) {
        lv = qv;
        lr = qr;
    }
#pragma unroll
    for (int stride = 32; stride > 0; stride >>= 1) cmpx(lv, lr, stride, (lane & stride) == 0);
}

// (m, s) := combination of two online log-sum-exp states
__device__ __forceinline__ void lse_combine(float &m, float &s, float pm, float ps)
{
    if (pm == -INFINITY) return;
    if (m == -INFINITY) {
        m = pm;
        s = ps;
        return;
    }
    const float mx = fmaxf(m, pm);
    s = s * expf(m - mx) + ps * expf(pm - mx);
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

constexpr int kWaves = 4;

__global__ __launch_bounds__(256) void logits_kernel(LogitsArgs a)
{
    __shared__ float s_v[kWaves][64];
    __shared__ int s_r[kWaves][64];
    __shared__ float s_m[kWaves], s_s[kWaves];
    __shared__ double s_d[256];
    __shared__ int s_last;

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int b = blockIdx.x, t = blockIdx.y;
    const int k = a.k;
    const float *yt = a.y + (int64_t)t * a.ldy;
    const int r0 = b * a.rpb;
    const int r1 = r0 + a.rpb < a.M ? r0 + a.rpb : a.M;

    float lv = -INFINITY, m = -INFINITY, s = 0.f;
    int lr = kRowEmpty;
    // 4 chunks of 64 rows per wave in flight: rows r0 + 256*(4i + j) + 64*w + lane
    for (int base = r0; base < r1; base += 4 * 256) {
        float v[4];
        int row[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            row[j] = base + 256 * j + 64 * w + lane;
            v[j] = row[j] < r1 ? yt[row[j]] : -INFINITY;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool in = row[j] < r1;
            if (in) {
                if (v[j] > m) {
                    s = s * expf(m - v[j]) + 1.f;
                    m = v[j];
                } else {
                    s += expf(v[j] - m);
                }
            }
            if (k > 0) {
                const int rr = in ? row[j] : kRowEmpty;
                const float tv = __shfl(lv, k - 1);
                const int tr = __shfl(lr, k - 1);
                if (__any(better(v[j], rr, tv, tr))) {
                    float cv = v[j];
                    int cr = rr;
                    wave_sort(cv, cr, lane);
                    wave_merge(lv, lr, cv, cr, lane);
                }
            }
        }
    }
    // wave log-sum-exp
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float pm = __shfl_xor(m, off), ps = __shfl_xor(s, off);
        lse_combine(m, s, pm, ps);
    }
    s_v[w][lane] = lv;
    s_r[w][lane] = lr;
    if (lane == 0) {
        s_m[w] = m;
        s_s[w] = s;
    }
    __syncthreads();

    // block partial: wave 0 merges the other waves' lists and states, then publishes
    const int kc = a.k;
    float *pf = a.part_f + ((int64_t)t * a.B + b) * (2 + kc);
    int32_t *pi = a.part_i + ((int64_t)t * a.B + b) * kc;
    uint32_t sink = 0;
    if (w == 0) {
        for (int o = 1; o < kWaves; ++o) {
            if (k > 0) wave_merge(lv, lr, s_v[o][lane], s_r[o][lane], lane);
            lse_combine(m, s, s_m[o], s_s[o]);
        }
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

    // last block of token t: merge the B partials in block order
    const float *tf = a.part_f + (int64_t)t * a.B * (2 + kc);
    const int32_t *ti = a.part_i + (int64_t)t * a.B * kc;
    // log-sum-exp: global max, then the scaled sums in double, fixed order
    float mx = -INFINITY;
    for (int bb = threadIdx.x; bb < a.B; bb += blockDim.x) mx = fmaxf(mx, ld_agent(tf + (int64_t)bb * (2 + kc)));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0) s_m[w] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    double acc = 0.0;
    for (int bb = threadIdx.x; bb < a.B; bb += blockDim.x) {
        const float bm = ld_agent(tf + (int64_t)bb * (2 + kc));
        const float bs = ld_agent(tf + (int64_t)bb * (2 + kc) + 1);
        if (bm != -INFINITY) acc += (double)bs * exp((double)bm - (double)mx);
    }
    s_d[threadIdx.x] = acc;
    // top-k: wave w merges the lists of blocks w, w + 4, ... (each already sorted, best first);
    // a list whose best entry does not beat the current k-th best is skipped whole
    lv = -INFINITY;
    lr = kRowEmpty;
    if (k > 0) {
        for (int bb = w; bb < a.B; bb += kWaves) {
            const float *bf = tf + (int64_t)bb * (2 + kc) + 2;
            const float cv0 = ld_agent(bf);
            const int cr0 = ld_agent(ti + (int64_t)bb * kc);
            if (!better(cv0, cr0, __shfl(lv, k - 1), __shfl(lr, k - 1))) continue;
            float cv = lane < kc ? ld_agent(bf + lane) : -INFINITY;
            int cr = lane < kc ? ld_agent(ti + (int64_t)bb * kc + lane) : kRowEmpty;
            wave_merge(lv, lr, cv, cr, lane);
        }
    }
    __syncthreads();  // s_m reads above are done before s_v / s_r are reused
    s_v[w][lane] = lv;
    s_r[w][lane] = lr;
    __syncthreads();
    if (w == 0) {
        if (k > 0)
            for (int o = 1; o < kWaves; ++o) wave_merge(lv, lr, s_v[o][lane], s_r[o][lane], lane);
        if (lane < kc) {
            a.vals[(int64_t)t * kc + lane] = lv;
            a.ids[(int64_t)t * kc + lane] = lr == kRowEmpty ? -1 : (a.index ? a.index[lr] : lr);
        }
        if (lane == 0 && a.lse) {
            double tot = 0.0;
            for (int i = 0; i < 256; ++i) tot += s_d[i];
            a.lse[t] = (float)((double)mx + log(tot));
        }
    }
    if (threadIdx.x == 0) __hip_atomic_store(&a.counter[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_logits(const LogitsArgs &a, hipStream_t st)
{
    LogitsArgs arg = a;
    void *args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void *>(&logits_kernel), dim3((unsigned)a.B, (unsigned)a.T),
                           dim3(256), args, 0, st);
}

}  // namespace qmatk
