// Backward segment reduction + fused exact SGD for gfx950.
//
// Section "Why the backward is the hard half" of the FBTriton TBE article: a
// read row's gradient is the sum over its run of the output-gradient slices of
// the bags that read it (times the per-sample weight); once that sum is
// finished the optimizer updates the row in place and the gradient is never
// materialised; one owner per run means a plain store, no atomics.
// Section "Three tiers, routed by run length": short runs are owned outright
// by one worker; long runs are cut into fixed-size chunks whose partial sums
// meet in a workspace and are added once all have landed (the article's fused
// tier: each chunk publishes its partial, fences, and counts itself in).
// Section "Where the backward speedup comes from": the short-run kernel's
// speed is latency hiding -- how many independent row loads are in flight.
//
// gfx950 design:
//  * a gradient row of D fp32 elements is covered by L lanes (VEC elements,
//    up to 16-byte loads); a 64-lane wavefront holds G = 64/L workers;
//  * short runs: each worker owns U runs at once (U slots).  It issues the U
//    weight-row loads up front, then walks the runs' contributions in lock
//    step, so U sample-id loads and U gradient-row loads are in flight per
//    step; a run of one lookup costs one dependent step, not U;
//  * long runs: the same launch carries chunk workers (one chunk of `chunk`
//    lookups each) that write partial sums; the worker finishing a run's last
//    chunk adds the run's partials in chunk order and applies the update, so
//    the result does not depend on scheduling;
//  * accumulation is fp64 for fp32 tables (long Zipf runs would otherwise
//    drift past 1e-5 relative) and fp32 for fp16 tables; w - lr*g is rounded
//    once to the storage type;
//  * work counts are read from device memory; grids are persistent loops.
#include "tbe_internal.h"

namespace tbe {
namespace {

template <typename T, int N>
struct alignas(sizeof(T) * N) Pack {
    T v[N];
};

__device__ __forceinline__ int find_table(const uint32_t* __restrict__ hash_off, int T,
                                          uint32_t key)
{
    int lo = 0, hi = T;  // hash_off[lo] <= key < hash_off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (hash_off[mid] <= key) lo = mid; else hi = mid;
    }
    return lo;
}

struct SegArgs {
    const TableDesc* tables;
    const uint32_t* hash_off;
    int32_t T;
    int32_t sumD;
    int32_t lpr_log2;      // lanes per worker (log2)
    int32_t max_D;
    const float* grad;
    const uint32_t* sorted_sample;
    const float* sorted_psw;
    const uint4* short_info;   // {key, start, len, table}
    const uint4* long_info;    // {key, start, len, first chunk}
    uint32_t* arrive;          // per long run: chunks whose partial has landed
    const uint32_t* counts;    // runs, short, long, chunks
    uint32_t chunk;
    uint32_t max_chunks;
    uint32_t max_long;
    float lr;
    uint32_t short_blocks;     // blocks [0, short_blocks) take short runs
};

template <typename WT, typename ACC, int VEC>
__device__ __forceinline__ void sgd_store(WT* __restrict__ wp, const Pack<WT, VEC>& w_old,
                                          const ACC (&acc)[VEC], float lr)
{
    Pack<WT, VEC> o;
#pragma unroll
    for (int k = 0; k < VEC; ++k)
        o.v[k] = static_cast<WT>(static_cast<ACC>(static_cast<float>(w_old.v[k])) -
                                 static_cast<ACC>(lr) * acc[k]);
    *reinterpret_cast<Pack<WT, VEC>*>(wp) = o;
}

// Sum of w_i * grad[sample_i, col .. col+VEC) over sorted positions [i0, i1).
template <typename ACC, int VEC, int UC, bool WEIGHTED>
__device__ __forceinline__ void seg_sum(const SegArgs& c, const float* __restrict__ gcol,
                                        uint32_t i0, uint32_t i1, bool tw, ACC (&acc)[VEC])
{
    for (uint32_t i = i0; i < i1; i += UC) {
        Pack<float, VEC> g[UC];
        float w[UC];
#pragma unroll
        for (int u = 0; u < UC; ++u) {
            const uint32_t ii = i + u;
            if (ii < i1) {
                const uint32_t smp = c.sorted_sample[ii];
                w[u] = (WEIGHTED && tw) ? c.sorted_psw[ii] : 1.f;
                g[u] = *reinterpret_cast<const Pack<float, VEC>*>(
                    gcol + static_cast<int64_t>(smp) * c.sumD);
            } else {
                w[u] = 0.f;
#pragma unroll
                for (int k = 0; k < VEC; ++k) g[u].v[k] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < UC; ++u)
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                if (WEIGHTED)
                    acc[k] += static_cast<ACC>(w[u]) * static_cast<ACC>(g[u].v[k]);
                else
                    acc[k] += static_cast<ACC>(g[u].v[k]);
            }
    }
}

template <typename WT, typename ACC, int VEC, int U, bool WEIGHTED>
__device__ __forceinline__ void short_runs(const SegArgs& c, WT* __restrict__ weights,
                                           uint32_t wave, uint32_t nwaves)
{
    const int lane = threadIdx.x & 63;
    const int g_log2 = 6 - c.lpr_log2;
    const int G = 1 << g_log2;
    const int grp = lane >> c.lpr_log2;
    const int sub = lane & ((1 << c.lpr_log2) - 1);
    const uint32_t nshort = c.counts[1];
    const uint32_t per_wave = static_cast<uint32_t>(G * U);
    for (uint32_t k0 = wave * per_wave; k0 < nshort; k0 += nwaves * per_wave) {
        uint4 info[U];
        TableDesc d[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t k = k0 + static_cast<uint32_t>(u * G + grp);
            info[u] = k < nshort ? c.short_info[k] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) d[u] = c.tables[info[u].w];
        for (int c0 = 0; c0 < c.max_D; c0 += (VEC << c.lpr_log2)) {
            const int col = c0 + sub * VEC;
            Pack<WT, VEC> w_old[U];
            ACC acc[U][VEC];
            uint32_t maxlen = 0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool act = info[u].z > 0 && col < d[u].D;
                if (act) {
                    WT* wrow = weights + d[u].w_off +
                               static_cast<int64_t>(info[u].x - d[u].hash_off) * d[u].D;
                    w_old[u] = *reinterpret_cast<const Pack<WT, VEC>*>(wrow + col);
                    maxlen = max(maxlen, info[u].z);
                } else {
                    info[u].z = act ? info[u].z : 0u;
                }
#pragma unroll
                for (int q = 0; q < VEC; ++q) acc[u][q] = ACC(0);
            }
            for (uint32_t j = 0; j < maxlen; ++j) {
                Pack<float, VEC> g[U];
                float w[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    w[u] = 0.f;
                    if (j < info[u].z) {
                        const uint32_t ii = info[u].y + j;
                        const uint32_t smp = c.sorted_sample[ii];
                        if (WEIGHTED)
                            w[u] = (d[u].flags & TD_WEIGHTED) ? c.sorted_psw[ii] : 1.f;
                        g[u] = *reinterpret_cast<const Pack<float, VEC>*>(
                            c.grad + static_cast<int64_t>(smp) * c.sumD + d[u].out_off + col);
                    } else {
#pragma unroll
                        for (int q = 0; q < VEC; ++q) g[u].v[q] = 0.f;
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int q = 0; q < VEC; ++q) {
                        if (WEIGHTED)
                            acc[u][q] += static_cast<ACC>(w[u]) * static_cast<ACC>(g[u].v[q]);
                        else
                            acc[u][q] += static_cast<ACC>(g[u].v[q]);
                    }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (info[u].z == 0) continue;
                WT* wrow = weights + d[u].w_off +
                           static_cast<int64_t>(info[u].x - d[u].hash_off) * d[u].D;
                sgd_store<WT, ACC, VEC>(wrow + col, w_old[u], acc[u], c.lr);
            }
        }
    }
}

// Long runs: one worker per chunk of `chunk` lookups writes its partial sum;
// the worker that completes a run's last chunk (per-run arrival counter,
// release fence before the count, acquire fence after) adds the run's
// partials in chunk order and applies the update.  Nothing waits.
template <typename WT, typename ACC, int VEC, bool WEIGHTED>
__device__ __forceinline__ void long_chunks(const SegArgs& c, WT* __restrict__ weights,
                                            ACC* __restrict__ partials, uint32_t wave,
                                            uint32_t nwaves)
{
    const int lane = threadIdx.x & 63;
    const int g_log2 = 6 - c.lpr_log2;
    const int grp = lane >> c.lpr_log2;
    const int sub = lane & ((1 << c.lpr_log2) - 1);
    const int leader = grp << c.lpr_log2;
    const uint32_t nlong = min(c.counts[2], c.max_long);
    const uint32_t nchunks = min(c.counts[3], c.max_chunks);
    for (uint32_t q0 = wave << g_log2; q0 < nchunks; q0 += nwaves << g_log2) {
        const uint32_t q = q0 + grp;
        const bool have = q < nchunks;
        uint32_t lo = 0;
        uint4 li = make_uint4(0, 0, 0, 0);
        TableDesc d{};
        if (have) {
            uint32_t hi = nlong;  // long run owning chunk q: last with first chunk <= q
            while (hi - lo > 1) {
                const uint32_t mid = (lo + hi) >> 1;
                if (c.long_info[mid].w <= q) lo = mid; else hi = mid;
            }
            li = c.long_info[lo];
            d = c.tables[find_table(c.hash_off, c.T, li.x)];
            const bool tw = WEIGHTED && (d.flags & TD_WEIGHTED);
            const uint32_t i0 = li.y + (q - li.w) * c.chunk;
            const uint32_t i1 = min(li.y + li.z, i0 + c.chunk);
            ACC* __restrict__ prow = partials + static_cast<int64_t>(q) * c.max_D;
            for (int c0 = 0; c0 < d.D; c0 += (VEC << c.lpr_log2)) {
                const int col = c0 + sub * VEC;
                if (col >= d.D) continue;
                ACC acc[VEC];
#pragma unroll
                for (int k = 0; k < VEC; ++k) acc[k] = ACC(0);
                seg_sum<ACC, VEC, 4, WEIGHTED>(c, c.grad + d.out_off + col, i0, i1, tw, acc);
#pragma unroll
                for (int k = 0; k < VEC; ++k) prow[col + k] = acc[k];
            }
        }
        __threadfence();                       // partials visible device-wide first
        uint32_t prior = 0;
        if (have && sub == 0) prior = atomicAdd(&c.arrive[lo], 1u);
        prior = __shfl(prior, leader);
        const uint32_t nq = (li.z + c.chunk - 1) / c.chunk;
        if (!have || prior + 1 != nq) continue;  // not the run's last chunk
        __threadfence();                       // see every other chunk's partial
        WT* __restrict__ wrow = weights + d.w_off + static_cast<int64_t>(li.x - d.hash_off) * d.D;
        for (int c0 = 0; c0 < d.D; c0 += (VEC << c.lpr_log2)) {
            const int col = c0 + sub * VEC;
            if (col >= d.D) continue;
            const Pack<WT, VEC> w_old = *reinterpret_cast<const Pack<WT, VEC>*>(wrow + col);
            ACC acc[VEC];
#pragma unroll
            for (int j = 0; j < VEC; ++j) acc[j] = ACC(0);
            for (uint32_t qq = li.w; qq < li.w + nq && qq < c.max_chunks; ++qq) {
                const ACC* pr = partials + static_cast<int64_t>(qq) * c.max_D + col;
#pragma unroll
                for (int j = 0; j < VEC; ++j) acc[j] += pr[j];
            }
            sgd_store<WT, ACC, VEC>(wrow + col, w_old, acc, c.lr);
        }
    }
}

template <typename WT, typename ACC, int VEC, int U, bool WEIGHTED>
__global__ __launch_bounds__(256) void k_segment(SegArgs c, WT* __restrict__ weights,
                                                 ACC* __restrict__ partials)
{
    const uint32_t wib = threadIdx.x >> 6;
    if (blockIdx.x < c.short_blocks)
        short_runs<WT, ACC, VEC, U, WEIGHTED>(c, weights, blockIdx.x * 4 + wib,
                                              c.short_blocks * 4);
    else
        long_chunks<WT, ACC, VEC, WEIGHTED>(c, weights, partials,
                                            (blockIdx.x - c.short_blocks) * 4 + wib,
                                            (gridDim.x - c.short_blocks) * 4);
}

uint32_t blocks_for(int64_t work_items, int64_t per_block, int64_t cap)
{
    int64_t b = (work_items + per_block - 1) / per_block;
    if (b > cap) b = cap;
    if (b < 1) b = 1;
    return static_cast<uint32_t>(b);
}

template <typename WT, typename ACC, int VEC>
hipError_t launch_all(const BwdArgs& a, SegArgs c)
{
    const BwdLayout& L = a.L;
    char* ws = a.ws;
    ACC* partials = reinterpret_cast<ACC*>(ws + L.off_partials);
    WT* w = static_cast<WT*>(a.weights);
    constexpr int U = 4;
    const int G = 1 << (6 - c.lpr_log2);
    c.short_blocks = blocks_for(L.N, int64_t(4) * G * U, 2048);
    const uint32_t b_chunk = blocks_for(L.max_chunks, int64_t(4) * G, 1024);
    if (a.psw)
        hipLaunchKernelGGL((k_segment<WT, ACC, VEC, U, true>), dim3(c.short_blocks + b_chunk),
                           dim3(256), 0, a.stream, c, w, partials);
    else
        hipLaunchKernelGGL((k_segment<WT, ACC, VEC, U, false>), dim3(c.short_blocks + b_chunk),
                           dim3(256), 0, a.stream, c, w, partials);
    return hipGetLastError();
}

}  // namespace

hipError_t run_segment_sgd(const BwdArgs& a)
{
    const tbe_plan* p = a.plan;
    const BwdLayout& L = a.L;
    if (L.N == 0) return hipSuccess;
    int vec = 4;
    for (int t = 0; t < p->T; ++t)
        while (p->dims[t] % vec) vec >>= 1;
    if (reinterpret_cast<uintptr_t>(a.grad) % (vec * 4)) vec = 1;
    const size_t wbytes = p->wdtype == TBE_F32 ? 4 : 2;
    while (vec > 1 && reinterpret_cast<uintptr_t>(a.weights) % (vec * wbytes)) vec >>= 1;
    const int lanes = (p->max_D + vec - 1) / vec;
    int lpr_log2 = 0;
    while ((1 << lpr_log2) < lanes && lpr_log2 < 6) ++lpr_log2;

    char* ws = a.ws;
    SegArgs c;
    c.tables = p->d_tables;
    c.hash_off = p->d_hash_off;
    c.T = p->T;
    c.sumD = p->sum_D;
    c.lpr_log2 = lpr_log2;
    c.max_D = p->max_D;
    c.grad = a.grad;
    c.sorted_sample = reinterpret_cast<const uint32_t*>(ws + L.off_sorted_sample);
    c.sorted_psw = reinterpret_cast<const float*>(ws + L.off_sorted_psw);
    c.short_info = reinterpret_cast<const uint4*>(ws + L.off_short_info);
    c.long_info = reinterpret_cast<const uint4*>(ws + L.off_long_info);
    c.arrive = reinterpret_cast<uint32_t*>(ws + L.off_arrive);
    c.counts = reinterpret_cast<const uint32_t*>(ws + L.off_ctl) + kCtlCounts;
    c.chunk = static_cast<uint32_t>(p->tuning.chunk);
    c.max_chunks = static_cast<uint32_t>(L.max_chunks);
    c.max_long = static_cast<uint32_t>(L.max_long);
    c.lr = a.lr;
    c.short_blocks = 0;
    if (p->wdtype == TBE_F32) {
        switch (vec) {
        case 4: return launch_all<float, double, 4>(a, c);
        case 2: return launch_all<float, double, 2>(a, c);
        default: return launch_all<float, double, 1>(a, c);
        }
    }
    switch (vec) {
    case 4: return launch_all<_Float16, float, 4>(a, c);
    case 2: return launch_all<_Float16, float, 2>(a, c);
    default: return launch_all<_Float16, float, 1>(a, c);
    }
}

}  // namespace tbe
