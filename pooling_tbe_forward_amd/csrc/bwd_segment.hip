// Backward segment reduction + fused exact SGD for gfx950.
//
// Section "Why the backward is the hard half" of the FBTriton TBE article: a
// read row's gradient is the sum over its run of the output-gradient slices of
// the bags that read it (times the per-sample weight); once that sum is
// finished the optimizer updates the row in place and the gradient is never
// materialised; one owner per run means a plain store, no atomics.
// Section "Three tiers, routed by run length": short runs are owned outright
// by one worker; long runs are cut into fixed-size chunks whose partial sums
// meet in a workspace, and a second kernel adds them and applies the update.
//
// gfx950 design:
//  * a row of D fp32 gradient elements is covered by L lanes (VEC elements,
//    16-byte loads); a 64-lane wavefront holds G = 64/L independent workers,
//    each owning one short run (or one long-run chunk, or one long run);
//  * every worker keeps U gradient-row loads in flight, and the weight row is
//    fetched before the contribution loop so its latency overlaps the sums;
//  * accumulation is fp64 for fp32 tables (long Zipf runs would otherwise
//    drift past 1e-5 relative) and fp32 for fp16 tables; the update
//    w - lr*g is rounded once to the storage type;
//  * long-run partials are combined in chunk order, so results are
//    deterministic and independent of scheduling;
//  * work counts are read from device memory; the grids are persistent loops.
#include "tbe_internal.h"

namespace tbe {
namespace {

template <typename T, int N>
struct alignas(sizeof(T) * N) Pack {
    T v[N];
};

// Table owning a linearized key: last t with hash_off[t] <= key.
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

struct SegCommon {
    const TableDesc* tables;
    const uint32_t* hash_off;
    int32_t T;
    int32_t sumD;
    int32_t lpr_log2;      // lanes per row worker (log2)
    const float* grad;
    const uint32_t* sorted_sample;
    const float* sorted_psw;
    const uint32_t* unique;
    const uint32_t* run_start;
    const uint32_t* run_len;
    const uint32_t* counts;
    float lr;
};

// Sum of w_i * grad[sample_i, col .. col+VEC) over sorted positions [i0, i1).
template <typename ACC, int VEC, int U, bool WEIGHTED>
__device__ __forceinline__ void seg_sum(const SegCommon& c, const float* __restrict__ gcol,
                                        uint32_t i0, uint32_t i1, bool tw, ACC (&acc)[VEC])
{
    for (uint32_t i = i0; i < i1; i += U) {
        Pack<float, VEC> g[U];
        float w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
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
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                if (WEIGHTED)
                    acc[k] += static_cast<ACC>(w[u]) * static_cast<ACC>(g[u].v[k]);
                else
                    acc[k] += static_cast<ACC>(g[u].v[k]);
            }
    }
}

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

// Short runs: one worker per run, whole run, then SGD.
template <typename WT, typename ACC, int VEC, int U, bool WEIGHTED>
__global__ __launch_bounds__(256) void k_short_sgd(SegCommon c, WT* __restrict__ weights,
                                                   const uint32_t* __restrict__ short_runs)
{
    const int lane = threadIdx.x & 63;
    const int g_log2 = 6 - c.lpr_log2;
    const int grp = lane >> c.lpr_log2;
    const int sub = lane & ((1 << c.lpr_log2) - 1);
    const uint32_t nshort = c.counts[1];
    const uint32_t wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const uint32_t nwaves = gridDim.x * (blockDim.x >> 6);
    for (uint32_t k0 = wave << g_log2; k0 < nshort; k0 += nwaves << g_log2) {
        const uint32_t k = k0 + grp;
        if (k >= nshort) continue;
        const uint32_t r = short_runs[k];
        const uint32_t s = c.run_start[r];
        const uint32_t len = c.run_len[r];
        const uint32_t key = c.unique[r];
        const int t = find_table(c.hash_off, c.T, key);
        const TableDesc d = c.tables[t];
        const bool tw = WEIGHTED && (d.flags & TD_WEIGHTED);
        WT* __restrict__ wrow = weights + d.w_off + static_cast<int64_t>(key - d.hash_off) * d.D;
        const float* __restrict__ gbase = c.grad + d.out_off;
        for (int c0 = 0; c0 < d.D; c0 += (VEC << c.lpr_log2)) {
            const int col = c0 + sub * VEC;
            if (col >= d.D) continue;
            const Pack<WT, VEC> w_old = *reinterpret_cast<const Pack<WT, VEC>*>(wrow + col);
            ACC acc[VEC];
#pragma unroll
            for (int q = 0; q < VEC; ++q) acc[q] = ACC(0);
            seg_sum<ACC, VEC, U, WEIGHTED>(c, gbase + col, s, s + len, tw, acc);
            sgd_store<WT, ACC, VEC>(wrow + col, w_old, acc, c.lr);
        }
    }
}

// Long runs, step 1: one worker per chunk of `chunk` lookups -> partial sum.
template <typename ACC, int VEC, int U, bool WEIGHTED>
__global__ __launch_bounds__(256) void k_long_split(SegCommon c,
                                                    const uint32_t* __restrict__ long_runs,
                                                    const uint32_t* __restrict__ long_chunk,
                                                    uint32_t chunk, ACC* __restrict__ partials,
                                                    int32_t max_D, uint32_t max_chunks)
{
    const int lane = threadIdx.x & 63;
    const int g_log2 = 6 - c.lpr_log2;
    const int grp = lane >> c.lpr_log2;
    const int sub = lane & ((1 << c.lpr_log2) - 1);
    const uint32_t nlong = c.counts[2];
    const uint32_t nchunks = min(c.counts[3], max_chunks);
    const uint32_t wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const uint32_t nwaves = gridDim.x * (blockDim.x >> 6);
    for (uint32_t q0 = wave << g_log2; q0 < nchunks; q0 += nwaves << g_log2) {
        const uint32_t q = q0 + grp;
        if (q >= nchunks) continue;
        // long run owning chunk q: last lr with long_chunk[lr] <= q
        uint32_t lo = 0, hi = nlong;
        while (hi - lo > 1) {
            const uint32_t mid = (lo + hi) >> 1;
            if (long_chunk[mid] <= q) lo = mid; else hi = mid;
        }
        const uint32_t r = long_runs[lo];
        const uint32_t s = c.run_start[r];
        const uint32_t len = c.run_len[r];
        const uint32_t key = c.unique[r];
        const int t = find_table(c.hash_off, c.T, key);
        const TableDesc d = c.tables[t];
        const bool tw = WEIGHTED && (d.flags & TD_WEIGHTED);
        const uint32_t i0 = s + (q - long_chunk[lo]) * chunk;
        const uint32_t i1 = min(s + len, i0 + chunk);
        const float* __restrict__ gbase = c.grad + d.out_off;
        ACC* __restrict__ prow = partials + static_cast<int64_t>(q) * max_D;
        for (int c0 = 0; c0 < d.D; c0 += (VEC << c.lpr_log2)) {
            const int col = c0 + sub * VEC;
            if (col >= d.D) continue;
            ACC acc[VEC];
#pragma unroll
            for (int k = 0; k < VEC; ++k) acc[k] = ACC(0);
            seg_sum<ACC, VEC, U, WEIGHTED>(c, gbase + col, i0, i1, tw, acc);
#pragma unroll
            for (int k = 0; k < VEC; ++k) prow[col + k] = acc[k];
        }
    }
}

// Long runs, step 2: one worker per long run adds its chunks' partials in
// chunk order, then SGD.
template <typename WT, typename ACC, int VEC>
__global__ __launch_bounds__(256) void k_long_combine(SegCommon c, WT* __restrict__ weights,
                                                      const uint32_t* __restrict__ long_runs,
                                                      const uint32_t* __restrict__ long_chunk,
                                                      const ACC* __restrict__ partials,
                                                      int32_t max_D)
{
    const int lane = threadIdx.x & 63;
    const int g_log2 = 6 - c.lpr_log2;
    const int grp = lane >> c.lpr_log2;
    const int sub = lane & ((1 << c.lpr_log2) - 1);
    const uint32_t nlong = c.counts[2];
    const uint32_t wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const uint32_t nwaves = gridDim.x * (blockDim.x >> 6);
    for (uint32_t k0 = wave << g_log2; k0 < nlong; k0 += nwaves << g_log2) {
        const uint32_t k = k0 + grp;
        if (k >= nlong) continue;
        const uint32_t r = long_runs[k];
        const uint32_t key = c.unique[r];
        const int t = find_table(c.hash_off, c.T, key);
        const TableDesc d = c.tables[t];
        WT* __restrict__ wrow = weights + d.w_off + static_cast<int64_t>(key - d.hash_off) * d.D;
        const uint32_t q0 = long_chunk[k], q1 = long_chunk[k + 1];
        for (int c0 = 0; c0 < d.D; c0 += (VEC << c.lpr_log2)) {
            const int col = c0 + sub * VEC;
            if (col >= d.D) continue;
            const Pack<WT, VEC> w_old = *reinterpret_cast<const Pack<WT, VEC>*>(wrow + col);
            ACC acc[VEC];
#pragma unroll
            for (int j = 0; j < VEC; ++j) acc[j] = ACC(0);
            for (uint32_t q = q0; q < q1; ++q) {
                const ACC* prow = partials + static_cast<int64_t>(q) * max_D + col;
#pragma unroll
                for (int j = 0; j < VEC; ++j) acc[j] += prow[j];
            }
            sgd_store<WT, ACC, VEC>(wrow + col, w_old, acc, c.lr);
        }
    }
}

uint32_t persistent_blocks(int64_t work_items, int lpr_log2)
{
    const int64_t per_block = int64_t(4) << (6 - lpr_log2);  // workers per block
    int64_t b = (work_items + per_block - 1) / per_block;
    if (b > 4096) b = 4096;
    if (b < 1) b = 1;
    return static_cast<uint32_t>(b);
}

template <typename WT, typename ACC, int VEC>
hipError_t launch_all(const BwdArgs& a, SegCommon c)
{
    const BwdLayout& L = a.L;
    const tbe_plan* p = a.plan;
    char* ws = a.ws;
    const uint32_t* short_runs = reinterpret_cast<const uint32_t*>(ws + L.off_short);
    const uint32_t* long_runs = reinterpret_cast<const uint32_t*>(ws + L.off_long);
    const uint32_t* long_chunk = reinterpret_cast<const uint32_t*>(ws + L.off_long_chunk);
    ACC* partials = reinterpret_cast<ACC*>(ws + L.off_partials);
    WT* w = static_cast<WT*>(a.weights);
    constexpr int U = 4;
    const int64_t tau = p->tuning.tau > 0 ? p->tuning.tau : 1;
    const uint32_t chunk = static_cast<uint32_t>(p->tuning.chunk);
    const uint32_t b_short = persistent_blocks(L.N, c.lpr_log2);
    const uint32_t b_chunk = persistent_blocks(L.max_chunks, c.lpr_log2);
    const uint32_t b_long = persistent_blocks(L.N / tau + 1, c.lpr_log2);
    if (a.psw) {
        hipLaunchKernelGGL((k_short_sgd<WT, ACC, VEC, U, true>), dim3(b_short), dim3(256), 0,
                           a.stream, c, w, short_runs);
        hipLaunchKernelGGL((k_long_split<ACC, VEC, U, true>), dim3(b_chunk), dim3(256), 0,
                           a.stream, c, long_runs, long_chunk, chunk, partials, p->max_D,
                           static_cast<uint32_t>(L.max_chunks));
    } else {
        hipLaunchKernelGGL((k_short_sgd<WT, ACC, VEC, U, false>), dim3(b_short), dim3(256), 0,
                           a.stream, c, w, short_runs);
        hipLaunchKernelGGL((k_long_split<ACC, VEC, U, false>), dim3(b_chunk), dim3(256), 0,
                           a.stream, c, long_runs, long_chunk, chunk, partials, p->max_D,
                           static_cast<uint32_t>(L.max_chunks));
    }
    hipLaunchKernelGGL((k_long_combine<WT, ACC, VEC>), dim3(b_long), dim3(256), 0, a.stream, c,
                       w, long_runs, long_chunk, partials, p->max_D);
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
    SegCommon c;
    c.tables = p->d_tables;
    c.hash_off = p->d_hash_off;
    c.T = p->T;
    c.sumD = p->sum_D;
    c.lpr_log2 = lpr_log2;
    c.grad = a.grad;
    c.sorted_sample = reinterpret_cast<const uint32_t*>(ws + L.off_sorted_sample);
    c.sorted_psw = reinterpret_cast<const float*>(ws + L.off_sorted_psw);
    c.unique = reinterpret_cast<const uint32_t*>(ws + L.off_unique);
    c.run_start = reinterpret_cast<const uint32_t*>(ws + L.off_run_start);
    c.run_len = reinterpret_cast<const uint32_t*>(ws + L.off_run_len);
    c.counts = reinterpret_cast<const uint32_t*>(ws + L.off_counts);
    c.lr = a.lr;
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
