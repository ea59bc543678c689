// Backward integer stage for gfx950: linearize, stable LSD radix sort,
// run-length encode, classify runs by length.
//
// Section "Why the backward is the hard half" of the FBTriton TBE article:
// the backward inverts the batch -- every lookup gets the key
// hash_size_cumsum[t] + row (rows of different tables never collide), the
// keys are sorted so that every row's contributors sit next to each other,
// and a run-length encode turns each row into one independent unit of work.
// Section "Three tiers, routed by run length": runs are split against a
// length threshold on the device, with counts that never go back to the host.
//
// Section "Using it, and the import that stops you" shows why the sort must be
// stable and sorted only once: per-sample weights must stay paired with their
// lookup.  Here the sort carries the lookup position j as payload, is stable,
// and its last pass gathers the sample id and per-sample weight of every
// sorted entry, so nothing is ever re-sorted.
//
// Kernels (all on the caller's stream, no host synchronisation):
//   k_linearize    one wavefront per bag: key[j], sample[j]; clears counters
//   per radix pass (digit of <= 8 bits, only ceil(log2(sum rows)) bits):
//     k_radix_up   per-tile digit counts, digit-major, plus global totals
//     k_radix_scan one wavefront per digit: exclusive offsets of every tile
//     k_radix_down stable scatter; ranks from wave ballots (a wave-level
//                  match of equal digits) and per-wave LDS counters
//   k_rle_count    per-tile run heads / long runs / long-run chunks
//   k_rle_scan     one workgroup: tile prefixes and the device totals
//   k_rle_write    unique keys, run starts and lengths, ordered short and long
//                  run lists (ordered compaction, so the lists ascend)
#include "tbe_internal.h"

namespace tbe {

namespace {
constexpr int kRadix = 256;
constexpr int kSortWaves = 4;
constexpr int kRleItems = 4;
constexpr int kRleTile = 256 * kRleItems;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int sort_rounds(int64_t N) { return N > (int64_t(1) << 21) ? 16 : 8; }
}  // namespace

BwdLayout bwd_layout(const tbe_plan* p, int32_t B, int64_t N)
{
    (void)B;
    BwdLayout L;
    L.N = N;
    int bits = 0;
    while (bits < 32 && (uint64_t(1) << bits) < uint64_t(p->sum_rows)) ++bits;
    L.nbits = bits;
    L.npasses = bits == 0 ? 1 : (bits + 7) / 8;
    const int per = bits == 0 ? 1 : (bits + L.npasses - 1) / L.npasses;
    int left = bits == 0 ? 1 : bits;
    for (int i = 0; i < L.npasses; ++i) {
        L.digit_bits[i] = per < left ? per : left;
        left -= L.digit_bits[i];
    }
    L.sort_tile = 64 * kSortWaves * sort_rounds(N);
    L.sort_blocks = static_cast<int32_t>((N + L.sort_tile - 1) / L.sort_tile);
    L.rle_tile = kRleTile;
    L.rle_blocks = static_cast<int32_t>((N + kRleTile - 1) / kRleTile);
    const int64_t tau = p->tuning.tau > 0 ? p->tuning.tau : 1;
    const int64_t C = p->tuning.chunk > 0 ? p->tuning.chunk : 1;
    int64_t mc = N / C + N / tau + 1;
    if (mc > N) mc = N;
    L.max_chunks = mc;

    const size_t n4 = align256(size_t(N + 1) * 4);
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t r = o; o += align256(bytes); return r; };
    L.off_keys[0] = take(n4);
    L.off_keys[1] = take(n4);
    L.off_vals[0] = take(n4);
    L.off_vals[1] = take(n4);
    L.off_sample = take(n4);
    L.off_sorted_sample = take(n4);
    L.off_sorted_psw = take(n4);
    L.off_hist = take(size_t(kRadix) * (L.sort_blocks > 0 ? L.sort_blocks : 1) * 4);
    L.off_unique = take(n4);
    L.off_run_start = take(n4);
    L.off_run_len = take(n4);
    L.off_short = take(n4);
    L.off_long = take(n4);
    L.off_long_chunk = take(n4);
    L.off_tile_counts = take(size_t(L.rle_blocks > 0 ? L.rle_blocks : 1) * 16);
    L.off_counts = take(size_t(16 + 4 * kRadix) * 4);
    const size_t acc = p->wdtype == TBE_F32 ? 8 : 4;
    L.off_partials = take(size_t(mc > 0 ? mc : 1) * p->max_D * acc);
    L.total = o;
    return L;
}

namespace {

__device__ __forceinline__ uint32_t wave_sum(uint32_t v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(v, d);
        if (lane >= d) v += o;
    }
    return v;
}

// ---------------------------------------------------------------------------
template <typename IT>
__global__ __launch_bounds__(256) void k_linearize(
    const TableDesc* __restrict__ tables, uint32_t B, uint32_t total_bags,
    const IT* __restrict__ indices, const IT* __restrict__ offsets, uint32_t* __restrict__ keys,
    uint32_t* __restrict__ sample, uint32_t* __restrict__ zero_buf, int32_t zero_n)
{
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < zero_n; i += blockDim.x) zero_buf[i] = 0u;
    const int lane = threadIdx.x & 63;
    const uint32_t nw = gridDim.x * (blockDim.x >> 6);
    for (uint32_t g = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x >> 6) +
                                                     (threadIdx.x >> 6));
         g < total_bags; g += nw) {
        const uint32_t t = g / B;
        const uint32_t b = g - t * B;
        const uint32_t hoff = tables[t].hash_off;
        const int64_t s = static_cast<int64_t>(offsets[g]);
        const int64_t e = static_cast<int64_t>(offsets[g + 1]);
        for (int64_t p = s + lane; p < e; p += 64) {
            keys[p] = hoff + static_cast<uint32_t>(indices[p]);
            sample[p] = b;
        }
    }
}

// ---------------------------------------------------------------------------
template <int R>
__global__ __launch_bounds__(256) void k_radix_up(
    const uint32_t* __restrict__ keys, uint32_t N, int shift, uint32_t mask, uint32_t nblocks,
    uint32_t* __restrict__ counts, uint32_t* __restrict__ totals)
{
    __shared__ uint32_t h[kRadix];
    const int tid = threadIdx.x;
    h[tid] = 0u;
    __syncthreads();
    const uint32_t base = blockIdx.x * (256u * R);
    uint32_t k[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t i = base + r * 256u + tid;
        k[r] = i < N ? keys[i] : 0u;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t i = base + r * 256u + tid;
        if (i < N) atomicAdd(&h[(k[r] >> shift) & mask], 1u);
    }
    __syncthreads();
    const uint32_t c = h[tid];
    counts[static_cast<size_t>(tid) * nblocks + blockIdx.x] = c;
    if (c) atomicAdd(&totals[tid], c);
}

__global__ __launch_bounds__(256) void k_radix_scan(uint32_t* __restrict__ counts,
                                                    uint32_t nblocks,
                                                    const uint32_t* __restrict__ totals)
{
    const int lane = threadIdx.x & 63;
    const int d = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (d >= kRadix) return;
    uint32_t part = 0;
    for (int k = lane; k < d; k += 64) part += totals[k];
    uint32_t run = wave_sum(part);
    uint32_t* row = counts + static_cast<size_t>(d) * nblocks;
    for (uint32_t b0 = 0; b0 < nblocks; b0 += 64) {
        const uint32_t b = b0 + lane;
        const uint32_t v = b < nblocks ? row[b] : 0u;
        const uint32_t inc = wave_incl_scan(v, lane);
        if (b < nblocks) row[b] = run + inc - v;
        run += __shfl(inc, 63);
    }
}

template <int R, bool FIRST, bool LAST>
__global__ __launch_bounds__(256) void k_radix_down(
    const uint32_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in,
    uint32_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out, uint32_t N, int shift,
    int nbits, uint32_t nblocks, const uint32_t* __restrict__ offs,
    const uint32_t* __restrict__ sample, const float* __restrict__ psw,
    uint32_t* __restrict__ sorted_sample, float* __restrict__ sorted_psw)
{
    __shared__ uint32_t wcnt[kSortWaves][kRadix];
    __shared__ uint32_t gofs[kRadix];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    for (int i = tid; i < kSortWaves * kRadix; i += 256) (&wcnt[0][0])[i] = 0u;
    gofs[tid] = offs[static_cast<size_t>(tid) * nblocks + blockIdx.x];
    __syncthreads();

    const uint32_t mask = (1u << nbits) - 1u;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const uint32_t wbase = blockIdx.x * (256u * R) + static_cast<uint32_t>(wave) * (64u * R);
    uint32_t k[R], v[R], dg[R], rk[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t i = wbase + r * 64u + lane;
        const bool ok = i < N;
        k[r] = ok ? keys_in[i] : 0u;
        v[r] = FIRST ? i : (ok ? vals_in[i] : 0u);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t i = wbase + r * 64u + lane;
        const bool ok = i < N;
        const uint32_t d = (k[r] >> shift) & mask;
        uint64_t peers = __ballot(ok);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool on = (d >> bit) & 1u;
            const uint64_t bal = __ballot(on);
            peers &= on ? bal : ~bal;
        }
        const uint32_t below = static_cast<uint32_t>(__popcll(peers & lt));
        uint32_t base = 0;
        if (ok) base = wcnt[wave][d];
        if (ok && below == 0) wcnt[wave][d] = base + static_cast<uint32_t>(__popcll(peers));
        dg[r] = d;
        rk[r] = base + below;
    }
    __syncthreads();
    {
        uint32_t run = 0;
#pragma unroll
        for (int w = 0; w < kSortWaves; ++w) {
            const uint32_t c = wcnt[w][tid];
            wcnt[w][tid] = run;
            run += c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t i = wbase + r * 64u + lane;
        if (i < N) {
            const uint32_t pos = gofs[dg[r]] + wcnt[wave][dg[r]] + rk[r];
            if (pos >= N) continue;  // unreachable when the counts are consistent
            keys_out[pos] = k[r];
            vals_out[pos] = v[r];
            if (LAST) {
                sorted_sample[pos] = sample[v[r]];
                if (psw) sorted_psw[pos] = psw[v[r]];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Length of the run whose head is at i: galloping then binary search.
__device__ __forceinline__ uint32_t run_length(const uint32_t* __restrict__ keys, uint32_t N,
                                               uint32_t i, uint32_t key)
{
    uint32_t lo = i, step = 1;
    while (lo + step < N && keys[lo + step] == key) {
        lo += step;
        step <<= 1;
    }
    uint32_t hi = (lo + step < N) ? lo + step : N;  // keys[hi] != key or hi == N
    while (hi - lo > 1) {
        const uint32_t mid = lo + (hi - lo) / 2;
        if (keys[mid] == key) lo = mid; else hi = mid;
    }
    return lo - i + 1;
}

struct RunInfo {
    uint32_t head, len, is_long, chunks;
};

__device__ __forceinline__ RunInfo run_info(const uint32_t* __restrict__ keys, uint32_t N,
                                            uint32_t i, uint32_t tau, uint32_t chunk)
{
    RunInfo ri{0, 0, 0, 0};
    if (i >= N) return ri;
    const uint32_t k = keys[i];
    if (i != 0 && keys[i - 1] == k) return ri;
    ri.head = 1;
    ri.len = run_length(keys, N, i, k);
    if (ri.len >= tau) {
        ri.is_long = 1;
        ri.chunks = (ri.len + chunk - 1) / chunk;
    }
    return ri;
}

__global__ __launch_bounds__(256) void k_rle_count(const uint32_t* __restrict__ keys, uint32_t N,
                                                   uint32_t tau, uint32_t chunk,
                                                   uint32_t* __restrict__ tile_counts)
{
    __shared__ uint32_t red[3][4];
    const int tid = threadIdx.x;
    const uint32_t i0 = blockIdx.x * kRleTile + tid * kRleItems;
    uint32_t h = 0, l = 0, c = 0;
#pragma unroll
    for (int q = 0; q < kRleItems; ++q) {
        const RunInfo ri = run_info(keys, N, i0 + q, tau, chunk);
        h += ri.head;
        l += ri.is_long;
        c += ri.chunks;
    }
    h = wave_sum(h);
    l = wave_sum(l);
    c = wave_sum(c);
    if ((tid & 63) == 0) {
        red[0][tid >> 6] = h;
        red[1][tid >> 6] = l;
        red[2][tid >> 6] = c;
    }
    __syncthreads();
    if (tid < 3)
        tile_counts[blockIdx.x * 4 + tid] = red[tid][0] + red[tid][1] + red[tid][2] + red[tid][3];
}

// One workgroup of 1024 threads: exclusive prefix of the per-tile
// (heads, long runs, chunks) and the device totals.
__global__ __launch_bounds__(1024) void k_rle_scan(uint32_t* __restrict__ tile_counts,
                                                   uint32_t ntiles, uint32_t N,
                                                   uint32_t* __restrict__ counts,
                                                   uint32_t* __restrict__ run_start,
                                                   uint32_t* __restrict__ long_chunk)
{
    __shared__ uint32_t wsum[3][16];
    __shared__ uint32_t carry[3];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    if (tid < 3) carry[tid] = 0;
    __syncthreads();
    for (uint32_t t0 = 0; t0 < ntiles; t0 += 1024) {
        const uint32_t t = t0 + tid;
        uint32_t v[3], inc[3];
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            v[c] = t < ntiles ? tile_counts[t * 4 + c] : 0u;
            inc[c] = wave_incl_scan(v[c], lane);
            if (lane == 63) wsum[c][wave] = inc[c];
        }
        __syncthreads();
        if (tid < 3) {
            uint32_t run = carry[tid];
            for (int w = 0; w < 16; ++w) {
                const uint32_t x = wsum[tid][w];
                wsum[tid][w] = run;
                run += x;
            }
            carry[tid] = run;
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 3; ++c)
            if (t < ntiles) tile_counts[t * 4 + c] = wsum[c][wave] + inc[c] - v[c];
        __syncthreads();
    }
    if (tid == 0) {
        const uint32_t runs = carry[0], nlong = carry[1], chunks = carry[2];
        counts[0] = runs;
        counts[1] = runs - nlong;
        counts[2] = nlong;
        counts[3] = chunks;
        run_start[runs] = N;
        long_chunk[nlong] = chunks;
    }
}

__global__ __launch_bounds__(256) void k_rle_write(
    const uint32_t* __restrict__ keys, uint32_t N, uint32_t tau, uint32_t chunk,
    const uint32_t* __restrict__ tile_prefix, uint32_t* __restrict__ unique,
    uint32_t* __restrict__ run_start, uint32_t* __restrict__ run_len,
    uint32_t* __restrict__ short_runs, uint32_t* __restrict__ long_runs,
    uint32_t* __restrict__ long_chunk)
{
    __shared__ uint32_t wsum[3][4];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const uint32_t i0 = blockIdx.x * kRleTile + tid * kRleItems;
    RunInfo ri[kRleItems];
    uint32_t v[3] = {0, 0, 0};
#pragma unroll
    for (int q = 0; q < kRleItems; ++q) {
        ri[q] = run_info(keys, N, i0 + q, tau, chunk);
        v[0] += ri[q].head;
        v[1] += ri[q].is_long;
        v[2] += ri[q].chunks;
    }
    uint32_t inc[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        inc[c] = wave_incl_scan(v[c], lane);
        if (lane == 63) wsum[c][wave] = inc[c];
    }
    __syncthreads();
    uint32_t base[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        uint32_t pre = tile_prefix[blockIdx.x * 4 + c];
        for (int w = 0; w < wave; ++w) pre += wsum[c][w];
        base[c] = pre + inc[c] - v[c];
    }
    uint32_t r = base[0], lb = base[1], cb = base[2];
#pragma unroll
    for (int q = 0; q < kRleItems; ++q) {
        if (!ri[q].head || r >= N || lb > r) continue;  // guards: unreachable when consistent
        const uint32_t i = i0 + q;
        unique[r] = keys[i];
        run_start[r] = i;
        run_len[r] = ri[q].len;
        if (ri[q].is_long) {
            long_runs[lb] = r;
            long_chunk[lb] = cb;
            ++lb;
            cb += ri[q].chunks;
        } else {
            short_runs[r - lb] = r;
        }
        ++r;
    }
}

template <int R>
hipError_t sort_passes(BwdArgs& a)
{
    const BwdLayout& L = a.L;
    const uint32_t N = static_cast<uint32_t>(L.N);
    const uint32_t nb = static_cast<uint32_t>(L.sort_blocks);
    char* ws = a.ws;
    uint32_t* keys[2] = {reinterpret_cast<uint32_t*>(ws + L.off_keys[0]),
                         reinterpret_cast<uint32_t*>(ws + L.off_keys[1])};
    uint32_t* vals[2] = {reinterpret_cast<uint32_t*>(ws + L.off_vals[0]),
                         reinterpret_cast<uint32_t*>(ws + L.off_vals[1])};
    uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.off_hist);
    uint32_t* counters = reinterpret_cast<uint32_t*>(ws + L.off_counts);
    uint32_t* sample = reinterpret_cast<uint32_t*>(ws + L.off_sample);
    uint32_t* ssample = reinterpret_cast<uint32_t*>(ws + L.off_sorted_sample);
    float* spsw = reinterpret_cast<float*>(ws + L.off_sorted_psw);
    int cur = 0;
    int shift = 0;
    for (int pass = 0; pass < L.npasses; ++pass) {
        const int nbits = L.digit_bits[pass];
        const uint32_t mask = (1u << nbits) - 1u;
        uint32_t* totals = counters + 16 + pass * kRadix;
        hipLaunchKernelGGL(k_radix_up<R>, dim3(nb), dim3(256), 0, a.stream, keys[cur], N, shift,
                           mask, nb, hist, totals);
        hipLaunchKernelGGL(k_radix_scan, dim3(kRadix / 4), dim3(256), 0, a.stream, hist, nb,
                           totals);
        const bool first = pass == 0, last = pass == L.npasses - 1;
        auto kern = first ? (last ? k_radix_down<R, true, true> : k_radix_down<R, true, false>)
                          : (last ? k_radix_down<R, false, true> : k_radix_down<R, false, false>);
        hipLaunchKernelGGL(kern, dim3(nb), dim3(256), 0, a.stream, keys[cur], vals[cur],
                           keys[cur ^ 1], vals[cur ^ 1], N, shift, nbits, nb, hist, sample, a.psw,
                           ssample, spsw);
        cur ^= 1;
        shift += nbits;
    }
    a.final_buf = cur;
    return hipGetLastError();
}

}  // namespace

hipError_t run_sort_rle(BwdArgs& a)
{
    const tbe_plan* p = a.plan;
    const BwdLayout& L = a.L;
    char* ws = a.ws;
    const uint32_t N = static_cast<uint32_t>(L.N);
    const uint32_t total_bags = static_cast<uint32_t>(p->T) * static_cast<uint32_t>(a.B);
    uint32_t* counters = reinterpret_cast<uint32_t*>(ws + L.off_counts);
    const int zero_n = 16 + 4 * kRadix;
    {
        const uint32_t waves = total_bags < 65536u ? total_bags : 65536u;
        const uint32_t blocks = (waves + 3) / 4 > 0 ? (waves + 3) / 4 : 1;
        uint32_t* keys0 = reinterpret_cast<uint32_t*>(ws + L.off_keys[0]);
        uint32_t* sample = reinterpret_cast<uint32_t*>(ws + L.off_sample);
        if (p->idtype == TBE_I64)
            hipLaunchKernelGGL(k_linearize<int64_t>, dim3(blocks), dim3(256), 0, a.stream,
                               p->d_tables, static_cast<uint32_t>(a.B), total_bags,
                               static_cast<const int64_t*>(a.indices),
                               static_cast<const int64_t*>(a.offsets), keys0, sample, counters,
                               zero_n);
        else
            hipLaunchKernelGGL(k_linearize<int32_t>, dim3(blocks), dim3(256), 0, a.stream,
                               p->d_tables, static_cast<uint32_t>(a.B), total_bags,
                               static_cast<const int32_t*>(a.indices),
                               static_cast<const int32_t*>(a.offsets), keys0, sample, counters,
                               zero_n);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (N == 0) {
        a.final_buf = 0;
        return hipSuccess;   // counters are zero; run_start[0] is never read
    }
    e = sort_rounds(L.N) == 16 ? sort_passes<16>(a) : sort_passes<8>(a);
    if (e != hipSuccess) return e;

    const uint32_t* skeys = reinterpret_cast<const uint32_t*>(ws + L.off_keys[a.final_buf]);
    uint32_t* tiles = reinterpret_cast<uint32_t*>(ws + L.off_tile_counts);
    const uint32_t tau = static_cast<uint32_t>(p->tuning.tau);
    const uint32_t chunk = static_cast<uint32_t>(p->tuning.chunk);
    const uint32_t nt = static_cast<uint32_t>(L.rle_blocks);
    hipLaunchKernelGGL(k_rle_count, dim3(nt), dim3(256), 0, a.stream, skeys, N, tau, chunk, tiles);
    hipLaunchKernelGGL(k_rle_scan, dim3(1), dim3(1024), 0, a.stream, tiles, nt, N, counters,
                       reinterpret_cast<uint32_t*>(ws + L.off_run_start),
                       reinterpret_cast<uint32_t*>(ws + L.off_long_chunk));
    hipLaunchKernelGGL(k_rle_write, dim3(nt), dim3(256), 0, a.stream, skeys, N, tau, chunk, tiles,
                       reinterpret_cast<uint32_t*>(ws + L.off_unique),
                       reinterpret_cast<uint32_t*>(ws + L.off_run_start),
                       reinterpret_cast<uint32_t*>(ws + L.off_run_len),
                       reinterpret_cast<uint32_t*>(ws + L.off_short),
                       reinterpret_cast<uint32_t*>(ws + L.off_long),
                       reinterpret_cast<uint32_t*>(ws + L.off_long_chunk));
    return hipGetLastError();
}

}  // namespace tbe
