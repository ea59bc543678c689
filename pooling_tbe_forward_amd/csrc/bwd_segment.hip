// Backward segment reduction + fused exact SGD for gfx950.
//
// Section "Why the backward is the hard half" of the FBTriton TBE article: a
// read row's gradient is the sum over its run of the output-gradient slices of
// the bags that read it (times the per-sample weight); once that sum is
// finished the optimizer updates the row in place and the gradient is never
// materialised; one owner per run means a plain store, no atomics.
// Section "Three tiers, routed by run length": short runs are owned outright
// by one worker; long runs are cut into fixed-size chunks whose partial sums
// meet in a workspace and a second kernel adds them and applies the update.
// Section "Where the backward speedup comes from": the short-run kernel's
// speed is latency hiding -- how many independent row loads are in flight.
//
// gfx950 design:
//  * a gradient row of D fp32 elements is covered by L lanes (VEC elements,
//    up to 16-byte loads); a 64-lane wavefront holds G = 64/L workers;
//  * short runs: each worker owns S runs at once.  It issues their weight-row
//    loads up front, then walks their contributions as one flat sequence:
//    L sample ids at once, U gradient rows in flight across run boundaries,
//    so a run of one lookup costs one dependent step, not one each;
//  * long runs: the same launch carries chunk workers (a block per chunk of
//    `chunk` lookups, or a wavefront for rows of 64 lanes) that write partial
//    sums; the next launch (a block per long run) adds each run's partials in
//    a fixed order and applies the update, so the result does not depend on
//    scheduling.  (Combining in the same launch, last arrival wins, needs a
//    device-scope release per chunk, which on gfx950 writes back and
//    invalidates the whole L2 -- far dearer than one more launch);
//  * weight rows are read and written with streaming (non-temporal) hints;
//  * accumulation is fp64 for fp32 tables (long Zipf runs would otherwise
//    drift past 1e-5 relative) and fp32 for fp16 tables; w - lr*g is rounded
//    once to the storage type;
//  * row-wise Adagrad (same section: one state value per row, raised by the
//    row's mean squared gradient, step lr / (sqrt(state) + eps)): the row's
//    sum of squares is reduced across the worker's lanes with lane swaps, so
//    a row must fit one worker (D <= 64 * VEC); one lane stores the state;
//  * work counts are read from device memory; grids are persistent loops.
#include "tbe_internal.h"

namespace tbe {
namespace {

template <typename T, int N>
struct alignas(sizeof(T) * N) Pack {
    T v[N];
};

// Load through a global-address-space pointer: the pointers here come out of
// a by-value argument struct, where the compiler would otherwise emit flat
// loads (which also count against the LDS counter).
template <typename T>
__device__ __forceinline__ T ldg(const T* p)
{
#if __HIP_DEVICE_COMPILE__
    return *(const __attribute__((address_space(1))) T*)(p);
#else
    return *p;   // host pass: never executed
#endif
}

// Streaming (non-temporal) load and store of a weight row, global address
// space.  A row is read once and written once per call: with the streaming
// hint the rows neither displace the output-gradient slab that every worker
// re-reads nor leave a backlog of dirty lines in the caches for the next
// kernel to write back (measured on the uniform step: segment kernel 84 -> 71
// us, and the forward that follows it 48 -> 38 us).  P is a Pack of 2, 4, 8
// or 16 bytes.
template <int BYTES>
struct RawVec;
template <> struct RawVec<16> { typedef uint32_t T __attribute__((ext_vector_type(4))); };
template <> struct RawVec<8> { typedef uint32_t T __attribute__((ext_vector_type(2))); };
template <> struct RawVec<4> { typedef uint32_t T; };
template <> struct RawVec<2> { typedef uint16_t T; };

template <typename P>
__device__ __forceinline__ P ldg_stream(const P* p)
{
#if __HIP_DEVICE_COMPILE__
    typedef typename RawVec<sizeof(P)>::T R;
    const R x = __builtin_nontemporal_load((const __attribute__((address_space(1))) R*)p);
    P r;
    __builtin_memcpy(&r, &x, sizeof(P));
    return r;
#else
    return *p;   // host pass: never executed
#endif
}

template <typename P>
__device__ __forceinline__ void stg_stream(P* p, const P& v)
{
#if __HIP_DEVICE_COMPILE__
    typedef typename RawVec<sizeof(P)>::T R;
    R x;
    __builtin_memcpy(&x, &v, sizeof(P));
    __builtin_nontemporal_store(x, (__attribute__((address_space(1))) R*)p);
#else
    *p = v;
#endif
}

__device__ __forceinline__ int find_table(const uint32_t* __restrict__ hash_off, int T,
                                          uint32_t key)
{
    int lo = 0, hi = T;  // hash_off[lo] <= key < hash_off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (ldg(hash_off + mid) <= key) lo = mid; else hi = mid;
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
    const void* sorted_payload;   // sample ids, or (sample, weight) pairs when weighted
    const uint4* short_info;   // {key, start, len, table}
    const uint2* short_first;  // {sample, weight bits} of each short run's first lookup
    const uint4* long_info;    // {key, start, len, first chunk}
    const uint32_t* counts;    // runs, short, long, chunks
    uint32_t chunk;
    uint32_t max_chunks;
    uint32_t max_long;
    float lr;
    float eps;                 // row-wise Adagrad only
    int32_t all_weighted;      // mean pooling: every table's payload weight applies
    float* state;              // row-wise Adagrad: fp32 state per row, by key
    uint32_t chunk_blocks;     // the grid's last chunk_blocks blocks take long-run chunks
    const uint32_t* mode;      // payload the integer stage left in the workspace
    uint32_t expect_mode;      // ... and the payload this call was told to expect
    uint32_t* err;             // the workspace's error word
};

// The workspace must hold the payload this launch reads (sample ids, or
// (sample, weight) pairs): a caller of the apply half that names the wrong one
// would have sample ids read at the wrong stride.  On a mismatch the kernel
// does no work and sets the error word's payload bit.
__device__ __forceinline__ bool payload_mismatch(const SegArgs& c)
{
    if (ldg(c.mode) == c.expect_mode) return false;
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(c.err, kErrPayload);
    return true;
}

enum Opt : int { kSgd = 0, kAdagrad = 1 };

// w - lr*g in the accumulator type, rounded once to the storage type.
template <typename WT, typename ACC, int VEC>
__device__ __forceinline__ Pack<WT, VEC> sgd_row(const Pack<WT, VEC>& w_old,
                                                 const ACC (&acc)[VEC], float lr)
{
    Pack<WT, VEC> o;
#pragma unroll
    for (int k = 0; k < VEC; ++k)
        o.v[k] = static_cast<WT>(static_cast<ACC>(static_cast<float>(w_old.v[k])) -
                                 static_cast<ACC>(lr) * acc[k]);
    return o;
}

template <typename WT, typename ACC, int VEC>
__device__ __forceinline__ void sgd_store(WT* __restrict__ wp, const Pack<WT, VEC>& w_old,
                                          const ACC (&acc)[VEC], float lr)
{
    stg_stream(reinterpret_cast<Pack<WT, VEC>*>(wp), sgd_row<WT, ACC, VEC>(w_old, acc, lr));
}

// Row-wise Adagrad for a row held by L lanes (VEC elements each; lanes past
// the row's D hold zeros): the row's sum of squares by lane swaps inside the
// worker, new state = old + sum / D kept in fp32, then
// w - lr / (sqrt(state) + eps) * g with g and the subtraction in the
// accumulator type, rounded once to the storage type.  The state and the
// rate are fp32 whatever the accumulator (relative error ~1e-7; the fp64
// forms cost registers, and occupancy, in the common fp32-sum path too).
// Every lane of the worker must call it.
template <typename WT, typename ACC, int VEC>
__device__ __forceinline__ Pack<WT, VEC> adagrad_row(const Pack<WT, VEC>& w_old,
                                                     const ACC (&acc)[VEC], float s_old, int D,
                                                     int L, float lr, float eps, float& s_new)
{
    float sq = 0.f;
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
        const float g = static_cast<float>(acc[k]);
        sq = fmaf(g, g, sq);
    }
    for (int m = L >> 1; m > 0; m >>= 1) sq += __shfl_xor(sq, m);
    s_new = s_old + sq / static_cast<float>(D);
    const ACC rate = static_cast<ACC>(lr / (sqrtf(s_new) + eps));
    Pack<WT, VEC> o;
#pragma unroll
    for (int k = 0; k < VEC; ++k)
        o.v[k] = static_cast<WT>(static_cast<ACC>(static_cast<float>(w_old.v[k])) - rate * acc[k]);
    return o;
}

// Sum, for S runs held by one worker (L lanes), of w_i * grad[sample_i, col..]
// over each run's contributions, walked as one flat sequence: the worker's
// lanes load L sample ids (and per-sample weights) at once, then U gradient
// rows are kept in flight at a time, across run boundaries.  pos0/len give
// each run's first sorted position and length; gcol its gradient column base.
//
// INLINE: the first contribution of each run comes in (fsmp, fw) from the run
// record, so a batch of one-lookup runs needs no payload load at all.
template <typename ACC, int VEC, int S, int U, bool WEIGHTED, bool INLINE>
__device__ __forceinline__ void flat_sum(const SegArgs& c, const uint32_t (&pos0)[S],
                                         const uint32_t (&len)[S],
                                         const float* const (&gcol)[S], const bool (&tw)[S],
                                         const uint32_t (&fsmp)[S], const float (&fw)[S],
                                         int sub, int L, int gbase, ACC (&acc)[S][VEC])
{
    uint32_t pre[S + 1];
    pre[0] = 0;
#pragma unroll
    for (int u = 0; u < S; ++u) pre[u + 1] = pre[u] + len[u];
    const uint32_t C = pre[S];
    for (uint32_t cb = 0; cb < C; cb += L) {
        // lane `sub` fetches contribution cb + sub
        const uint32_t ci = cb + sub;
        uint32_t my_smp = 0;
        float my_w = 1.f;
        int sl = 0;
#pragma unroll
        for (int u = 1; u < S; ++u) sl += ci >= pre[u] ? 1 : 0;
        uint32_t p = pos0[0], first_smp = 0;
        float first_w = 1.f;
        bool w_on = false, is_first = false;
#pragma unroll
        for (int u = 0; u < S; ++u)
            if (u == sl) {
                p = pos0[u] + (ci - pre[u]);
                w_on = tw[u];
                is_first = ci == pre[u];
                first_smp = fsmp[u];
                first_w = fw[u];
            }
        const bool need = ci < C && !(INLINE && is_first);
        if (INLINE && ci < C && is_first) {
            my_smp = first_smp;
            if (w_on) my_w = first_w;
        }
        if (__ballot(need)) {   // one load per lane, unconditional within the wave
            const uint32_t pp = need ? p : pos0[0];
            if (WEIGHTED) {
                const uint2 pv = ldg(static_cast<const uint2*>(c.sorted_payload) + pp);
                if (need) {
                    my_smp = pv.x;
                    if (w_on) my_w = __uint_as_float(pv.y);
                }
            } else {
                const uint32_t sv = ldg(static_cast<const uint32_t*>(c.sorted_payload) + pp);
                if (need) my_smp = sv;
            }
        }
        const uint32_t n = min(static_cast<uint32_t>(L), C - cb);
        for (uint32_t j0 = 0; j0 < n; j0 += U) {
            // all U row loads are issued unconditionally (an idle slot reads
            // the first gradient row and is masked afterwards), so they are
            // in flight together
            Pack<float, VEC> g[U];
            float w[U];
            int sl[U];
            bool on[U];
#pragma unroll
            for (int q = 0; q < U; ++q) {
                const uint32_t j = j0 + q;
                const uint32_t smp = __shfl(my_smp, gbase + static_cast<int>(j & 63));
                w[q] = WEIGHTED ? __shfl(my_w, gbase + static_cast<int>(j & 63)) : 1.f;
                sl[q] = 0;
#pragma unroll
                for (int u = 1; u < S; ++u) sl[q] += (cb + j) >= pre[u] ? 1 : 0;
                const float* base = gcol[0];
#pragma unroll
                for (int u = 1; u < S; ++u) base = (sl[q] == u) ? gcol[u] : base;
                on[q] = j < n && base != nullptr;
                const float* src = on[q] ? base + static_cast<int64_t>(smp) * c.sumD : c.grad;
                g[q] = ldg(reinterpret_cast<const Pack<float, VEC>*>(src));
            }
#pragma unroll
            for (int q = 0; q < U; ++q)
#pragma unroll
                for (int u = 0; u < S; ++u)
                    if (on[q] && sl[q] == u)
#pragma unroll
                        for (int k = 0; k < VEC; ++k) {
                            if (WEIGHTED)   // w*g is exact in fp64; explicit fma in fp32
                                acc[u][k] = fma(static_cast<ACC>(w[q]),
                                                static_cast<ACC>(g[q].v[k]), acc[u][k]);
                            else
                                acc[u][k] += static_cast<ACC>(g[q].v[k]);
                        }
        }
    }
}

// One batch of S short runs per worker: prefetch the S weight rows, sum the
// runs' contributions, apply SGD.
// Table descriptor t: from the LDS copy when the block staged one, else from
// global memory.
template <bool LDSD>
__device__ __forceinline__ TableDesc table_desc(const SegArgs& c, const TableDesc* sdesc, int t)
{
    if (LDSD) return sdesc[t];
    return ldg(c.tables + t);
}

template <typename WT, typename ACC, int VEC, int S, int U, bool WEIGHTED, bool LDSD, int OPT>
__device__ __forceinline__ void short_batch(const SegArgs& c, WT* __restrict__ weights,
                                            const TableDesc* sdesc,
                                            const uint4 (&info)[S], const uint2 (&first)[S],
                                            int sub, int L, int gbase)
{
    uint32_t fsmp[S];
    float fw[S];
#pragma unroll
    for (int u = 0; u < S; ++u) {
        fsmp[u] = first[u].x;
        fw[u] = __uint_as_float(first[u].y);
    }
    for (int c0 = 0; c0 < c.max_D; c0 += VEC * L) {
        const int col = c0 + sub * VEC;
        Pack<WT, VEC> w_old[S];
        ACC acc[S][VEC];
        WT* wrow[S];
        const float* gcol[S];
        bool tw[S];
        uint32_t len[S], pos0[S];
        float s_old[S];
        int Dr[S];
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const TableDesc d = table_desc<LDSD>(c, sdesc, static_cast<int>(info[u].w));
            // a run whose table is narrower than this column slab contributes
            // nothing here (its lanes keep the loop shape but load no rows)
            const bool act = info[u].z > 0 && col < d.D;
            len[u] = info[u].z;
            pos0[u] = info[u].y;
            wrow[u] = weights + d.w_off + static_cast<int64_t>(info[u].x - d.hash_off) * d.D + col;
            gcol[u] = act ? c.grad + d.out_off + col : nullptr;
            tw[u] = WEIGHTED && (c.all_weighted || (d.flags & TD_WEIGHTED));
            // unconditional (an idle slot reads the first row of the weights)
            w_old[u] = ldg_stream(reinterpret_cast<const Pack<WT, VEC>*>(act ? wrow[u] : weights));
            Dr[u] = d.D;
            if (OPT == kAdagrad)   // every lane of the worker: the state feeds all of them
                s_old[u] = ldg(c.state + (info[u].z > 0 ? info[u].x : 0u));
#pragma unroll
            for (int q = 0; q < VEC; ++q) acc[u][q] = ACC(0);
        }
        flat_sum<ACC, VEC, S, U, WEIGHTED, true>(c, pos0, len, gcol, tw, fsmp, fw, sub, L, gbase,
                                                 acc);
        // all S updates first, then the stores (a wait for one row's old
        // value never includes another row's store)
        Pack<WT, VEC> o[S];
        float s_new[S];
#pragma unroll
        for (int u = 0; u < S; ++u) {
            if (OPT == kAdagrad)
                o[u] = adagrad_row<WT, ACC, VEC>(w_old[u], acc[u], s_old[u], Dr[u], L, c.lr,
                                                 c.eps, s_new[u]);
            else
                o[u] = sgd_row<WT, ACC, VEC>(w_old[u], acc[u], c.lr);
        }
#pragma unroll
        for (int u = 0; u < S; ++u) {
            if (gcol[u]) stg_stream(reinterpret_cast<Pack<WT, VEC>*>(wrow[u]), o[u]);
            if (OPT == kAdagrad && sub == 0 && info[u].z > 0) c.state[info[u].x] = s_new[u];
        }
    }
}

// Short runs.  Batches of G*S consecutive run records are dealt to the
// wavefronts round-robin (neighbouring runs of a Zipf table, which are the
// long ones, land on different wavefronts); a batch is read with one load
// (one record per lane, the next batch already in flight) and handed to the G
// workers S at a time through lane shuffles.  Runs shorter than kF32Run
// lookups sum in fp32 (error well inside tolerance); longer ones (only when
// tau is raised) and fp16 tables use the ACC type.
constexpr uint32_t kF32Run = 256;
// A wave loads a batch of G * S run records one per lane, so G = 64 / L must
// not exceed 64 / S: workers are at least 2^kMinLprLog2 lanes wide (S = 2),
// even where a row fits one lane (the second lane then idles).
constexpr int kMinLprLog2 = 1;

template <typename WT, typename ACC, int VEC, int S, int U, bool WEIGHTED, bool LDSD, int OPT>
__device__ __forceinline__ void short_runs(const SegArgs& c, WT* __restrict__ weights,
                                           const TableDesc* sdesc, uint32_t wave, uint32_t nwaves)
{
    const int lane = threadIdx.x & 63;
    const int g_log2 = 6 - c.lpr_log2;
    const int G = 1 << g_log2;
    const int L = 1 << c.lpr_log2;
    const int grp = lane >> c.lpr_log2;
    const int sub = lane & (L - 1);
    const int gbase = grp << c.lpr_log2;
    const uint32_t nshort = ldg(c.counts + 1);
    const uint32_t per = static_cast<uint32_t>(G * S);
    const uint32_t kend = nshort;
    uint32_t k0 = wave * per;
    uint4 nxt = make_uint4(0, 0, 0, 0);
    uint2 nxtf = make_uint2(0, 0);
    if (lane < static_cast<int>(per) && k0 + lane < kend) {
        nxt = ldg(c.short_info + k0 + lane);
        nxtf = ldg(c.short_first + k0 + lane);
    }
    for (; k0 < kend; k0 += nwaves * per) {
        const uint4 mine = nxt;
        const uint2 minef = nxtf;
        const uint32_t k1 = k0 + nwaves * per;
        nxt = make_uint4(0, 0, 0, 0);
        nxtf = make_uint2(0, 0);
        if (lane < static_cast<int>(per) && k1 + lane < kend) {
            nxt = ldg(c.short_info + k1 + lane);
            nxtf = ldg(c.short_first + k1 + lane);
        }
        uint4 info[S];
        uint2 first[S];
        uint32_t maxlen = 0;
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int src = u * G + grp;
            info[u].x = __shfl(mine.x, src);
            info[u].y = __shfl(mine.y, src);
            info[u].z = __shfl(mine.z, src);
            info[u].w = __shfl(mine.w, src);
            first[u].x = __shfl(minef.x, src);
            first[u].y = __shfl(minef.y, src);
            maxlen = max(maxlen, info[u].z);
        }
        if (sizeof(ACC) == 8 && maxlen < kF32Run)
            short_batch<WT, float, VEC, S, U, WEIGHTED, LDSD, OPT>(c, weights, sdesc, info, first,
                                                                   sub, L, gbase);
        else
            short_batch<WT, ACC, VEC, S, U, WEIGHTED, LDSD, OPT>(c, weights, sdesc, info, first,
                                                                 sub, L, gbase);
    }
}

// One wavefront per chunk (rows of L = 64 lanes): the wave keeps 8 gradient
// rows in flight over the whole chunk and writes its partial; the four waves
// of a block take four chunks.
template <typename ACC, int VEC, bool WEIGHTED>
__device__ __forceinline__ void long_chunks_wave(const SegArgs& c, ACC* __restrict__ partials,
                                                 uint32_t wave, uint32_t nwaves)
{
    const int lane = threadIdx.x & 63;
    const uint32_t nlong = min(ldg(c.counts + 2), c.max_long);
    const uint32_t nchunks = min(ldg(c.counts + 3), c.max_chunks);
    for (uint32_t q = wave; q < nchunks; q += nwaves) {
        uint32_t lo = 0, hi = nlong;  // long run owning chunk q: last with first chunk <= q
        while (hi - lo > 1) {
            const uint32_t mid = (lo + hi) >> 1;
            if (ldg(c.long_info + mid).w <= q) lo = mid; else hi = mid;
        }
        const uint4 li = ldg(c.long_info + lo);
        const TableDesc d = ldg(c.tables + find_table(c.hash_off, c.T, li.x));
        const bool tw = WEIGHTED && (c.all_weighted || (d.flags & TD_WEIGHTED));
        const uint32_t i0 = li.y + (q - li.w) * c.chunk;
        const uint32_t i1 = min(li.y + li.z, i0 + c.chunk);
        ACC* __restrict__ prow = partials + static_cast<int64_t>(q) * c.max_D;
        for (int c0 = 0; c0 < d.D; c0 += 64 * VEC) {
            const int col = c0 + lane * VEC;
            const uint32_t p0[1] = {i0};
            const uint32_t ln[1] = {i1 - i0};
            const float* const gc[1] = {col < d.D ? c.grad + d.out_off + col : nullptr};
            const bool twa[1] = {tw};
            ACC acc[1][VEC];
#pragma unroll
            for (int k = 0; k < VEC; ++k) acc[0][k] = ACC(0);
            const uint32_t nof[1] = {0};
            const float now[1] = {1.f};
            flat_sum<ACC, VEC, 1, 8, WEIGHTED, false>(c, p0, ln, gc, twa, nof, now, lane, 64, 0,
                                                      acc);
            if (col < d.D) {
                Pack<ACC, VEC> o;
#pragma unroll
                for (int k = 0; k < VEC; ++k) o.v[k] = acc[0][k];
                *reinterpret_cast<Pack<ACC, VEC>*>(prow + col) = o;
            }
        }
    }
}

// Long runs, step 1: one block per chunk of `chunk` lookups writes the
// chunk's partial sum (fp64 for fp32 tables) to the workspace.  The block's
// 256 / L slots of L lanes take consecutive sub-ranges of the chunk, each
// with 8 gradient rows in flight; the slots are folded in a fixed order (lane
// swaps inside a wave, then the four waves through LDS), so the partial does
// not depend on scheduling and a chunk's dependent chain is one slot's share
// of it rather than the whole chunk (stress workload: segment kernel 101 ->
// 89 us, band 94 -> 77 us).  Rows as wide as a wavefront (L = 64) take
// long_chunks_wave instead: there the block form measured slower (mixed
// workload 526 -> 552 us).
template <typename ACC, int VEC, bool WEIGHTED>
__device__ __forceinline__ void long_chunks_block(const SegArgs& c, ACC* __restrict__ partials,
                                                  Pack<ACC, VEC> (*red)[64], uint32_t blk,
                                                  uint32_t nblk)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lpr = c.lpr_log2;
    const int L = 1 << lpr;
    const int sub = lane & (L - 1);
    const int gbase = (lane >> lpr) << lpr;
    const uint32_t slot = static_cast<uint32_t>(tid >> lpr);
    const uint32_t nslots = 256u >> lpr;
    const uint32_t nlong = min(ldg(c.counts + 2), c.max_long);
    const uint32_t nchunks = min(ldg(c.counts + 3), c.max_chunks);
    for (uint32_t q = blk; q < nchunks; q += nblk) {
        uint32_t lo = 0, hi = nlong;  // long run owning chunk q: last with first chunk <= q
        while (hi - lo > 1) {
            const uint32_t mid = (lo + hi) >> 1;
            if (ldg(c.long_info + mid).w <= q) lo = mid; else hi = mid;
        }
        const uint4 li = ldg(c.long_info + lo);
        const TableDesc d = ldg(c.tables + find_table(c.hash_off, c.T, li.x));
        const bool tw = WEIGHTED && (c.all_weighted || (d.flags & TD_WEIGHTED));
        const uint32_t i0 = li.y + (q - li.w) * c.chunk;
        const uint32_t len = min(li.y + li.z, i0 + c.chunk) - i0;
        const uint32_t per = (len + nslots - 1) / nslots;   // this slot's share
        const uint32_t s0 = min(len, slot * per);
        const uint32_t s1 = min(len, s0 + per);
        ACC* __restrict__ prow = partials + static_cast<int64_t>(q) * c.max_D;
        for (int c0 = 0; c0 < d.D; c0 += (VEC << lpr)) {
            const int col = c0 + sub * VEC;
            const uint32_t p0[1] = {i0 + s0};
            const uint32_t ln[1] = {s1 - s0};
            const float* const gc[1] = {col < d.D ? c.grad + d.out_off + col : nullptr};
            const bool twa[1] = {tw};
            ACC acc[1][VEC];
#pragma unroll
            for (int k = 0; k < VEC; ++k) acc[0][k] = ACC(0);
            const uint32_t nof[1] = {0};
            const float now[1] = {1.f};
            flat_sum<ACC, VEC, 1, 8, WEIGHTED, false>(c, p0, ln, gc, twa, nof, now, sub, L,
                                                      gbase, acc);
            for (int m = 32; m >= L; m >>= 1)
#pragma unroll
                for (int k = 0; k < VEC; ++k) acc[0][k] += __shfl_xor(acc[0][k], m);
            if (lane < L) {
                Pack<ACC, VEC> o;
#pragma unroll
                for (int k = 0; k < VEC; ++k) o.v[k] = acc[0][k];
                red[wave][lane] = o;
            }
            __syncthreads();
            if (wave == 0 && lane < L && col < d.D) {
                Pack<ACC, VEC> o;
#pragma unroll
                for (int k = 0; k < VEC; ++k)
                    o.v[k] = ((red[0][lane].v[k] + red[1][lane].v[k]) + red[2][lane].v[k]) +
                             red[3][lane].v[k];
                *reinterpret_cast<Pack<ACC, VEC>*>(prow + col) = o;
            }
            __syncthreads();   // red is reused by the next slab or chunk
        }
    }
}

// Long runs, step 2 (next launch, so every partial is visible without a
// device-wide cache flush): one block per long run.  The block's 256 lanes
// form 256 / L chunk slots of L lanes (one row slab); slot s adds the run's
// chunks s, s + slots, s + 2 * slots, ... (4 loads in flight), then the slots
// are folded in a fixed order -- lane swaps inside a wave, then the four waves
// through LDS -- so the sum does not depend on scheduling, and wave 0 applies
// the update.  The longest run's combine is this launch's critical path; a
// block per run shortens it by the slot count (stress workload: 31 -> 11 us).
// Row-wise Adagrad: one slab per row, and lanes past the row's D keep zeros
// so the whole worker takes part in the sum of squares.
template <typename WT, typename ACC, int VEC, int OPT>
__global__ __launch_bounds__(256) void k_long_combine(SegArgs c, WT* __restrict__ weights,
                                                      const ACC* __restrict__ partials)
{
    __shared__ Pack<ACC, VEC> red[4][64];   // each wave's folded slab sum
    if (payload_mismatch(c)) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lpr = c.lpr_log2;
    const int L = 1 << lpr;
    const int sub = lane & (L - 1);
    const uint32_t slot = static_cast<uint32_t>(tid >> lpr);
    const uint32_t nslots = 256u >> lpr;
    const uint32_t nlong = min(ldg(c.counts + 2), c.max_long);
    for (uint32_t k = blockIdx.x; k < nlong; k += gridDim.x) {
        const uint4 li = ldg(c.long_info + k);
        const TableDesc d = ldg(c.tables + find_table(c.hash_off, c.T, li.x));
        WT* __restrict__ wrow = weights + d.w_off + static_cast<int64_t>(li.x - d.hash_off) * d.D;
        const uint32_t nq = (li.z + c.chunk - 1) / c.chunk;
        const uint32_t qend = min(li.w + nq, c.max_chunks);
        const int slab = VEC << lpr;
        const int nslab = OPT == kAdagrad ? 1 : (d.D + slab - 1) / slab;
        for (int sl = 0; sl < nslab; ++sl) {
            const int col = sl * slab + sub * VEC;
            const bool act = col < d.D;
            const int cc = act ? col : 0;
            Pack<WT, VEC> w_old;
            float s_old = 0.f;
            if (wave == 0) {   // the updating wave's row slab and state, early
                w_old = ldg_stream(reinterpret_cast<const Pack<WT, VEC>*>(wrow + cc));
                if (OPT == kAdagrad) s_old = ldg(c.state + li.x);
            }
            ACC acc[VEC];
#pragma unroll
            for (int j = 0; j < VEC; ++j) acc[j] = ACC(0);
            for (uint32_t q0 = li.w + slot; q0 < qend; q0 += 4 * nslots) {
                Pack<ACC, VEC> part[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {   // unconditional: past the end re-reads the last
                    const uint32_t qm = q0 + m * nslots;
                    const uint32_t qc = qm < qend ? qm : qend - 1;
                    part[m] = ldg(reinterpret_cast<const Pack<ACC, VEC>*>(
                        partials + static_cast<int64_t>(qc) * c.max_D + cc));
                }
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    if (act && q0 + m * nslots < qend)
#pragma unroll
                        for (int j = 0; j < VEC; ++j) acc[j] += part[m].v[j];
            }
            // fold the slots of a wave (lanes that differ only in the slot bits)
            for (int m = 32; m >= L; m >>= 1)
#pragma unroll
                for (int j = 0; j < VEC; ++j) acc[j] += __shfl_xor(acc[j], m);
            if (lane < L) {
                Pack<ACC, VEC> o;
#pragma unroll
                for (int j = 0; j < VEC; ++j) o.v[j] = acc[j];
                red[wave][lane] = o;
            }
            __syncthreads();
            if (wave == 0) {
                const int ln = lane & (L - 1);
#pragma unroll
                for (int j = 0; j < VEC; ++j)
                    acc[j] = ((red[0][ln].v[j] + red[1][ln].v[j]) + red[2][ln].v[j]) +
                             red[3][ln].v[j];
                if (OPT == kAdagrad) {   // every lane of the wave takes part in the swaps
                    float s_new;
                    const Pack<WT, VEC> o = adagrad_row<WT, ACC, VEC>(w_old, acc, s_old, d.D, L,
                                                                      c.lr, c.eps, s_new);
                    if (lane < L && act) stg_stream(reinterpret_cast<Pack<WT, VEC>*>(wrow + col), o);
                    if (lane == 0) c.state[li.x] = s_new;
                } else if (lane < L && act) {
                    sgd_store<WT, ACC, VEC>(wrow + col, w_old, acc, c.lr);
                }
            }
            __syncthreads();   // red is reused by the next slab or run
        }
    }
}

constexpr int kLdsTables = 256;   // table descriptors staged in LDS

// BLOCKCHUNK: long-run chunks take a block each (rows narrower than a
// wavefront) rather than a wavefront each; an instantiation of its own, since
// the block form's code measured slower in the other kernels (mixed workload
// 527 -> 558 us) even where it never runs.
template <typename WT, typename ACC, int VEC, int S, int U, bool WEIGHTED, int OPT,
          bool BLOCKCHUNK>
__global__ __launch_bounds__(256) void k_segment(SegArgs c, WT* __restrict__ weights,
                                                 ACC* __restrict__ partials)
{
    static_assert((S << (6 - kMinLprLog2)) <= 64, "a batch is loaded one record per lane");
    __shared__ TableDesc sdesc[kLdsTables];
    __shared__ Pack<ACC, VEC> red[BLOCKCHUNK ? 4 : 1][64];
    if (payload_mismatch(c)) return;
    const uint32_t wib = threadIdx.x >> 6;
    // blocks [0, gridDim.x - chunk_blocks) take short runs (dispatched first:
    // measured faster than chunks first), the rest long-run chunks
    const uint32_t short_blocks = gridDim.x - c.chunk_blocks;
    if (blockIdx.x < short_blocks) {
        const uint32_t wave = blockIdx.x * 4 + wib;
        const uint32_t nwaves = short_blocks * 4;
        if (c.T <= kLdsTables) {
            for (int i = threadIdx.x; i < c.T; i += 256) sdesc[i] = ldg(c.tables + i);
            __syncthreads();
            short_runs<WT, ACC, VEC, S, U, WEIGHTED, true, OPT>(c, weights, sdesc, wave, nwaves);
        } else {
            short_runs<WT, ACC, VEC, S, U, WEIGHTED, false, OPT>(c, weights, sdesc, wave, nwaves);
        }
    }
    else if constexpr (BLOCKCHUNK)
        long_chunks_block<ACC, VEC, WEIGHTED>(c, partials, red, blockIdx.x - short_blocks,
                                              c.chunk_blocks);
    else
        long_chunks_wave<ACC, VEC, WEIGHTED>(c, partials, (blockIdx.x - short_blocks) * 4 + wib,
                                             c.chunk_blocks * 4);
}

uint32_t blocks_for(int64_t work_items, int64_t per_block, int64_t cap)
{
    int64_t b = (work_items + per_block - 1) / per_block;
    if (b > cap) b = cap;
    if (b < 1) b = 1;
    return static_cast<uint32_t>(b);
}

template <typename WT, typename ACC, int VEC, int S, int U, int OPT, bool BLOCKCHUNK>
void launch_seg_c(const BwdArgs& a, dim3 grid, const SegArgs& c, WT* w, ACC* partials)
{
    if (a.payload_pairs)
        hipLaunchKernelGGL((k_segment<WT, ACC, VEC, S, U, true, OPT, BLOCKCHUNK>), grid,
                           dim3(256), 0, a.stream, c, w, partials);
    else
        hipLaunchKernelGGL((k_segment<WT, ACC, VEC, S, U, false, OPT, BLOCKCHUNK>), grid,
                           dim3(256), 0, a.stream, c, w, partials);
}

template <typename WT, typename ACC, int VEC, int S, int U, int OPT>
void launch_seg(const BwdArgs& a, dim3 grid, const SegArgs& c, WT* w, ACC* partials)
{
    if (c.lpr_log2 < 6)   // rows narrower than a wavefront: a block per chunk
        launch_seg_c<WT, ACC, VEC, S, U, OPT, true>(a, grid, c, w, partials);
    else
        launch_seg_c<WT, ACC, VEC, S, U, OPT, false>(a, grid, c, w, partials);
}

template <typename WT, typename ACC, int VEC, int OPT>
hipError_t launch_all(const BwdArgs& a, SegArgs c)
{
    const BwdLayout& L = a.L;
    char* ws = a.ws;
    ACC* partials = reinterpret_cast<ACC*>(ws + L.off_partials);
    WT* w = static_cast<WT*>(a.weights);
    const int G = 1 << (6 - c.lpr_log2);
    const uint32_t short_blocks = blocks_for(L.N, int64_t(4) * G * 2, 2048);  // G*S runs per wave batch
    // a block per chunk (rows narrower than a wave), else a wave per chunk
    c.chunk_blocks = c.lpr_log2 == 6 ? blocks_for(L.max_chunks, 4, 1024)
                                     : blocks_for(L.max_chunks, 1, 4096);
    // a block per long run (at most 4096: measured best of 1024..8192 on the
    // stress, band and mixed workloads)
    const uint32_t b_long = blocks_for(L.max_long, 1, 4096);
    const dim3 grid(short_blocks + c.chunk_blocks);
    // short-run batches: S = 2 runs per worker, U = 4 gradient rows in flight
    // (measured best of S in {1,2,4,8} x U in {4,8} on the uniform, stress and
    // mixed workloads)
    launch_seg<WT, ACC, VEC, 2, 4, OPT>(a, grid, c, w, partials);
    stage_mark(a.plan, 4, a.stream);
    hipLaunchKernelGGL((k_long_combine<WT, ACC, VEC, OPT>), dim3(b_long), dim3(256), 0, a.stream,
                       c, w, static_cast<const ACC*>(partials));
    stage_mark(a.plan, 5, a.stream);
    return hipGetLastError();
}

}  // namespace

namespace {
// Elements per lane of the segment kernels: the widest load every table's D,
// grad_output and the weights allow.
int segment_vec(const BwdArgs& a)
{
    const tbe_plan* p = a.plan;
    int vec = 4;
    for (int t = 0; t < p->T; ++t)
        while (p->dims[t] % vec) vec >>= 1;
    if (reinterpret_cast<uintptr_t>(a.grad) % (vec * 4)) vec = 1;
    const size_t wbytes = p->wdtype == TBE_F32 ? 4 : 2;
    while (vec > 1 && reinterpret_cast<uintptr_t>(a.weights) % (vec * wbytes)) vec >>= 1;
    return vec;
}

template <int OPT>
hipError_t dispatch_segment(const BwdArgs& a, const SegArgs& c, int vec)
{
    if (a.plan->wdtype == TBE_F32) {
        switch (vec) {
        case 4: return launch_all<float, double, 4, OPT>(a, c);
        case 2: return launch_all<float, double, 2, OPT>(a, c);
        default: return launch_all<float, double, 1, OPT>(a, c);
        }
    }
    switch (vec) {
    case 4: return launch_all<_Float16, float, 4, OPT>(a, c);
    case 2: return launch_all<_Float16, float, 2, OPT>(a, c);
    default: return launch_all<_Float16, float, 1, OPT>(a, c);
    }
}
}  // namespace

bool adagrad_supported(const BwdArgs& a)
{
    return (a.plan->max_D + segment_vec(a) - 1) / segment_vec(a) <= 64;
}

hipError_t run_segment_sgd(const BwdArgs& a)
{
    const tbe_plan* p = a.plan;
    const BwdLayout& L = a.L;
    if (L.N == 0) return hipSuccess;
    const int vec = segment_vec(a);
    const int lanes = (p->max_D + vec - 1) / vec;
    int lpr_log2 = kMinLprLog2;
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
    c.sorted_payload = ws + L.off_vals[a.final_buf];
    c.short_info = reinterpret_cast<const uint4*>(ws + L.off_short_info);
    c.short_first = reinterpret_cast<const uint2*>(ws + L.off_short_first);
    c.long_info = reinterpret_cast<const uint4*>(ws + L.off_long_info);
    c.counts = reinterpret_cast<const uint32_t*>(ws + L.off_ctl) + kCtlCounts;
    c.chunk = static_cast<uint32_t>(p->tuning.chunk);
    c.max_chunks = static_cast<uint32_t>(L.max_chunks);
    c.max_long = static_cast<uint32_t>(L.max_long);
    c.lr = a.lr;
    c.eps = a.eps;
    c.state = a.state;
    c.all_weighted = p->pooling == TBE_POOL_MEAN ? 1 : 0;
    c.chunk_blocks = 0;
    c.mode = reinterpret_cast<const uint32_t*>(ws + L.off_ctl) + kCtlMode;
    c.expect_mode = a.payload_pairs ? kModePairs : kModeSample;
    c.err = reinterpret_cast<uint32_t*>(ws + L.off_ctl) + kCtlError;
    if (a.state) return dispatch_segment<kAdagrad>(a, c, vec);
    return dispatch_segment<kSgd>(a, c, vec);
}

}  // namespace tbe
