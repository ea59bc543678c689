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
//  * work is cut into items, one column block of one table (cw columns, so
//    the table's grad_output slab B x cw x 4 bytes stays in one XCD's L2),
//    dealt to the eight XCDs in a fixed order; one persistent launch, whose
//    waves walk their XCD's items (see k_segment below);
//  * a column block of a gradient row is covered by L lanes (VEC elements,
//    up to 16-byte loads); a 64-lane wavefront holds G = 64/L workers;
//  * short runs: each worker owns S runs at once.  It issues their weight-row
//    loads up front, then walks their contributions as one flat sequence:
//    L sample ids at once, U gradient rows in flight across run boundaries,
//    so a run of one lookup costs one dependent step, not one each.  The
//    next unit's run records and sample ids are fetched while the current
//    unit is summed, and its updated rows are stored after those loads;
//  * long runs: an item's units also include its long runs' chunks (`chunk`
//    lookups each; a wave's workers split a chunk and are folded in a fixed
//    order) whose partial sums go to the workspace; the next launch (a block
//    per long run) adds each run's partials in a fixed order and applies the
//    update, so the result does not depend on scheduling.  (Combining in the
//    same launch, last arrival wins, needs a device-scope release per chunk,
//    which on gfx950 writes back and invalidates the whole L2 -- far dearer
//    than one more launch);
//  * weight rows are read and written with streaming (non-temporal) hints;
//  * accumulation is fp64 for fp32 tables (long Zipf runs would otherwise
//    drift past 1e-5 relative) and fp32 for fp16 tables; w - lr*g is rounded
//    once to the storage type;
//  * row-wise Adagrad (same section: one state value per row, raised by the
//    row's mean squared gradient, step lr / (sqrt(state) + eps)): the row's
//    sum of squares is reduced across the worker's lanes with lane swaps, so
//    a row must fit one worker (D <= 64 * VEC); one lane stores the state;
//  * work counts and per-table run ranges are read from device memory (the
//    run-length encode writes them); nothing goes back to the host.
#include "tbe_internal.h"

namespace tbe {
namespace {

template <typename T, int N>
struct alignas(sizeof(T) * N) Pack {
    T v[N];
};

template <int BYTES>
struct RawVec;
template <> struct RawVec<32> { typedef uint32_t T __attribute__((ext_vector_type(8))); };
template <> struct RawVec<16> { typedef uint32_t T __attribute__((ext_vector_type(4))); };
template <> struct RawVec<8> { typedef uint32_t T __attribute__((ext_vector_type(2))); };
template <> struct RawVec<4> { typedef uint32_t T; };
template <> struct RawVec<2> { typedef uint16_t T; };

// Load through a global-address-space pointer: the pointers here come out of
// a by-value argument struct, where the compiler would otherwise emit flat
// loads (which also count against the LDS counter, so every wait for an LDS
// or lane-shuffle result would also wait for them).  A struct (a Pack, a
// HIP vector type) is loaded as a plain vector and copied: a struct copied
// straight out of the cast pointer is rewritten into element loads through
// the original, generic pointer, and so compiles to flat loads again.
template <typename T>
__device__ __forceinline__ T ldg(const T* p)
{
#if __HIP_DEVICE_COMPILE__
    if constexpr (__is_class(T)) {
        typedef typename RawVec<sizeof(T)>::T R;
        const R x = *(const __attribute__((address_space(1))) R*)(p);
        T r;
        __builtin_memcpy(&r, &x, sizeof(T));
        return r;
    } else {
        return *(const __attribute__((address_space(1))) T*)(p);
    }
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
    int32_t lpr_log2;      // lanes per row slab of the combine (log2; from the widest row)
    int32_t wl_log2;       // lanes per worker of the segment kernel (log2)
    int32_t cw;            // columns per item (column block width)
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
    const uint32_t* tab_ranges;   // [3][T+1]: first short run, long run, chunk of each table
    const uint2* chunk_info;      // {first sorted position, length} of each chunk
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
    // lane `sub` fetches the sample id (and weight) of contribution cb + sub;
    // the next group's are fetched while the current group's rows are summed
    auto fetch = [&](uint32_t cb, uint32_t& my_smp, float& my_w) {
        const uint32_t ci = cb + sub;
        my_smp = 0;
        my_w = 1.f;
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
    };
    uint32_t nsmp;
    float nw;
    fetch(0, nsmp, nw);
    for (uint32_t cb = 0; cb < C; cb += L) {
        const uint32_t my_smp = nsmp;
        const float my_w = nw;
        if (cb + L < C) fetch(cb + L, nsmp, nw);
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

// Short runs are summed in fp32 below kF32Run lookups (error well inside
// tolerance); longer ones (only when tau is raised) and fp16 tables use the
// ACC type.
constexpr uint32_t kF32Run = 256;
// A wave loads a unit of G * S run records one per lane, so G = 64 / L must
// not exceed 64 / S: workers are at least 2^kMinLprLog2 lanes wide (S = 2),
// even where a row fits one lane (the second lane then idles).
constexpr int kMinLprLog2 = 1;
constexpr int kLdsTables = 256;   // table descriptors and item offsets staged in LDS
constexpr int kCombineLdsHash = 2048;   // the combine's table search in LDS up to this many tables

// A wave-uniform value kept in a scalar register (values read from LDS land in
// vector registers, one copy per lane).
__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ TableDesc uniform_desc(const TableDesc& d)
{
    TableDesc r;
    uint32_t w[8];
    __builtin_memcpy(w, &d, sizeof(TableDesc));
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = uni(w[k]);
    __builtin_memcpy(&r, w, sizeof(TableDesc));
    return r;
}

// One unit of short runs: up to G*S consecutive short runs of one table (one
// record per lane), S per worker, for one column block of the table.  Each
// worker prefetches its S weight rows, walks the runs' contributions as one
// flat sequence (U gradient rows in flight), then applies the update; all S
// updates are computed before the stores (a wait for one row's old value
// never includes another row's store).
// The unit's run records, one per lane (zero past the unit's end).
__device__ __forceinline__ void unit_records(const SegArgs& c, uint32_t k0, uint32_t n, int lane,
                                             uint4& rec, uint2& first)
{
    rec = make_uint4(0, 0, 0, 0);
    first = make_uint2(0, 0);
    if (lane < static_cast<int>(n)) {
        rec = ldg(c.short_info + k0 + lane);
        first = ldg(c.short_first + k0 + lane);
    }
}

// Updated rows of a short unit, stored during the next unit: the vector memory
// counter is one in-order counter for loads and stores, so stores issued
// before a unit's first loads would make every wait for those loads wait for
// the stores too; issued after them, they complete while the loads are in
// flight.
template <typename WT, int VEC, int S, int OPT>
struct PendingRows {
    Pack<WT, VEC> o[S];
    WT* wrow[S];
    float s_new[S];
    uint32_t skey[S];
    uint32_t on = 0;    // bit u: row u is to be stored
    uint32_t son = 0;   // bit u: state u is to be stored (row-wise Adagrad)

    __device__ __forceinline__ void flush(float* state)
    {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            if (on & (1u << u)) stg_stream(reinterpret_cast<Pack<WT, VEC>*>(wrow[u]), o[u]);
            if (OPT == kAdagrad && (son & (1u << u))) state[skey[u]] = s_new[u];
        }
        on = son = 0;
    }
};

template <typename WT, typename ACC, int VEC, int S, int U, bool WEIGHTED, int OPT>
__device__ __forceinline__ void short_unit(const SegArgs& c, WT* __restrict__ weights,
                                           const TableDesc& d, const uint4& mine,
                                           const uint2& minef, int col, int sub, int L, int G,
                                           int grp, int gbase, PendingRows<WT, VEC, S, OPT>& pend)
{
    const bool tw = WEIGHTED && (c.all_weighted || (d.flags & TD_WEIGHTED));
    const bool act_col = col < d.D;
    uint32_t len[S], pos0[S], fsmp[S], key[S];
    float fw[S];
    bool twa[S];
    uint32_t maxlen = 0;
#pragma unroll
    for (int u = 0; u < S; ++u) {
        const int src = u * G + grp;
        key[u] = __shfl(mine.x, src);
        pos0[u] = __shfl(mine.y, src);
        len[u] = __shfl(mine.z, src);
        fsmp[u] = __shfl(minef.x, src);
        fw[u] = __uint_as_float(__shfl(minef.y, src));
        twa[u] = tw;
        maxlen = max(maxlen, len[u]);
    }
    auto body = [&](auto acc_tag) {
        using A = decltype(acc_tag);
        Pack<WT, VEC> w_old[S];
        A acc[S][VEC];
        WT* wrow[S];
        const float* gcol[S];
        float s_old[S];
#pragma unroll
        for (int u = 0; u < S; ++u) {
            // a slot without a run (len 0) or a lane past the row keeps the
            // loop shape but loads no gradient rows
            const bool act = len[u] > 0 && act_col;
            wrow[u] = weights + d.w_off + static_cast<int64_t>(key[u] - d.hash_off) * d.D + col;
            gcol[u] = act ? c.grad + d.out_off + col : nullptr;
            // unconditional (an idle slot reads the first row of the weights)
            w_old[u] = ldg_stream(reinterpret_cast<const Pack<WT, VEC>*>(act ? wrow[u] : weights));
            if (OPT == kAdagrad)   // every lane of the worker: the state feeds all of them
                s_old[u] = ldg(c.state + (len[u] > 0 ? key[u] : 0u));
#pragma unroll
            for (int q = 0; q < VEC; ++q) acc[u][q] = A(0);
        }
        pend.flush(c.state);   // the previous unit's rows, now that this unit's loads are out
        flat_sum<A, VEC, S, U, WEIGHTED, true>(c, pos0, len, gcol, twa, fsmp, fw, sub, L, gbase,
                                               acc);
#pragma unroll
        for (int u = 0; u < S; ++u) {
            if (OPT == kAdagrad)
                pend.o[u] = adagrad_row<WT, A, VEC>(w_old[u], acc[u], s_old[u], d.D, L, c.lr,
                                                    c.eps, pend.s_new[u]);
            else
                pend.o[u] = sgd_row<WT, A, VEC>(w_old[u], acc[u], c.lr);
            pend.wrow[u] = wrow[u];
            if (gcol[u]) pend.on |= 1u << u;
            if (OPT == kAdagrad) {
                pend.skey[u] = key[u];
                if (sub == 0 && len[u] > 0) pend.son |= 1u << u;
            }
        }
    };
    if (sizeof(ACC) == 8 && maxlen < kF32Run)
        body(float(0));
    else
        body(ACC(0));
}

// One long-run chunk (`chunk` consecutive lookups of one long run) for one
// column block: the wave's G workers take consecutive shares of it, each
// with 8 gradient rows in flight, and are folded in a fixed order (lane
// swaps), so the partial does not depend on scheduling; worker 0 writes the
// chunk's partial (fp64 for fp32 tables) to the workspace.
template <typename ACC, int VEC, bool WEIGHTED>
__device__ __forceinline__ void chunk_unit(const SegArgs& c, ACC* __restrict__ partials,
                                           const TableDesc& d, uint32_t q, int col, int lane,
                                           int sub, int L, int G, int grp, int gbase)
{
    const uint2 ci = ldg(c.chunk_info + q);
    const bool tw = WEIGHTED && (c.all_weighted || (d.flags & TD_WEIGHTED));
    const uint32_t i0 = ci.x;
    const uint32_t len = ci.y;
    const uint32_t per = (len + G - 1) / G;   // this worker's share
    const uint32_t s0 = min(len, static_cast<uint32_t>(grp) * per);
    const uint32_t s1 = min(len, s0 + per);
    const uint32_t p0[1] = {i0 + s0};
    const uint32_t ln[1] = {s1 - s0};
    const float* const gc[1] = {col < d.D ? c.grad + d.out_off + col : nullptr};
    const bool twa[1] = {tw};
    ACC acc[1][VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[0][k] = ACC(0);
    const uint32_t nof[1] = {0};
    const float now[1] = {1.f};
    flat_sum<ACC, VEC, 1, 8, WEIGHTED, false>(c, p0, ln, gc, twa, nof, now, sub, L, gbase, acc);
    for (int m = 32; m >= L; m >>= 1)
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc[0][k] += __shfl_xor(acc[0][k], m);
    if (grp == 0 && col < d.D) {
        Pack<ACC, VEC> o;
#pragma unroll
        for (int k = 0; k < VEC; ++k) o.v[k] = acc[0][k];
        *reinterpret_cast<Pack<ACC, VEC>*>(partials + static_cast<int64_t>(q) * c.max_D + col) = o;
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
    __shared__ uint32_t shash[kCombineLdsHash + 1];   // tables' first keys, when few enough
    if (payload_mismatch(c)) return;
    const int tid = threadIdx.x;
    // a run's table is found by a search over the tables' first keys: in LDS
    // (one load round per block) rather than a chain of dependent loads
    const bool lds_hash = c.T <= kCombineLdsHash;
    if (lds_hash) {
        for (int i = tid; i <= c.T; i += 256) shash[i] = ldg(c.hash_off + i);
        __syncthreads();
    }
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
        int t;
        if (lds_hash) {
            int lo = 0, hi = c.T;   // shash[lo] <= key < shash[hi]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (shash[mid] <= li.x) lo = mid; else hi = mid;
            }
            t = lo;
        } else {
            t = find_table(c.hash_off, c.T, li.x);
        }
        const TableDesc d = ldg(c.tables + t);
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

// Segment reduce + update, one persistent launch.  Work is cut into items, a
// table's column block (cw columns: the table's grad_output slab is then
// B x cw x 4 bytes, sized to stay in one XCD's L2), and an item's units are
// its long-run chunks and its short-run units.  Blocks are dealt to the eight
// XCDs round-robin (block b runs on XCD b mod 8), so XCD x takes items x,
// x + 8, ... and its waves split each item's units round-robin; an XCD's L2
// then holds the slabs of the one or two items its waves are on, rather than
// the slabs of every table the chip is working on.  Column blocks of equal
// width make items of one workload cost about the same, which keeps the XCDs
// even; with fewer than 16 items each is dealt as several slices (slice s
// of n takes the item's units u = s mod n, so every slice gets its share of
// the dearer chunks), so no XCD idles.  (A shared cursor handing units out
// one atomic at a time measured about nine times slower: atomics on one
// address complete one after another.)
template <typename WT, typename ACC, int VEC, int S, int U, bool WEIGHTED, int OPT>
__global__ __launch_bounds__(256, sizeof(ACC) == 4 ? 5 : 1) void k_segment(
    SegArgs c, WT* __restrict__ weights, ACC* __restrict__ partials)
{
    static_assert((S << (6 - kMinLprLog2)) <= 64, "a unit is loaded one record per lane");
    __shared__ TableDesc sdesc[kLdsTables];
    __shared__ uint32_t sitem[kLdsTables + 1];   // first item of each table
    if (payload_mismatch(c)) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const bool lds = c.T <= kLdsTables;
    const int L = 1 << c.wl_log2;
    const int G = 64 >> c.wl_log2;
    const int grp = lane >> c.wl_log2;
    const int sub = lane & (L - 1);
    const int gbase = grp << c.wl_log2;
    if (lds) {
        for (int i = tid; i < c.T; i += 256) sdesc[i] = ldg(c.tables + i);
        __syncthreads();
        if (tid < 64) {   // items per table: its column blocks
            uint32_t run = 0;
            for (int b0 = 0; b0 < c.T; b0 += 64) {
                const int t = b0 + lane;
                const uint32_t nb = t < c.T ? static_cast<uint32_t>((sdesc[t].D + c.cw - 1) / c.cw)
                                            : 0u;
                uint32_t inc = nb;
#pragma unroll
                for (int dd = 1; dd < 64; dd <<= 1) {
                    const uint32_t o = __shfl_up(inc, dd);
                    if (lane >= dd) inc += o;
                }
                if (t < c.T) sitem[t] = run + inc - nb;
                run += __shfl(inc, 63);
            }
            if (lane == 0) sitem[c.T] = run;
        }
        __syncthreads();
    }
    // without the LDS staging (very many tables) an item is a whole table
    const uint32_t nitems = lds ? sitem[c.T] : static_cast<uint32_t>(c.T);
    const uint32_t nsplit = nitems >= 16 ? 1u : (16u + nitems - 1) / nitems;
    const uint32_t npieces = nitems * nsplit;
    const uint32_t T1 = static_cast<uint32_t>(c.T) + 1;
    const uint32_t xcd = blockIdx.x & 7u;
    const uint32_t wx = (blockIdx.x >> 3) * 4 + (tid >> 6);
    const uint32_t nwx = (gridDim.x >> 3) * 4;
    const uint32_t GS = static_cast<uint32_t>(G * S);
    PendingRows<WT, VEC, S, OPT> pend;
    for (uint32_t pc = xcd; pc < npieces; pc += 8) {
        const uint32_t it = pc / nsplit, sl = pc - it * nsplit;
        int t = static_cast<int>(it), cb = 0;
        if (lds) {   // last table whose first item is <= it
            int lo = 0, hi = c.T;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (sitem[mid] <= it) lo = mid; else hi = mid;
            }
            t = lo;
            cb = static_cast<int>(it - sitem[t]);
        }
        t = static_cast<int>(uni(static_cast<uint32_t>(t)));
        cb = static_cast<int>(uni(static_cast<uint32_t>(cb)));
        const TableDesc d = uniform_desc(lds ? sdesc[t] : ldg(c.tables + t));
        const int col = cb * c.cw + sub * VEC;
        const uint32_t fs0 = uni(ldg(c.tab_ranges + t)), fs1 = uni(ldg(c.tab_ranges + t + 1));
        const uint32_t fc0 = uni(ldg(c.tab_ranges + 2 * T1 + t));
        const uint32_t nch = uni(ldg(c.tab_ranges + 2 * T1 + t + 1)) - fc0;
        const uint32_t nu = nch + (fs1 - fs0 + GS - 1) / GS;   // chunks, then short units
        // the waves that take a piece's (dearer) chunks move with the piece
        const uint32_t rot = (pc >> 3) * 131u % nwx;
        const uint32_t step = nsplit * nwx;
        uint32_t u = sl + nsplit * ((wx + rot) % nwx);
        // a short unit's records are fetched one unit ahead
        uint4 nrec;
        uint2 nfirst;
        auto fetch = [&](uint32_t uu) {
            const uint32_t k0 = fs0 + (uu - nch) * GS;
            unit_records(c, k0, uu >= nch && uu < nu ? min(GS, fs1 - k0) : 0u, lane, nrec, nfirst);
        };
        fetch(u);
        for (; u < nu; u += step) {
            const uint4 rec = nrec;
            const uint2 first = nfirst;
            fetch(u + step);
            if (u < nch) {
                pend.flush(c.state);
                chunk_unit<ACC, VEC, WEIGHTED>(c, partials, d, fc0 + u, col, lane, sub, L, G, grp,
                                               gbase);
            } else {
                short_unit<WT, ACC, VEC, S, U, WEIGHTED, OPT>(c, weights, d, rec, first, col, sub,
                                                              L, G, grp, gbase, pend);
            }
        }
    }
    pend.flush(c.state);
}

uint32_t blocks_for(int64_t work_items, int64_t per_block, int64_t cap)
{
    int64_t b = (work_items + per_block - 1) / per_block;
    if (b > cap) b = cap;
    if (b < 1) b = 1;
    return static_cast<uint32_t>(b);
}

// Persistent blocks of a 256-thread kernel on the whole device (all XCDs): as
// many as are resident, at most max_per_cu per CU, a multiple of 8 so every
// XCD gets the same number.  The occupancy query is cached per kernel (the
// devices a process uses are alike).
template <auto Kernel>
uint32_t persistent_blocks(int max_per_cu)
{
    static int cus = 0, per = 0;
    if (!per) {
        int dev = 0, c = 0, r = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&r, Kernel, 256, 0) != hipSuccess ||
            c <= 0 || r <= 0)
            return 2048;
        cus = c;
        per = r;
    }
    const int b = cus * (per < max_per_cu ? per : max_per_cu);
    return static_cast<uint32_t>(((b + 7) / 8) * 8);
}

// Blocks per CU when a column block's grad_output slab (B x cw x 4 bytes) is
// larger than an XCD's 4 MB L2, so the waves' gradient reads miss whatever
// their number: then fewer waves are faster.  Measured on the production-scale
// workload (33.5 MB slabs; segment kernel, ms, by waves per SIMD): 6: 6.40,
// 5: 5.93, 4: 5.60-5.67, 3: 5.50, 2: 5.68.  Slabs that fit keep every resident
// wave (the small-table workload's 4 MB slabs: 6: 88 us, 5: 92, 4: 97).
constexpr int kBigSlabBlocksPerCu = 3;
constexpr int64_t kXcdL2Bytes = int64_t(4) << 20;

template <typename WT, typename ACC, int VEC, int OPT>
hipError_t launch_all(const BwdArgs& a, SegArgs c)
{
    const BwdLayout& L = a.L;
    char* ws = a.ws;
    ACC* partials = reinterpret_cast<ACC*>(ws + L.off_partials);
    WT* w = static_cast<WT*>(a.weights);
    // a block per long run (at most 4096: measured best of 1024..8192 on the
    // stress, band and mixed workloads)
    const uint32_t b_long = blocks_for(L.max_long, 1, 4096);
    // short-run units: S = 2 runs per worker, U = 4 gradient rows in flight
    constexpr int S = 2, U = 4;
    const int max_per_cu =
        int64_t(a.B) * c.cw * 4 > kXcdL2Bytes ? kBigSlabBlocksPerCu : 1 << 30;
    if (a.payload_pairs) {
        constexpr auto k = k_segment<WT, ACC, VEC, S, U, true, OPT>;
        hipLaunchKernelGGL(k, dim3(persistent_blocks<k>(max_per_cu)), dim3(256), 0, a.stream, c,
                           w, partials);
    } else {
        constexpr auto k = k_segment<WT, ACC, VEC, S, U, false, OPT>;
        hipLaunchKernelGGL(k, dim3(persistent_blocks<k>(max_per_cu)), dim3(256), 0, a.stream, c,
                           w, partials);
    }
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
    // Worker width: a column block of cw = vec * 2^wl columns makes a
    // table's grad_output slab B * cw * 4 bytes; the widest block within the
    // tuning's slab target, but workers of at least 16 lanes (narrower ones
    // measured slower: each block re-reads its runs' records and payload),
    // whole rows when the update needs them (row-wise Adagrad) or the tables
    // are too many to stage.
    int wl_log2 = lpr_log2;
    const int64_t slab = int64_t(p->tuning.seg_slab_kib) * 1024;
    if (!a.state && slab > 0 && p->T <= kLdsTables) {
        while (wl_log2 > 4 && int64_t(a.B) * (int64_t(vec) << wl_log2) * 4 > slab) --wl_log2;
    }

    char* ws = a.ws;
    SegArgs c;
    c.tables = p->d_tables;
    c.hash_off = p->d_hash_off;
    c.T = p->T;
    c.sumD = p->sum_D;
    c.lpr_log2 = lpr_log2;
    c.wl_log2 = wl_log2;
    c.cw = vec << wl_log2;
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
    c.tab_ranges = reinterpret_cast<const uint32_t*>(ws + L.off_tab_ranges);
    c.chunk_info = reinterpret_cast<const uint2*>(ws + L.off_chunk_info);
    c.mode = reinterpret_cast<const uint32_t*>(ws + L.off_ctl) + kCtlMode;
    c.expect_mode = a.payload_pairs ? kModePairs : kModeSample;
    c.err = reinterpret_cast<uint32_t*>(ws + L.off_ctl) + kCtlError;
    if (a.state) return dispatch_segment<kAdagrad>(a, c, vec);
    return dispatch_segment<kSgd>(a, c, vec);
}

}  // namespace tbe
