// Backward integer stage for gfx950: linearize, stable LSD radix sort,
// run-length encode, classify runs by length.
//
// Section "Why the backward is the hard half" of the FBTriton TBE article:
// the backward inverts the batch -- every lookup gets the key
// hash_size_cumsum[t] + row (rows of different tables never collide), the
// keys are sorted so that every row's contributors sit next to each other,
// and a run-length encode turns each row into one independent unit of work.
// Section "Three tiers, routed by run length": runs are classified against a
// length threshold on the device, and the counts never go back to the host.
// Section "Using it, and the import that stops you": per-sample weights must
// stay paired with their lookup, so the sort is stable and carries the
// lookup's sample id and per-sample weight as its payload -- nothing is ever
// sorted twice and no weight is looked up again by position.
//
// Kernels (caller's stream, no host synchronisation).  A batch's lookups come
// table by table and keys of different tables never collide, so by default
// each table's segment of lookup positions is sorted on its own, on row bits
// only (the widest table's), with look-back chains inside one table; with
// very many tables, or few tiles per table, one sort runs over all keys.
//   k_seg_setup (per table) lays out radix tiles inside the tables' segments
//               and zeroes the per-table digit counts
//   k_count     (per table) digit counts of every radix pass from the ids
//               alone, and the bag holding each tile's first position
//   k_prep      (one sort) per block of bags: key[j] and its payload (j itself
//               for the sort_rle entry point; the bag's sample id, plus the
//               per-sample weight or 1/L when there is one, for the
//               backward), digit histograms of every radix pass (equal digits
//               of a wavefront merged by ballots, then LDS, then one global
//               add per digit), and clears the look-back words
//   k_onesweep  one launch per radix pass (digits of up to 9 bits over the
//               key bits that need sorting): a tile takes a ticket in launch
//               order, ranks its keys stably (wave ballots find equal digits,
//               per-wave LDS counters order them), looks back over earlier
//               tiles' published digit counts for its offsets, and scatters
//               key + payload.  The first pass of a per-table sort reads the
//               ids and weights itself and finds each position's bag (the
//               payload k_prep would have written)
//   k_rle       one launch: run heads, lengths (galloping search), the short /
//               long split and the long-run chunk counts; tile offsets come
//               from the same look-back, so the run lists stay in key order
//
// Look-back waits are bounded: a tile that waits more than ~2^24 polls for a
// predecessor raises an error flag and goes on, so a kernel always ends.
// Tile tickets, digit totals and the error word live in the workspace's control
// block, which is zero when a call starts and zero again when it ends.
#include "tbe_internal.h"

namespace tbe {

namespace {
constexpr int kRadix = 256;
// Digits are at most this wide: keys of 25-27 bits take three 9-bit passes
// instead of four of 7 or fewer, and 17-18 bits two instead of three.
constexpr int kMaxDigitBits = 9;
static_assert((1 << kMaxDigitBits) <= kRadixMax, "digit totals hold the widest digit");
constexpr int kSortThreads = 1024;   // 16 waves per radix tile
constexpr int kRleThreads = 1024;
constexpr int kRleItems = 8;         // sorted positions per thread (two 16-byte loads)
constexpr int kRleItemsSmall = 4;    // ... for small batches (see kSmallN)
constexpr int kRleMaxT = 2048;       // hash offsets staged in LDS up to this many tables
constexpr uint32_t kFlagAgg = 1u << 30;
constexpr uint32_t kFlagInc = 2u << 30;
constexpr uint32_t kValMask = (1u << 30) - 1u;
constexpr uint32_t kSpinLimit = 1u << 24;
constexpr int kPrepMaxBags = 2048;   // bags per k_prep block (LDS offsets cache)
constexpr int kPrepKeys = 1024;      // target keys per k_prep block
constexpr int kPrepThreads = 512;    // measured: 512 or 256 threads per block beat 1024

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int kSortRounds = 8;       // keys per thread in a radix tile
constexpr int kSortRoundsSmall = 4;  // ... for small batches (see kSmallN)
// Batches of at most kSmallN lookups use tiles of half the depth in the radix
// passes and the run-length encode: with a few tens of tiles every tile has a
// CU of its own, and shorter tiles finish sooner.  Beyond it the longer
// look-back chain over twice the tiles costs more.  Measured: uniform
// workload (328K lookups) radix 45 -> 43 us and encode 17 -> 14 us; stress
// (1.6M) and mixed (4.9M) slower with the short tiles.
constexpr int64_t kSmallN = int64_t(1) << 19;
constexpr int kSegMaxTables = 1024;  // segmented sort: tables laid out by one block
}  // namespace

BwdLayout bwd_layout(const tbe_plan* p, int32_t B, int64_t N)
{
    BwdLayout L;
    L.N = N;
    const bool small = N <= kSmallN;
    L.sort_tile = kSortThreads * (small ? kSortRoundsSmall : kSortRounds);
    const int64_t gtiles = (N + L.sort_tile - 1) / L.sort_tile;
    // Keys of different tables never collide and a batch's lookups come table
    // by table, so each table's segment of lookup positions can be sorted on
    // its own: on row bits only (the widest table's, not those of the sum of
    // all rows), with look-back chains that stay inside one table.  Taken
    // when tables are few against the tiles (each table then adds at most one
    // part-filled tile).
    const int sm = p->tuning.sort_mode;
    L.seg = p->T > 0 && N > 0 && p->T <= kSegMaxTables && sm != 1 &&
            (sm == 2 || 2 * int64_t(p->T) <= gtiles);
    int64_t key_range = p->sum_rows;
    if (L.seg) {
        key_range = 1;
        for (int t = 0; t < p->T; ++t) key_range = p->rows[t] > key_range ? p->rows[t] : key_range;
    }
    int bits = 0;
    while (bits < 32 && (uint64_t(1) << bits) < uint64_t(key_range)) ++bits;
    L.nbits = bits;
    L.npasses = bits == 0 ? 1 : (bits + kMaxDigitBits - 1) / kMaxDigitBits;
    const int per = bits == 0 ? 1 : (bits + L.npasses - 1) / L.npasses;
    int left = bits == 0 ? 1 : bits;
    for (int i = 0; i < L.npasses; ++i) {
        L.digit_bits[i] = per < left ? per : left;
        left -= L.digit_bits[i];
    }
    L.sort_blocks = static_cast<int32_t>(gtiles + (L.seg ? p->T : 0));
    L.rle_tile = kRleThreads * (small ? kRleItemsSmall : kRleItems);
    L.rle_blocks = static_cast<int32_t>((N + L.rle_tile - 1) / L.rle_tile);
    const int64_t total_bags = int64_t(p->T) * B;
    int64_t pb = (N + kPrepKeys - 1) / kPrepKeys;   // ~kPrepKeys keys per k_prep block
    if (pb > 1024) pb = 1024;
    const int64_t need = (total_bags + kPrepMaxBags - 1) / kPrepMaxBags;
    if (pb < need) pb = need;
    if (pb > total_bags) pb = total_bags;
    if (pb < 1) pb = 1;
    L.prep_blocks = static_cast<int32_t>(pb);
    L.prep_bags = static_cast<int32_t>((total_bags + pb - 1) / pb);
    if (L.seg) {   // blocks of one table each (its digit counts are the table's)
        int64_t bpb = L.prep_bags;
        if (bpb > B) bpb = B;
        if (bpb < 1) bpb = 1;
        L.prep_bags = static_cast<int32_t>(bpb);
        L.prep_bpt = static_cast<int32_t>((B + bpb - 1) / bpb);
        L.prep_blocks = L.prep_bpt * p->T;
        L.seg_copies = L.prep_bpt < kTotCopies ? L.prep_bpt : kTotCopies;
    }
    const int64_t tau = p->tuning.tau > 0 ? p->tuning.tau : 1;
    const int64_t C = p->tuning.chunk > 0 ? p->tuning.chunk : 1;
    int64_t mc = N / C + N / tau + 1;
    if (mc > N) mc = N;
    L.max_chunks = mc;
    int64_t ml = N / tau + 1;
    if (ml > N) ml = N;
    L.max_long = ml;

    const size_t n4 = align256(size_t(N + 1) * 4);
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t r = o; o += align256(bytes); return r; };
    L.off_ctl = take(size_t(kCtlWords) * 4);   // fixed at offset 0 for every layout
    L.off_keys[0] = take(n4);
    L.off_keys[1] = take(n4);
    L.off_vals[0] = take(2 * n4);   // payload: 4 bytes, or 8 with per-sample weights
    L.off_vals[1] = take(2 * n4);
    L.off_status = take(size_t(L.npasses) * kRadixMax * (L.sort_blocks > 0 ? L.sort_blocks : 1) * 4);
    L.off_rle_status = take(size_t(3) * (L.rle_blocks > 0 ? L.rle_blocks : 1) * 4);
    L.status_words = (L.off_rle_status - L.off_status) / 4 +
                     size_t(3) * (L.rle_blocks > 0 ? L.rle_blocks : 1);
    L.off_unique = take(n4);
    L.off_run_start = take(n4);
    L.off_run_len = take(n4);
    L.off_short = take(n4);
    L.off_long = take(n4);
    L.off_short_info = take(size_t(N + 1) * 16);
    L.off_short_first = take(size_t(N + 1) * 8);
    L.off_long_info = take(size_t(ml + 1) * 16);
    L.off_tab_ranges = take(size_t(3) * (p->T + 1) * 4);
    L.off_chunk_info = take(size_t(mc > 0 ? mc : 1) * 8);
    const size_t acc = p->wdtype == TBE_F32 ? 8 : 4;
    L.off_partials = take(size_t(mc > 0 ? mc : 1) * p->max_D * acc);
    if (L.seg) {
        L.off_tab_tot = take(size_t(p->T) * L.seg_copies * L.npasses * kRadixMax * 4);
        L.off_seg_tiles = take(size_t(L.sort_blocks) * 16);
        L.off_tile_bag = take(size_t(L.sort_blocks) * 4);
        L.off_seg_first = take(size_t(p->T + 1) * 4);
    }
    L.total = o;
    return L;
}

namespace {

// Load through a global-address-space pointer (a pointer cast from void*
// otherwise compiles to a flat load, which also counts against the LDS
// counter); a HIP vector type is loaded as a plain vector and copied.
template <typename T>
__device__ __forceinline__ T gload(const T* p)
{
#if __HIP_DEVICE_COMPILE__
    if constexpr (sizeof(T) == 8 && __is_class(T)) {
        typedef uint32_t V __attribute__((ext_vector_type(2)));
        const V x = *(const __attribute__((address_space(1))) V*)(p);
        T r;
        __builtin_memcpy(&r, &x, sizeof(T));
        return r;
    } else {
        static_assert(!__is_class(T), "scalars and 8-byte vector types only");
        return *(const __attribute__((address_space(1))) T*)(p);
    }
#else
    return *p;   // host pass: never executed
#endif
}

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

// Inclusive maximum over a wavefront's lanes in lane order (values >= 0),
// with data-parallel-primitive moves: shifts by 1, 2, 4, 8 inside each row of
// 16 lanes, then row 0's and row 2's last lanes into rows 1 and 3, then lane
// 31 into rows 2 and 3.  Lanes with no source lane take 0.
__device__ __forceinline__ uint32_t dpp_max(uint32_t v, uint32_t o) { return o > v ? o : v; }
__device__ __forceinline__ uint32_t wave_incl_max(uint32_t v)
{
    int x = static_cast<int>(v);
    x = static_cast<int>(dpp_max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false)));  // row_shr:1
    x = static_cast<int>(dpp_max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false)));  // row_shr:2
    x = static_cast<int>(dpp_max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false)));  // row_shr:4
    x = static_cast<int>(dpp_max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false)));  // row_shr:8
    x = static_cast<int>(dpp_max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false)));  // row_bcast:15
    x = static_cast<int>(dpp_max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false)));  // row_bcast:31
    return static_cast<uint32_t>(x);
}

__device__ __forceinline__ uint32_t ld_acq(const uint32_t* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_rel(uint32_t* p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive prefix of `value` over tiles 0..tile-1 through the status words
// st[0..tile) (one word per tile, stride `stride`).  Publishes this tile's
// aggregate first and its inclusive prefix last.  Predecessors are read W at a
// time (independent loads), so a chain of published aggregates is crossed W
// tiles per memory round trip.
template <int W>
__device__ __forceinline__ uint32_t lookback(uint32_t* st, uint32_t stride, uint32_t tile,
                                             uint32_t value, uint32_t* err)
{
    if (tile == 0) {
        st_rel(st, kFlagInc | value);
        return 0;
    }
    uint32_t excl = 0;
    int64_t tp = static_cast<int64_t>(tile) - 1;
    uint32_t spins = 0;
    uint32_t s[W];
    // the first window is read before this tile's aggregate is published: a
    // wait for the loads then does not include the store
#pragma unroll
    for (int i = 0; i < W; ++i)
        s[i] = (tp - i >= 0) ? ld_acq(st + static_cast<size_t>(tp - i) * stride) : kFlagInc;
    st_rel(st + static_cast<size_t>(tile) * stride, kFlagAgg | value);
    while (true) {
        uint32_t consumed = 0;
        bool stop = false, done = false;
#pragma unroll
        for (int i = 0; i < W; ++i) {
            if (!stop) {
                const uint32_t f = s[i] & ~kValMask;
                if (f == 0) {
                    stop = true;        // not published yet: fetch again from here
                } else {
                    excl += s[i] & kValMask;
                    ++consumed;
                    if (f == kFlagInc) stop = done = true;
                }
            }
        }
        if (done) break;
        tp -= consumed;
        if (consumed == 0) {
            if (++spins > kSpinLimit) {
                atomicOr(err, kErrLookback);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
#pragma unroll
        for (int i = 0; i < W; ++i)
            s[i] = (tp - i >= 0) ? ld_acq(st + static_cast<size_t>(tp - i) * stride) : kFlagInc;
    }
    st_rel(st + static_cast<size_t>(tile) * stride, kFlagInc | ((excl + value) & kValMask));
    return excl;
}

// Tile ticket in launch order.  The block that takes the last ticket resets
// the counter, so it is zero again for the next launch.
__device__ __forceinline__ uint32_t take_ticket(uint32_t* ticket, uint32_t ntiles)
{
    const uint32_t t = atomicAdd(ticket, 1u);
    if (t == ntiles - 1) st_rel(ticket, 0u);
    return t;
}

// ---------------------------------------------------------------------------
__global__ void k_fill_zero(uint32_t* __restrict__ p, int n)
{
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

struct PassBits {
    int32_t npasses;
    int32_t shift[4];
    int32_t bits[4];
    uint32_t mask[4];
};

// Payload carried through the sort next to each key.
enum PayloadMode : int {
    kPayloadPos = 0,      // lookup position j (the sort_rle entry point)
    kPayloadSample = 1,   // sample id b of the lookup's bag
    kPayloadSampleW = 2,  // (b, per-sample weight bits) pair
    kPayloadMean = 3,     // (b, weight / bag length) pair: mean pooling
};

// One block per run of whole bags (about kPrepKeys lookups), one lookup per
// thread per step: the bag of a lookup comes from a branchless binary search
// over the block's bag starts in LDS, so the searches of a thread's lookups
// interleave.  (One sort over every table's keys; the per-table sort counts
// with k_count and makes keys and payloads in its first radix pass.)
template <typename IT, int MODE>
__global__ __launch_bounds__(kPrepThreads) void k_prep(
    const TableDesc* __restrict__ tables, uint32_t B, uint32_t total_bags, uint32_t bags_per_block,
    const IT* __restrict__ indices, const IT* __restrict__ offsets,
    const float* __restrict__ psw, uint32_t* __restrict__ keys, void* __restrict__ vals,
    uint32_t* __restrict__ totals, PassBits pb, uint32_t* __restrict__ status,
    size_t status_words)
{
    __shared__ uint32_t hist[4][kRadixMax];
    __shared__ uint32_t boff[kPrepMaxBags + 1];   // bag starts, relative to the block's first lookup
    __shared__ uint32_t hoff[kPrepMaxBags + 1];   // first key of each table the block touches
    __shared__ uint32_t hwt[MODE == kPayloadMean ? kPrepMaxBags + 1 : 1];   // tables' weighted flag
    const int tid = threadIdx.x;
    for (int i = tid; i < 4 * kRadixMax; i += kPrepThreads) (&hist[0][0])[i] = 0u;
    const uint32_t g0 = blockIdx.x * bags_per_block;
    const uint32_t nb = g0 < total_bags ? min(bags_per_block, total_bags - g0) : 0u;
    const uint32_t t_first = nb ? g0 / B : 0;
    const uint32_t t_count = nb ? (g0 + nb - 1) / B - t_first + 1 : 0;   // <= nb
    const int64_t P0 = nb ? static_cast<int64_t>(offsets[g0]) : 0;
    for (uint32_t i = tid; i <= nb && nb > 0; i += kPrepThreads)
        boff[i] = static_cast<uint32_t>(static_cast<int64_t>(offsets[g0 + i]) - P0);
    for (uint32_t i = tid; i < t_count; i += kPrepThreads) {
        hoff[i] = tables[t_first + i].hash_off;
        if (MODE == kPayloadMean) hwt[i] = (tables[t_first + i].flags & TD_WEIGHTED) ? 1u : 0u;
    }
    __syncthreads();
    const uint32_t len = nb ? boff[nb] : 0u;
    uint32_t top = 1;
    while (top < nb) top <<= 1;
    constexpr int UN = 8;
    for (uint32_t base = 0; base < len; base += kPrepThreads * UN) {
        IT id[UN];
        float wv[UN];
        uint32_t g[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const uint32_t rp = base + u * kPrepThreads + tid;
            id[u] = rp < len ? indices[P0 + rp] : IT(0);
            wv[u] = ((MODE == kPayloadSampleW || (MODE == kPayloadMean && psw)) && rp < len)
                        ? psw[P0 + rp] : 1.f;
            g[u] = 0;
        }
        // g[u]: the last bag whose start is <= rp (that bag is not empty);
        // branch-free, so the searches of the used slots interleave
        const uint32_t nu = (len - base + kPrepThreads - 1) / kPrepThreads;   // slots in use
        for (uint32_t st = top; st > 0; st >>= 1) {
#pragma unroll
            for (int u = 0; u < UN; ++u) {
                if (u < nu) {
                    const uint32_t rp = base + u * kPrepThreads + tid;
                    const uint32_t c = g[u] + st;
                    const uint32_t v = boff[c < nb ? c : nb - 1];
                    g[u] = (c < nb && v <= rp) ? c : g[u];
                }
            }
        }
        // keys and payloads first, histograms next, stores last: a store's
        // registers are not reused before the loop ends, so no wait on it
        uint32_t key[UN], pay[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const uint32_t gg = g0 + g[u];
            const uint32_t t = gg / B;
            key[u] = hoff[t - t_first] + static_cast<uint32_t>(id[u]);
            pay[u] = gg - t * B;
            if (MODE == kPayloadPos) pay[u] = static_cast<uint32_t>(P0 + base + u * kPrepThreads + tid);
            if (MODE == kPayloadMean) {   // d(mean)/d(row) = weight / bag length
                const float w = (psw && hwt[t - t_first]) ? wv[u] : 1.f;
                wv[u] = w / static_cast<float>(boff[g[u] + 1] - boff[g[u]]);
            }
        }
        // digit counts (the order of the adds does not matter).  The lanes
        // whose digit equals the wave's first active lane's are merged into
        // one add: a bag's ids come from one table, so the upper digits are
        // often one value across the wave, and same-address LDS adds would
        // otherwise serialize; the other lanes add one each.
        const int lane = tid & 63;
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const bool ok = base + u * kPrepThreads + tid < len;
            const uint32_t dk = key[u];
            if (ok)
                for (int q = 0; q < pb.npasses; ++q) {
                    const uint32_t d = (dk >> pb.shift[q]) & pb.mask[q];
                    const uint32_t d0 = __builtin_amdgcn_readfirstlane(d);
                    const uint64_t same = __ballot(d == d0);
                    if (d != d0)
                        atomicAdd(&hist[q][d], 1u);
                    else if (lane == __builtin_ctzll(same))
                        atomicAdd(&hist[q][d0], static_cast<uint32_t>(__popcll(same)));
                }
        }
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const uint32_t rp = base + u * kPrepThreads + tid;
            if (rp < len) {
                const int64_t p = P0 + rp;
                keys[p] = key[u];
                if (MODE == kPayloadSampleW || MODE == kPayloadMean)
                    static_cast<uint2*>(vals)[p] = make_uint2(pay[u], __float_as_uint(wv[u]));
                else
                    static_cast<uint32_t*>(vals)[p] = pay[u];
            }
        }
    }
    __syncthreads();
    // digit totals are spread over kTotCopies copies (fewer adds per address)
    uint32_t* tcopy = totals + (blockIdx.x % kTotCopies) * (4 * kRadixMax);
    for (int i = tid; i < 4 * kRadixMax; i += kPrepThreads) {
        const int q = i / kRadixMax;
        const uint32_t c = hist[q][i % kRadixMax];
        if (q < pb.npasses && c) atomicAdd(&tcopy[i], c);
    }
    // the look-back words of the radix passes and the run-length encode
    for (size_t i = blockIdx.x * size_t(kPrepThreads) + tid; i < status_words;
         i += size_t(gridDim.x) * kPrepThreads)
        status[i] = 0u;
}

// ---------------------------------------------------------------------------
// Key pass of a per-table sort whose first radix pass reads the batch itself:
// digit counts only.  seg_bpt blocks per table, each over bags_per_block
// bags of that one table, so its counts are the table's (added to one of
// seg_copies copies, zeroed by k_seg_setup); the ids are streamed two batches
// deep (the next batch loads while this one is counted) and nothing is
// written per lookup.  For each radix tile that starts among the block's
// lookups, the bag holding that first position (within its table) goes to
// tile_bag[seg_first[t] + tile index in the table].
template <typename IT>
__global__ __launch_bounds__(kPrepThreads) void k_count(
    uint32_t B, uint32_t bags_per_block, const IT* __restrict__ indices,
    const IT* __restrict__ offsets, PassBits pb, uint32_t* __restrict__ status,
    size_t status_words, uint32_t seg_bpt, uint32_t seg_copies, uint32_t* __restrict__ tab_tot,
    uint32_t* __restrict__ tile_bag, const uint32_t* __restrict__ seg_first, uint32_t sort_tile)
{
    __shared__ uint32_t hist[4][kRadixMax];
    __shared__ uint32_t boff[kPrepMaxBags + 1];   // bag starts, relative to the block's first lookup
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    for (int i = tid; i < 4 * kRadixMax; i += kPrepThreads) (&hist[0][0])[i] = 0u;
    const uint32_t t = blockIdx.x / seg_bpt, j = blockIdx.x - t * seg_bpt;
    const uint32_t b0 = j * bags_per_block;
    const uint32_t nb = b0 < B ? min(bags_per_block, B - b0) : 0u;
    const size_t g0 = size_t(t) * B + b0;
    const int64_t P0 = static_cast<int64_t>(offsets[g0]);
    const uint32_t len = static_cast<uint32_t>(static_cast<int64_t>(offsets[g0 + nb]) - P0);
    const int64_t T0 = static_cast<int64_t>(offsets[size_t(t) * B]);   // the table's first lookup
    // this block's bag starts, loaded now and staged after the counts
    constexpr int BPT = (kPrepMaxBags + kPrepThreads) / kPrepThreads;
    uint32_t bs[BPT];
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
        const uint32_t i = k * kPrepThreads + tid;
        bs[k] = i <= nb ? static_cast<uint32_t>(static_cast<int64_t>(offsets[g0 + i]) - P0) : 0u;
    }
    __syncthreads();   // counters cleared
    constexpr int UN = 8;
    constexpr uint32_t kStep = kPrepThreads * UN;
    auto load = [&](uint32_t base, uint32_t (&id)[UN]) {
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const uint32_t rp = base + u * kPrepThreads + tid;
            id[u] = rp < len ? static_cast<uint32_t>(indices[P0 + rp]) : 0u;
        }
    };
    uint32_t cur[UN], nxt[UN];
    load(0, cur);
    for (uint32_t base = 0; base < len; base += kStep) {
        if (base + kStep < len) load(base + kStep, nxt);
        // digit counts; lanes sharing the wave's first active lane's digit
        // add once (a table's rows often share their upper digits)
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            if (base + u * kPrepThreads + tid < len)
                for (int q = 0; q < pb.npasses; ++q) {
                    const uint32_t d = (cur[u] >> pb.shift[q]) & pb.mask[q];
                    const uint32_t d0 = __builtin_amdgcn_readfirstlane(d);
                    const uint64_t same = __ballot(d == d0);
                    if (d != d0)
                        atomicAdd(&hist[q][d], 1u);
                    else if (lane == __builtin_ctzll(same))
                        atomicAdd(&hist[q][d0], static_cast<uint32_t>(__popcll(same)));
                }
        }
#pragma unroll
        for (int u = 0; u < UN; ++u) cur[u] = nxt[u];
    }
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
        const uint32_t i = k * kPrepThreads + tid;
        if (i <= nb) boff[i] = bs[k];
    }
    __syncthreads();
    {   // one copy of this table's counts (blocks of the table share the copies)
        uint32_t* tt = tab_tot + (size_t(t) * seg_copies + j % seg_copies) * pb.npasses * kRadixMax;
        for (int i = tid; i < pb.npasses * kRadixMax; i += kPrepThreads) {
            const uint32_t c = hist[i / kRadixMax][i % kRadixMax];
            if (c) atomicAdd(&tt[i], c);
        }
    }
    // tiles of this table whose first position (relative to the table's first
    // lookup) falls in [rel0, rel0 + len)
    uint32_t top = 1;
    while (top < nb) top <<= 1;
    const uint32_t rel0 = static_cast<uint32_t>(P0 - T0);
    for (uint32_t kt = (rel0 + sort_tile - 1) / sort_tile + tid; kt * sort_tile < rel0 + len;
         kt += kPrepThreads) {
        const uint32_t rp = kt * sort_tile - rel0;
        uint32_t g = 0;   // the last bag whose start is <= rp (not empty)
        for (uint32_t st = top; st > 0; st >>= 1) {
            const uint32_t c = g + st;
            g = (c < nb && boff[c] <= rp) ? c : g;
        }
        tile_bag[seg_first[t] + kt] = b0 + g;
    }
    // the look-back words of the radix passes and the run-length encode
    for (size_t i = blockIdx.x * size_t(kPrepThreads) + tid; i < status_words;
         i += size_t(gridDim.x) * kPrepThreads)
        status[i] = 0u;
}

// ---------------------------------------------------------------------------
// Segmented sort set-up, before the key pass.  Block 0 lays out the tiles,
// each inside one table's segment of lookup positions, in table order (slots
// past the last tile are marked unused: table 0xFFFFFFFF), and writes each
// table's first tile slot to first_out[T + 1]; the other blocks zero the
// per-table digit counts the key pass adds to.  Everything is written whole,
// every call.
template <typename IT>
__global__ __launch_bounds__(1024) void k_seg_setup(
    const IT* __restrict__ offsets, uint32_t B, int32_t T, uint32_t* __restrict__ tab_tot,
    uint32_t tot_words, uint4* __restrict__ tiles, uint32_t ntiles, uint32_t tile,
    uint32_t* __restrict__ first_out)
{
    const int tid = threadIdx.x;
    if (blockIdx.x > 0) {
        for (size_t i = size_t(blockIdx.x - 1) * 1024 + tid; i < tot_words;
             i += size_t(gridDim.x - 1) * 1024)
            tab_tot[i] = 0u;
        return;
    }
    static_assert(kSegMaxTables <= 1024, "one thread per table");
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t first_of[kSegMaxTables + 1], seg_s[kSegMaxTables], seg_e[kSegMaxTables];
    const int lane = tid & 63, wave = tid >> 6;
    uint32_t s = 0, e = 0, n = 0;
    if (tid < T) {
        s = static_cast<uint32_t>(offsets[size_t(tid) * B]);
        e = static_cast<uint32_t>(offsets[size_t(tid + 1) * B]);
        n = e > s ? (e - s + tile - 1) / tile : 0u;
    }
    const uint32_t inc = wave_incl_scan(n, lane);
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    uint32_t first = inc - n;
    for (int w = 0; w < wave; ++w) first += wsum[w];
    if (tid < T) {
        first_of[tid] = first;
        first_out[tid] = first;
        seg_s[tid] = s;
        seg_e[tid] = e;
    }
    if (tid == T - 1) {
        first_of[T] = first + n;
        first_out[T] = first + n;
    }
    __syncthreads();
    const uint32_t used = first_of[T];
    for (uint32_t i = tid; i < ntiles; i += 1024) {
        if (i >= used) {
            tiles[i] = make_uint4(0u, 0u, 0u, 0xFFFFFFFFu);
            continue;
        }
        int lo = 0, hi = T - 1;   // the last table whose first tile is at or before i
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (first_of[mid] <= i) lo = mid; else hi = mid - 1;
        }
        const uint32_t k = i - first_of[lo];
        tiles[i] = make_uint4(seg_s[lo] + k * tile, min(seg_e[lo], seg_s[lo] + (k + 1) * tile),
                              seg_s[lo], static_cast<uint32_t>(lo));
    }
}

// ---------------------------------------------------------------------------
// One radix pass over NB-bit digits.  A tile is kSortThreads x R keys; wave w
// ranks rounds of 64 keys with ballots (equal digits of a round are found bit
// by bit) and its own LDS digit counters, so the rank is stable inside the
// tile.  The ticket and the digit-totals loads are issued together, so they
// cost one round trip.
// LOWLDS: keys and then the payload go through one 32-bit staging buffer
// (with each staged position's digit beside it, for its output position), so
// a tile needs about 63 KB of LDS instead of 89 KB and, with a 4-byte payload
// (at most 64 VGPRs), two tiles share a CU.
// Segmented sort (seg.tiles set): a tile's keys, positions and digit counts
// come from its slot in seg.tiles (one table's segment), digits are of the
// row (key - the table's first key), and the look-back stops at the table's
// first tile.
// FIRST (the first pass of a segmented sort, after a counts-only key pass):
// a tile reads the ids itself (key = the table's first key + row) and makes
// its payload: the bag of each position comes from marks at the bags' first
// positions in LDS and a running maximum over positions, starting from the
// bag that holds the tile's first position (tile_bag).  Mean pooling's
// weight / bag length: each marked bag's length is kept at its first
// position too, and a second running maximum (of marked positions) finds the
// first position of each position's bag.
struct FirstPass {
    const void* indices;        // int32, or int64 when i64
    const void* offsets;        // [T * B + 1], same type
    const float* psw;           // per-sample weights (payload pairs; may be null with mean)
    const uint32_t* tile_bag;   // [ntiles] bag (within its table) of each tile's first position
    const TableDesc* tables;    // weighted flags (mean pooling)
    uint32_t B;
    uint32_t i64;
    uint32_t pos_payload;       // payload = lookup position instead of the bag
    uint32_t mean;              // payload = (bag, weight / bag length)
};

struct SegPass {
    const uint4* tiles;      // [ntiles] {first position, end, table's first position, table}
    const uint32_t* tot;     // this pass's digit counts of table t, copy c at
    uint32_t stride;         //   tot + t * stride + c * cstride
    uint32_t cstride;
    uint32_t copies;
    const uint32_t* hash_off;
};

template <int R, typename PT, int NB, bool LOWLDS, bool FIRST>
__global__ __launch_bounds__(kSortThreads) __attribute__((amdgpu_waves_per_eu(LOWLDS ? 8 : 4))) void k_onesweep(
    const uint32_t* __restrict__ keys_in, const PT* __restrict__ vals_in,
    uint32_t* __restrict__ keys_out, PT* __restrict__ vals_out, uint32_t N, int shift,
    const uint32_t* __restrict__ totals, uint32_t* __restrict__ status,
    uint32_t* __restrict__ ticket, uint32_t* __restrict__ err, uint32_t ntiles,
    uint32_t* __restrict__ prev_totals, SegPass seg, FirstPass fp)
{
    static_assert(!FIRST || sizeof(PT) == 4 || sizeof(PT) == 8, "payload: bag, position or pair");
    constexpr int NW = kSortThreads / 64;
    constexpr int RX = NB > 8 ? 512 : 256;   // digit counters
    constexpr int NQ = kSortThreads / RX;    // thread groups covering every digit
    static_assert(!LOWLDS || NB <= 8, "the low-LDS tile stages digits as bytes");
    static_assert(RX <= kRadixMax && NW % NQ == 0, "digit layout");
    __shared__ uint32_t wcnt[NW][RX];
    __shared__ uint32_t part[NQ][RX];
    __shared__ uint32_t gofs[RX];
    __shared__ uint32_t lbase[RX];
    __shared__ uint32_t delta[RX];
    __shared__ uint32_t wsum[RX / 64];
    __shared__ uint32_t s_tile;
    __shared__ uint32_t sk[kSortThreads * R];
    __shared__ PT sv[LOWLDS ? 1 : kSortThreads * R];
    __shared__ uint8_t sdig[LOWLDS ? kSortThreads * R : 1];
    __shared__ uint32_t wmax[FIRST ? kSortThreads / 64 : 1];
    __shared__ uint32_t wlen[FIRST ? kSortThreads / 64 : 1];   // mean: length of each wave's last marked bag
    // mean: bag lengths at their first positions, in the payload staging
    // buffer (free until the staging)
    uint32_t* const len_at = reinterpret_cast<uint32_t*>(&sv[0]);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    constexpr uint32_t kTile = uint32_t(kSortThreads) * R;
    uint32_t tot = 0, tile, t0, tend, base0 = 0, hoff = 0, lb_base = 0, lb_tile, tab = 0;
    if (seg.tiles == nullptr) {
        // the ticket is taken by a wave that loads no totals, so the two overlap
        if (tid == RX % kSortThreads) s_tile = take_ticket(ticket, ntiles);
        if (tid < RX) {
#pragma unroll
            for (int cp = 0; cp < kTotCopies; ++cp) tot += totals[cp * 4 * kRadixMax + tid];
        }
        // the previous pass's digit totals are no longer needed: leave them zero
        if (blockIdx.x == 0 && prev_totals && tid < kRadixMax)
#pragma unroll
            for (int cp = 0; cp < kTotCopies; ++cp) prev_totals[cp * 4 * kRadixMax + tid] = 0u;
        for (int i = tid; i < NW * RX; i += kSortThreads) (&wcnt[0][0])[i] = 0u;
        __syncthreads();
        tile = __builtin_amdgcn_readfirstlane(s_tile);
        if (tile >= ntiles) {          // only with an uninitialised control block
            if (tid == 0) atomicOr(err, kErrControl);
            return;
        }
        t0 = tile * kTile;
        tend = (N - t0) < kTile ? N : t0 + kTile;
        lb_tile = tile;
    } else {
        if (tid == 0) s_tile = take_ticket(ticket, ntiles);
        for (int i = tid; i < NW * RX; i += kSortThreads) (&wcnt[0][0])[i] = 0u;
        if constexpr (FIRST) {   // bag marks (and lengths)
            for (int i = tid; i < static_cast<int>(kTile); i += kSortThreads) sk[i] = 0u;
            if (sizeof(PT) == 8 && !LOWLDS && fp.mean)
                for (int i = tid; i < static_cast<int>(kTile); i += kSortThreads) len_at[i] = 0u;
        }
        __syncthreads();
        tile = __builtin_amdgcn_readfirstlane(s_tile);
        if (tile >= ntiles) {
            if (tid == 0) atomicOr(err, kErrControl);
            return;
        }
        const uint4 sl = seg.tiles[tile];
        const uint32_t t = __builtin_amdgcn_readfirstlane(sl.w);
        if (t == 0xFFFFFFFFu) return;   // a slot past the last tile
        tab = t;
        t0 = __builtin_amdgcn_readfirstlane(sl.x);
        tend = __builtin_amdgcn_readfirstlane(sl.y);
        base0 = __builtin_amdgcn_readfirstlane(sl.z);
        hoff = seg.hash_off[t];
        if (tid < RX) {   // branch-free, so the loads of the copies overlap
            const uint32_t* tp = seg.tot + size_t(t) * seg.stride + tid;
            uint32_t v[kTotCopies];
#pragma unroll
            for (int c = 0; c < kTotCopies; ++c)
                v[c] = tp[size_t(c < seg.copies ? c : 0) * seg.cstride];
#pragma unroll
            for (int c = 0; c < kTotCopies; ++c) tot += c < seg.copies ? v[c] : 0u;
        }
        lb_tile = (t0 - base0) / kTile;   // the tile's index inside its table
        lb_base = tile - lb_tile;         // the table's first tile
    }
    constexpr uint32_t mask = (1u << NB) - 1u;
    const uint32_t wbase = t0 + static_cast<uint32_t>(wave) * (64u * R);
    uint32_t k[R], dg[R], rk[R];
    PT v[R];
    // FIRST: the bag holding the tile's first position, and the first 1024
    // bags after it (their first positions), loaded under the rank
    constexpr bool MEANOK = FIRST && sizeof(PT) == 8 && !LOWLDS;   // tiles that can pool means
    const bool mean = MEANOK && fp.mean != 0u;
    uint32_t fb = 0u, st_first = 0u, en_first = 0u, len_fb = 0u;
    uint32_t mlen[R];   // mean: each position's bag length when its bag starts in this wave
    bool tab_w = false;
    size_t ob = 0;
    auto bag_start = [&](uint32_t c) {
        return fp.i64 ? static_cast<uint32_t>(static_cast<const int64_t*>(fp.offsets)[ob + c])
                      : static_cast<uint32_t>(static_cast<const int32_t*>(fp.offsets)[ob + c]);
    };
    if constexpr (FIRST) {
        fb = __builtin_amdgcn_readfirstlane(fp.tile_bag[tile]);
        if (fb >= fp.B) {   // only with an inconsistent tile_bag
            if (tid == 0) atomicOr(err, kErrControl);
            fb = 0u;
        }
        ob = size_t(tab) * fp.B;
        // the ids (an int64 id's low word: rows are below 2^32) and weights
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t i = wbase + r * 64u + lane;
            const bool ok = i < tend;
            uint32_t row = 0u;
            if (ok) row = static_cast<const uint32_t*>(fp.indices)[fp.i64 ? 2u * i : i];   // i < 2^30
            k[r] = hoff + row;
            if constexpr (sizeof(PT) == 8) {
                uint32_t wb = 0u;
                if (ok && fp.psw) wb = __float_as_uint(fp.psw[i]);
                v[r].y = wb;
            }
        }
        if (fb + 1u + tid < fp.B) {
            st_first = bag_start(fb + 1u + tid);
            if (mean) en_first = bag_start(fb + 2u + tid);   // fb + 2 + tid <= B
        }
        if (mean) {
            len_fb = __builtin_amdgcn_readfirstlane(bag_start(fb + 1u) - bag_start(fb));
            tab_w = fp.psw && (__builtin_amdgcn_readfirstlane(fp.tables[tab].flags) & TD_WEIGHTED);
        }
    }
    uint32_t inc = 0;
    if (tid < RX) {
        inc = wave_incl_scan(tot, lane);
        if (lane == 63) wsum[wave] = inc;
    }
    __syncthreads();
    if (tid < RX) {
        uint32_t pre = 0;
        for (int w = 0; w < wave; ++w) pre += wsum[w];
        gofs[tid] = base0 + pre + inc - tot;   // first output position of digit tid
    }

    if constexpr (!FIRST) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t i = wbase + r * 64u + lane;
            const bool ok = i < tend;
            k[r] = ok ? keys_in[i] : 0u;
            if (ok) v[r] = vals_in[i];
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t i = wbase + r * 64u + lane;
        const bool ok = i < tend;
        const uint32_t d = ((k[r] - hoff) >> shift) & mask;
        // lanes whose digit differs from this lane's in some bit, as two
        // 32-bit halves: per bit, the ballot of the bit xor this lane's bit
        // spread over a word (this shape compiles to three-input bit ops)
        uint32_t xlo = 0u, xhi = 0u;
#pragma unroll
        for (int bit = 0; bit < NB; ++bit) {
            const uint32_t m = static_cast<uint32_t>(static_cast<int32_t>(d << (31 - bit)) >> 31);
            const uint64_t bal = __ballot(m != 0u);
            xlo |= static_cast<uint32_t>(bal) ^ m;
            xhi |= static_cast<uint32_t>(bal >> 32) ^ m;
        }
        const uint64_t okm = __ballot(ok);
        const uint32_t plo = ~xlo & static_cast<uint32_t>(okm);
        const uint32_t phi = ~xhi & static_cast<uint32_t>(okm >> 32);
        // peers in lower lanes, and all peers
        const uint32_t below = __builtin_amdgcn_mbcnt_hi(phi, __builtin_amdgcn_mbcnt_lo(plo, 0u));
        const uint32_t npeer = static_cast<uint32_t>(__popc(plo) + __popc(phi));
        uint32_t base = 0;
        if (ok) base = wcnt[wave][d];
        if (ok && below == 0) wcnt[wave][d] = base + npeer;
        dg[r] = d;
        rk[r] = base + below;
    }
    if constexpr (FIRST) {
        // mark each bag that starts inside the tile at its first position
        // (the largest of bags starting together is the one not empty); the
        // barrier that ends the rank ends the first 1024 bags' marks
        uint32_t c = fb + 1u + tid;
        uint32_t st = st_first, en = en_first;
        for (;;) {
            const bool more = c < fp.B && st < tend;
            if (more && st > t0) {
                atomicMax(&sk[st - t0], c);
                if (mean) atomicMax(&len_at[st - t0], en - st);   // empty bags add 0
            }
            if (!__syncthreads_or(tid == kSortThreads - 1 && more)) break;
            c += kSortThreads;
            if (c < fp.B) {
                st = bag_start(c);
                if (mean) en = bag_start(c + 1u);
            }
        }
        // each position's bag: running maximum over the wave's positions
        // (the rounds are scanned side by side, then carried in order)
        uint32_t bm[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            bm[r] = wave_incl_max(sk[static_cast<uint32_t>(wave) * (64u * R) + r * 64u + lane]);
        uint32_t run = fb;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t m = bm[r] > run ? bm[r] : run;
            if constexpr (sizeof(PT) == 8)
                v[r].x = m;
            else
                v[r] = m;
            const uint32_t last = __builtin_amdgcn_readlane(bm[r], 63);
            run = last > run ? last : run;
        }
        if (lane == 0) wmax[wave] = run;   // read after the next barrier
        if (mean) {
            // the first position of each position's bag when it starts in
            // this wave (0: it started earlier), and that bag's length
            uint32_t srun = 0u;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t li = static_cast<uint32_t>(wave) * (64u * R) + r * 64u + lane;
                uint32_t m = wave_incl_max(sk[li] != 0u ? li : 0u);
                m = m > srun ? m : srun;
                srun = __builtin_amdgcn_readlane(m, 63);
                mlen[r] = m != 0u ? len_at[m] : 0u;
            }
            if (lane == 0) wlen[wave] = srun != 0u ? len_at[srun] : 0u;
        }
    } else {
        __syncthreads();
    }
    // per digit: exclusive prefix over the waves (NQ groups of NW/NQ waves),
    // the tile's digit total, and its exclusive prefix over digits (lbase)
    const int d = tid & (RX - 1), q = tid / RX;
    uint32_t all = 0, dinc = 0;
    {
        constexpr int G = NW / NQ;
        uint32_t run = 0;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const uint32_t c = wcnt[q * G + j][d];
            wcnt[q * G + j][d] = run;
            run += c;
        }
        part[q][d] = run;
        __syncthreads();
        uint32_t pre = 0;
        for (int j = 0; j < q; ++j) pre += part[j][d];
        if (q > 0)
#pragma unroll
            for (int j = 0; j < G; ++j) wcnt[q * G + j][d] += pre;
        if (q == 0) {
#pragma unroll
            for (int j = 0; j < NQ; ++j) all += part[j][d];
            dinc = wave_incl_scan(all, lane);
            if (lane == 63) wsum[wave] = dinc;
        }
    }
    __syncthreads();
    uint32_t lb = 0;
    if (q == 0) {
        for (int w = 0; w < wave; ++w) lb += wsum[w];
        lb += dinc - all;
        lbase[d] = lb;
    }
    __syncthreads();
    if constexpr (FIRST) {   // the bags carried in from earlier waves
        uint32_t prior = 0u;
        for (int w = 0; w < wave; ++w) prior = wmax[w] > prior ? wmax[w] : prior;
        uint32_t clen = len_fb;   // mean: length of the bag carried in from earlier waves
        if (mean)
            for (int w = 0; w < wave; ++w) clen = wlen[w] != 0u ? wlen[w] : clen;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if constexpr (sizeof(PT) == 8) {
                v[r].x = v[r].x > prior ? v[r].x : prior;
                if constexpr (MEANOK) {
                    if (mean) {   // d(mean)/d(row) = weight / bag length
                        const uint32_t bl = mlen[r] != 0u ? mlen[r] : clen;
                        const float w = tab_w ? __uint_as_float(v[r].y) : 1.f;
                        v[r].y = __float_as_uint(w / static_cast<float>(bl));
                    }
                }
            } else {
                const uint32_t b = v[r] > prior ? v[r] : prior;
                v[r] = fp.pos_payload ? wbase + r * 64u + lane : b;
            }
        }
    }
    // stage the tile in LDS in output order; meanwhile waves 0-3 look back
    // for the tile's global digit offsets
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t i = wbase + r * 64u + lane;
        if (i < tend) {
            const uint32_t lp = lbase[dg[r]] + wcnt[wave][dg[r]] + rk[r];
            sk[lp] = k[r];
            if constexpr (LOWLDS)
                sdig[lp] = static_cast<uint8_t>(dg[r]);
            else
                sv[lp] = v[r];
        }
    }
    if (q == 0)
        delta[d] = gofs[d] + lookback<16>(status + size_t(lb_base) * RX + d, RX, lb_tile, all, err) - lb;
    __syncthreads();
    // write out: consecutive threads store consecutive positions of a digit
    const uint32_t cnt = tend - t0;
    if constexpr (!LOWLDS) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t e = r * kSortThreads + tid;
            if (e < cnt) {
                const uint32_t key = sk[e];
                const uint32_t pos = delta[((key - hoff) >> shift) & mask] + e;
                if (pos >= N) continue;  // unreachable when the counts are consistent
                keys_out[pos] = key;
                vals_out[pos] = sv[e];
            }
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t e = r * kSortThreads + tid;
            if (e < cnt) {
                const uint32_t pos = delta[sdig[e]] + e;
                if (pos < N) keys_out[pos] = sk[e];   // pos < N unless the counts are inconsistent
            }
        }
        // each 32-bit word of the payload through the same buffer
        constexpr int W = sizeof(PT) / 4;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            __syncthreads();   // every read of the buffer's previous contents is done
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t i = wbase + r * 64u + lane;
                if (i < tend) {
                    const uint32_t lp = lbase[dg[r]] + wcnt[wave][dg[r]] + rk[r];
                    uint32_t word[W];
                    __builtin_memcpy(word, &v[r], sizeof(PT));
                    sk[lp] = word[w];
                }
            }
            __syncthreads();
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t e = r * kSortThreads + tid;
                if (e < cnt) {
                    const uint32_t pos = delta[sdig[e]] + e;
                    if (pos < N)
                        reinterpret_cast<uint32_t*>(vals_out)[static_cast<size_t>(pos) * W + w] =
                            sk[e];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Exclusive prefix over tiles 0..tile-1, computed by one whole wavefront: lane l
// reads the word of tile tp-l, so one memory round trip crosses up to 64
// published tiles.  Same flags and publication order as lookback().
__device__ __forceinline__ uint32_t lookback_wave(uint32_t* st, uint32_t tile, uint32_t value,
                                                  uint32_t* err, int lane)
{
    if (tile == 0) {
        if (lane == 0) st_rel(st, kFlagInc | value);
        return 0;
    }
    uint32_t excl = 0;
    int64_t tp = static_cast<int64_t>(tile) - 1;
    uint32_t spins = 0;
    // first window before publishing (see lookback())
    uint32_t s = (tp - lane >= 0) ? ld_acq(st + (tp - lane)) : kFlagInc;
    if (lane == 0) st_rel(st + tile, kFlagAgg | value);
    while (true) {
        const uint32_t f = s & ~kValMask;
        const uint64_t unpub = __ballot(f == 0);
        const uint64_t incl = __ballot(f == kFlagInc);
        const int first_unpub = unpub ? __builtin_ctzll(unpub) : 64;
        const int first_inc = incl ? __builtin_ctzll(incl) : 64;
        if (first_inc < first_unpub) {
            excl += wave_sum(lane <= first_inc ? (s & kValMask) : 0u);
            break;
        }
        excl += wave_sum(lane < first_unpub ? (s & kValMask) : 0u);
        tp -= first_unpub;
        if (first_unpub == 0) {
            if (++spins > kSpinLimit) {
                if (lane == 0) atomicOr(err, kErrLookback);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        s = (tp - lane >= 0) ? ld_acq(st + (tp - lane)) : kFlagInc;
    }
    if (lane == 0) st_rel(st + tile, kFlagInc | ((excl + value) & kValMask));
    return excl;
}

// In-place exclusive scan of a [Q][kRleThreads / 64] table of counts
// (round-major), by one wavefront; returns the table total on every lane.
template <int Q>
__device__ __forceinline__ uint32_t scan_table(uint32_t* tab, int lane)
{
    static_assert(Q * (kRleThreads / 64) == 64 || Q * (kRleThreads / 64) == 128,
                  "one or two entries per lane");
    if constexpr (Q * (kRleThreads / 64) == 64) {
        const uint32_t x1 = tab[lane];
        const uint32_t inc1 = wave_incl_scan(x1, lane);
        tab[lane] = inc1 - x1;
        return __shfl(inc1, 63);
    }
    const uint32_t x = tab[2 * lane], y = tab[2 * lane + 1];
    const uint32_t inc = wave_incl_scan(x + y, lane);
    const uint32_t ex = inc - x - y;
    tab[2 * lane] = ex;
    tab[2 * lane + 1] = ex + x;
    return __shfl(inc, 63);
}

// GLOBAL: hash_off is in global memory (loaded as such, so the compiler cannot
// merge the LDS and global searches into one flat-load search).
template <bool GLOBAL>
__device__ __forceinline__ int find_table(const uint32_t* hash_off, int T, uint32_t key)
{
    int lo = 0, hi = T;  // hash_off[lo] <= key < hash_off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        const uint32_t h = GLOBAL ? gload(hash_off + mid) : hash_off[mid];
        if (h <= key) lo = mid; else hi = mid;
    }
    return lo;
}

// First position >= from whose key differs from `key` (N if none), found by
// one wavefront: 32 exponentially spaced probes, then rounds of 64 evenly
// spaced probes inside the bracket.  Keys are sorted, so "differs" is monotone.
__device__ __forceinline__ uint32_t run_end_wave(const uint32_t* __restrict__ keys, uint32_t N,
                                                 uint32_t from, uint32_t key, int lane)
{
    if (from >= N) return N;
    uint64_t p = from + ((lane < 32) ? ((uint64_t(1) << lane) - 1) : (uint64_t(1) << 40));
    bool diff = p >= N || keys[p] != key;
    uint64_t bal = __ballot(diff);   // lane 63 probes past N, so bal != 0
    const int l = __builtin_ctzll(bal);
    if (l == 0) return from;
    uint64_t lo = from + ((uint64_t(1) << (l - 1)) - 1);   // same key
    uint64_t hi = from + ((uint64_t(1) << l) - 1);         // differs or past N
    if (hi > N) hi = N;
    while (hi - lo > 1) {
        const uint64_t step = (hi - lo + 63) / 64;
        uint64_t q = lo + (lane + 1) * step;
        if (q > hi) q = hi;
        diff = q >= hi || keys[q] != key;   // hi itself is known to differ
        bal = __ballot(diff);
        const int m = __builtin_ctzll(bal);
        const uint64_t nhi = lo + (m + 1) * step;
        hi = nhi < hi ? nhi : hi;
        lo = lo + m * step;
    }
    return static_cast<uint32_t>(hi);
}

// Run-length encode of the sorted keys.  A tile is Q rounds (kRleItems, or
// kRleItemsSmall for small batches) of
// kRleThreads consecutive positions (round q, thread i: position
// tile*Q*kRleThreads + q*kRleThreads + i), so every store of a round is coalesced.
// Run indices come from per-(round, wave) ballot counts scanned in position
// order; run lengths from the next head's position (kept in LDS), except for
// the tile's last run, which one wavefront follows past the tile's end.
// FIRST: 0 = no payload (the sort_rle entry point), 1 = payload is the sample
// id, 2 = payload is (sample id, per-sample weight).  With a payload, each
// short run's first (sample, weight) is stored next to its record, so a run of
// one lookup needs no payload load in the segment kernel.
template <bool API, int FIRST, int Q>
__global__ __launch_bounds__(kRleThreads) void k_rle(
    const uint32_t* __restrict__ keys, const void* __restrict__ payload,
    uint2* __restrict__ short_first, uint32_t N, uint32_t tau, uint32_t chunk, uint32_t ntiles,
    uint32_t* __restrict__ rstatus, uint32_t* __restrict__ ticket, uint32_t* __restrict__ err,
    const uint32_t* __restrict__ hash_off, int32_t T, uint4* __restrict__ short_info,
    uint4* __restrict__ long_info, uint32_t* __restrict__ counts,
    uint32_t* __restrict__ mode_word, uint32_t max_long, uint32_t* __restrict__ prev_totals,
    uint32_t* __restrict__ unique, uint32_t* __restrict__ run_start,
    uint32_t* __restrict__ run_len, uint32_t* __restrict__ short_ids,
    uint32_t* __restrict__ long_ids, uint32_t* __restrict__ tab_ranges,
    uint2* __restrict__ chunk_info, uint32_t max_chunks)
{
    constexpr int NW = kRleThreads / 64;
    constexpr int kTile = kRleThreads * Q;
    __shared__ uint32_t hp[kTile + 1];           // head positions in run order
    __shared__ uint32_t s_hash[kRleMaxT + 1];
    __shared__ uint32_t cnt[3][Q * NW];          // heads, long runs, chunks per (round, wave)
    __shared__ uint32_t s_tot[3];
    __shared__ uint32_t texcl[3];
    __shared__ uint32_t s_tile, s_end;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (tid == 0) s_tile = take_ticket(ticket, ntiles);
    if (blockIdx.x == 0 && prev_totals && tid < kRadixMax)   // the last radix pass is done with them
#pragma unroll
        for (int cp = 0; cp < kTotCopies; ++cp) prev_totals[cp * 4 * kRadixMax + tid] = 0u;
    const bool lds_hash = T <= kRleMaxT;
    if (lds_hash)
        for (int i = tid; i <= T; i += kRleThreads) s_hash[i] = hash_off[i];
    __syncthreads();
    const uint32_t tile = s_tile;
    if (tile >= ntiles) {          // only with an uninitialised control block
        if (tid == 0) atomicOr(err, kErrControl);
        return;
    }
    const uint32_t t0 = tile * kTile;
    const uint32_t tend = (N - t0) < uint32_t(kTile) ? N : t0 + kTile;

    // every load is issued unconditionally (positions past the end are
    // clamped to N-1 and ignored), so all 2-3 x Q of them are in flight at once
    uint32_t kk[Q], kp[Q];
    uint2 pay[Q];
    bool head[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const uint32_t p = t0 + q * kRleThreads + tid;
        const uint32_t pc = p < N ? p : N - 1;
        kk[q] = keys[pc];
        kp[q] = keys[pc > 0 ? pc - 1 : 0];
        pay[q] = make_uint2(0u, 0x3f800000u);   // weight 1.0 unless the payload has one
        if (FIRST == 1) pay[q].x = gload(static_cast<const uint32_t*>(payload) + pc);
        if (FIRST == 2) pay[q] = gload(static_cast<const uint2*>(payload) + pc);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const uint32_t p = t0 + q * kRleThreads + tid;
        head[q] = p < tend && (p == 0 || kk[q] != kp[q]);
        if (p >= tend) kk[q] = 0u;
    }
    // the tile's last run may continue into later tiles: the wave holding the
    // tile's last position finds where it ends (a full tile ends at round Q-1,
    // thread kRleThreads-1)
    if (wave == NW - 1) {
        const uint32_t klast = __shfl(kk[Q - 1], 63);
        const uint32_t e = tend == N ? N : run_end_wave(keys, N, tend, klast, lane);
        if (lane == 0) s_end = e;
    }
    uint64_t hb[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        hb[q] = __ballot(head[q]);
        if (lane == 0) cnt[0][q * NW + wave] = static_cast<uint32_t>(__popcll(hb[q]));
    }
    __syncthreads();
    if (wave == 0) {
        const uint32_t tot = scan_table<Q>(cnt[0], lane);
        if (lane == 0) {
            s_tot[0] = tot;
            hp[tot] = s_end;
        }
    }
    __syncthreads();
    uint32_t lh[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        lh[q] = cnt[0][q * NW + wave] + static_cast<uint32_t>(__popcll(hb[q] & lt));
        if (head[q]) hp[lh[q]] = t0 + q * kRleThreads + tid;
    }
    __syncthreads();
    uint32_t len[Q], ce[Q];
    uint64_t lbal[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const uint32_t p = t0 + q * kRleThreads + tid;
        len[q] = head[q] ? hp[lh[q] + 1] - p : 0u;
        const bool isl = head[q] && len[q] >= tau;
        const uint32_t nc = isl ? (len[q] + chunk - 1) / chunk : 0u;
        lbal[q] = __ballot(isl);
        uint32_t wtot = 0;
        ce[q] = 0;
        if (lbal[q]) {   // chunk prefix only where this wave has a long run
            const uint32_t inc = wave_incl_scan(nc, lane);
            ce[q] = inc - nc;
            wtot = __shfl(inc, 63);
        }
        if (lane == 0) {
            cnt[1][q * NW + wave] = static_cast<uint32_t>(__popcll(lbal[q]));
            cnt[2][q * NW + wave] = wtot;
        }
    }
    __syncthreads();
    if (wave == 1 || wave == 2) {
        const uint32_t tot = scan_table<Q>(cnt[wave], lane);
        if (lane == 0) s_tot[wave] = tot;
    }
    __syncthreads();
    if (wave < 3) {
        const uint32_t val = s_tot[wave];
        const uint32_t ex = lookback_wave(rstatus + static_cast<size_t>(wave) * ntiles, tile, val,
                                          err, lane);
        if (lane == 0) {
            texcl[wave] = ex;
            if (tile == ntiles - 1) counts[wave == 0 ? 0 : (wave == 1 ? 2 : 3)] = ex + val;
        }
    }
    __syncthreads();
    if (tile == ntiles - 1 && tid == 0) {
        const uint32_t R = texcl[0] + s_tot[0];
        counts[1] = R - (texcl[1] + s_tot[1]);
        if (API) run_start[R] = N;
        // per-table ranges past the last table that has lookups: empty, at
        // the end of every list
        const uint32_t klast = keys[N - 1];
        const int tl = lds_hash ? find_table<false>(s_hash, T, klast) : find_table<true>(hash_off, T, klast);
        for (int u = tl + 1; u <= T; ++u) {
            tab_ranges[u] = R - (texcl[1] + s_tot[1]);
            tab_ranges[(T + 1) + u] = texcl[1] + s_tot[1];
            tab_ranges[2 * (T + 1) + u] = texcl[2] + s_tot[2];
        }
        // which payload the sorted entries carry, for the segment kernels'
        // check of what their caller says
        *mode_word = FIRST == 2 ? kModePairs : (FIRST == 1 ? kModeSample : kModeNone);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        if (!head[q]) continue;
        const uint32_t i = t0 + q * kRleThreads + tid;
        const uint32_t r = texcl[0] + lh[q];
        const uint32_t lb = texcl[1] + cnt[1][q * NW + wave] +
                            static_cast<uint32_t>(__popcll(lbal[q] & lt));
        if (r >= N || lb > r) continue;  // guards: unreachable when consistent
        const uint32_t key = kk[q];
        if (API) {
            unique[r] = key;
            run_start[r] = i;
            run_len[r] = len[q];
        }
        const int t = lds_hash ? find_table<false>(s_hash, T, key) : find_table<true>(hash_off, T, key);
        // chunks of the long runs before this one
        const uint32_t cb = texcl[2] + cnt[2][q * NW + wave] + ce[q];
        // the first run of its table (the previous key is in an earlier
        // table) starts that table's ranges, and those of the tables without
        // lookups before it
        const uint32_t tkey0 = lds_hash ? s_hash[t] : gload(hash_off + t);
        if (i == 0 || kp[q] < tkey0) {
            const int tp = i == 0 ? -1
                         : (lds_hash ? find_table<false>(s_hash, T, kp[q]) : find_table<true>(hash_off, T, kp[q]));
            for (int u = tp + 1; u <= t; ++u) {
                tab_ranges[u] = r - lb;
                tab_ranges[(T + 1) + u] = lb;
                tab_ranges[2 * (T + 1) + u] = cb;
            }
        }
        if (len[q] >= tau) {
            if (lb < max_long) long_info[lb] = make_uint4(key, i, len[q], cb);
            if (API) long_ids[lb] = r;
        } else {
            short_info[r - lb] = make_uint4(key, i, len[q], static_cast<uint32_t>(t));
            if (FIRST) short_first[r - lb] = pay[q];
            if (API) short_ids[r - lb] = r;
        }
    }
    // every chunk's {first sorted position, length}, written by the whole
    // wavefront run by run (a run of 100K lookups has hundreds of chunks)
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const bool isl = head[q] && len[q] >= tau;
        uint64_t m = __ballot(isl);
        if (!m) continue;
        const uint32_t cb = texcl[2] + cnt[2][q * NW + wave] + ce[q];
        const uint32_t start = t0 + q * kRleThreads + tid;
        while (m) {
            const int l = __builtin_ctzll(m);
            m &= m - 1;
            const uint32_t cbl = __shfl(cb, l), st = __shfl(start, l), ln = __shfl(len[q], l);
            const uint32_t ncl = (ln + chunk - 1) / chunk;
            for (uint32_t j = lane; j < ncl; j += 64)
                if (cbl + j < max_chunks)
                    chunk_info[cbl + j] = make_uint2(st + j * chunk, min(chunk, ln - j * chunk));
        }
    }
}

template <int R, typename PT, int NB, bool LOWLDS, bool FIRST>
void launch_onesweep(BwdArgs& a, uint32_t nb, const uint32_t* keys_in, const PT* vals_in,
                     uint32_t* keys_out, PT* vals_out, uint32_t N, int shift, int pass,
                     uint32_t* ctl, uint32_t* status)
{
    const BwdLayout& L = a.L;
    SegPass seg{};
    if (L.seg) {
        seg.tiles = reinterpret_cast<const uint4*>(a.ws + L.off_seg_tiles);
        seg.tot = reinterpret_cast<const uint32_t*>(a.ws + L.off_tab_tot) + pass * kRadixMax;
        seg.cstride = static_cast<uint32_t>(L.npasses * kRadixMax);
        seg.stride = seg.cstride * L.seg_copies;
        seg.copies = static_cast<uint32_t>(L.seg_copies);
        seg.hash_off = a.plan->d_hash_off;
    }
    FirstPass fp{};
    if (FIRST) {
        fp.indices = a.indices;
        fp.offsets = a.offsets;
        fp.psw = a.psw;
        fp.tile_bag = reinterpret_cast<const uint32_t*>(a.ws + L.off_tile_bag);
        fp.B = static_cast<uint32_t>(a.B);
        fp.i64 = a.plan->idtype == TBE_I64 ? 1u : 0u;
        fp.pos_payload = a.payload_mode == kPayloadPos ? 1u : 0u;
        fp.mean = a.payload_mode == kPayloadMean ? 1u : 0u;
        fp.tables = a.plan->d_tables;
    }
    hipLaunchKernelGGL((k_onesweep<R, PT, NB, LOWLDS, FIRST>), dim3(nb), dim3(kSortThreads), 0, a.stream, keys_in,
                       vals_in, keys_out, vals_out, N, shift, ctl + kCtlTotals + pass * kRadixMax,
                       status + static_cast<size_t>(pass) * kRadixMax * nb,
                       ctl + kCtlTicket + pass, ctl + kCtlError, nb,
                       pass > 0 && !L.seg ? ctl + kCtlTotals + (pass - 1) * kRadixMax : nullptr,
                       seg, fp);
}

// The low-LDS tile stages digits as bytes, so a 9-bit pass takes the
// full-LDS tile whatever the tile count.
template <int R, typename PT, bool LOWLDS, bool FIRST>
auto pick_onesweep(int nbits)
{
    auto f = nbits <= 1 ? launch_onesweep<R, PT, 1, LOWLDS, FIRST>
           : nbits == 2 ? launch_onesweep<R, PT, 2, LOWLDS, FIRST>
           : nbits == 3 ? launch_onesweep<R, PT, 3, LOWLDS, FIRST>
           : nbits == 4 ? launch_onesweep<R, PT, 4, LOWLDS, FIRST>
           : nbits == 5 ? launch_onesweep<R, PT, 5, LOWLDS, FIRST>
           : nbits == 6 ? launch_onesweep<R, PT, 6, LOWLDS, FIRST>
           : nbits == 7 ? launch_onesweep<R, PT, 7, LOWLDS, FIRST>
                        : launch_onesweep<R, PT, 8, LOWLDS, FIRST>;
    if (nbits >= 9) f = launch_onesweep<R, PT, 9, false, FIRST>;
    return f;
}

// Passes of more tiles than an MI355X has CUs with a 4-byte payload take the
// low-LDS tile, two per CU.  Measured: production-scale workload (10K tiles)
// radix sort 1765 -> 1477 us, small-table workload (514 tiles) 41 -> 37 us;
// at 88 tiles of 4096 keys (uniform) it was slower (35 -> 37 us).  With an
// 8-byte payload it needs more than 64 VGPRs (8-16 spilled when forced;
// mixed 133 -> 181 us).
constexpr uint32_t kLowLdsMinTiles = 256;

template <int R, typename PT>
hipError_t sort_passes(BwdArgs& a)
{
    const BwdLayout& L = a.L;
    const uint32_t N = static_cast<uint32_t>(L.N);
    const uint32_t nb = static_cast<uint32_t>(L.sort_blocks);
    char* ws = a.ws;
    uint32_t* keys[2] = {reinterpret_cast<uint32_t*>(ws + L.off_keys[0]),
                         reinterpret_cast<uint32_t*>(ws + L.off_keys[1])};
    PT* vals[2] = {reinterpret_cast<PT*>(ws + L.off_vals[0]),
                   reinterpret_cast<PT*>(ws + L.off_vals[1])};
    uint32_t* ctl = reinterpret_cast<uint32_t*>(ws + L.off_ctl);
    uint32_t* status = reinterpret_cast<uint32_t*>(ws + L.off_status);
    int cur = 0;
    int shift = 0;
    const bool low = sizeof(PT) == 4 && nb > kLowLdsMinTiles;
    for (int pass = 0; pass < L.npasses; ++pass) {
        const int nbits = L.digit_bits[pass];
        // one instantiation per digit width: the rank tests only the digit's bits;
        // the first pass of a per-table sort reads the ids itself
        const bool first = pass == 0 && L.seg;
        auto* f = first ? pick_onesweep<R, PT, false, true>(nbits) : pick_onesweep<R, PT, false, false>(nbits);
        if constexpr (sizeof(PT) == 4)
            if (low)
                f = first ? pick_onesweep<R, PT, true, true>(nbits) : pick_onesweep<R, PT, true, false>(nbits);
        f(a, nb, keys[cur], vals[cur], keys[cur ^ 1], vals[cur ^ 1], N, shift, pass, ctl, status);
        cur ^= 1;
        shift += nbits;
    }
    a.final_buf = cur;
    return hipGetLastError();
}

template <typename IT, int MODE>
void launch_prep(const BwdArgs& a, const PassBits& pb, uint32_t total_bags)
{
    const BwdLayout& L = a.L;
    char* ws = a.ws;
    if (L.seg) {
        const uint32_t words = static_cast<uint32_t>(a.plan->T) * L.seg_copies * L.npasses * kRadixMax;
        const uint32_t zb = (words + 16 * 1024 - 1) / (16 * 1024);
        hipLaunchKernelGGL((k_seg_setup<IT>), dim3(1 + zb), dim3(1024), 0, a.stream,
                           static_cast<const IT*>(a.offsets), static_cast<uint32_t>(a.B),
                           a.plan->T, reinterpret_cast<uint32_t*>(ws + L.off_tab_tot), words,
                           reinterpret_cast<uint4*>(ws + L.off_seg_tiles),
                           static_cast<uint32_t>(L.sort_blocks),
                           static_cast<uint32_t>(L.sort_tile),
                           reinterpret_cast<uint32_t*>(ws + L.off_seg_first));
    }
    if (L.seg) {   // counts only: the first radix pass makes keys and payloads
        hipLaunchKernelGGL((k_count<IT>), dim3(L.prep_blocks), dim3(kPrepThreads), 0, a.stream,
                           static_cast<uint32_t>(a.B), static_cast<uint32_t>(L.prep_bags),
                           static_cast<const IT*>(a.indices), static_cast<const IT*>(a.offsets),
                           pb, reinterpret_cast<uint32_t*>(ws + L.off_status), L.status_words,
                           static_cast<uint32_t>(L.prep_bpt), static_cast<uint32_t>(L.seg_copies),
                           reinterpret_cast<uint32_t*>(ws + L.off_tab_tot),
                           reinterpret_cast<uint32_t*>(ws + L.off_tile_bag),
                           reinterpret_cast<const uint32_t*>(ws + L.off_seg_first),
                           static_cast<uint32_t>(L.sort_tile));
        return;
    }
    hipLaunchKernelGGL((k_prep<IT, MODE>), dim3(L.prep_blocks), dim3(kPrepThreads), 0, a.stream,
                       a.plan->d_tables, static_cast<uint32_t>(a.B), total_bags,
                       static_cast<uint32_t>(L.prep_bags), static_cast<const IT*>(a.indices),
                       static_cast<const IT*>(a.offsets), a.psw,
                       reinterpret_cast<uint32_t*>(ws + L.off_keys[0]),
                       static_cast<void*>(ws + L.off_vals[0]),
                       reinterpret_cast<uint32_t*>(ws + L.off_ctl) + kCtlTotals, pb,
                       reinterpret_cast<uint32_t*>(ws + L.off_status), L.status_words);
}

}  // namespace

hipError_t run_sort_rle(BwdArgs& a, bool api_outputs)
{
    const tbe_plan* p = a.plan;
    const BwdLayout& L = a.L;
    char* ws = a.ws;
    const uint32_t N = static_cast<uint32_t>(L.N);
    const uint32_t total_bags = static_cast<uint32_t>(p->T) * static_cast<uint32_t>(a.B);
    uint32_t* ctl = reinterpret_cast<uint32_t*>(ws + L.off_ctl);
    if (N == 0 || total_bags == 0) {
        a.final_buf = 0;
        hipLaunchKernelGGL(k_fill_zero, dim3(1), dim3(64), 0, a.stream, ctl + kCtlCounts, 4);
        return hipGetLastError();
    }
    PassBits pb{};
    pb.npasses = L.npasses;
    {
        int s = 0;
        for (int i = 0; i < L.npasses; ++i) {
            pb.shift[i] = s;
            pb.bits[i] = L.digit_bits[i];
            pb.mask[i] = (1u << L.digit_bits[i]) - 1u;
            s += L.digit_bits[i];
        }
    }
    const int mode = api_outputs ? kPayloadPos
                   : p->pooling == TBE_POOL_MEAN ? kPayloadMean
                   : (a.psw ? kPayloadSampleW : kPayloadSample);
    a.payload_pairs = mode == kPayloadSampleW || mode == kPayloadMean;
    a.payload_mode = mode;   // the per-table sort's first radix pass makes it
    const bool i64 = p->idtype == TBE_I64;
    if (L.seg)   // counts only: the payload is made by the first radix pass
        i64 ? launch_prep<int64_t, kPayloadSample>(a, pb, total_bags)
            : launch_prep<int32_t, kPayloadSample>(a, pb, total_bags);
    else if (mode == kPayloadPos)
        i64 ? launch_prep<int64_t, kPayloadPos>(a, pb, total_bags)
            : launch_prep<int32_t, kPayloadPos>(a, pb, total_bags);
    else if (mode == kPayloadSample)
        i64 ? launch_prep<int64_t, kPayloadSample>(a, pb, total_bags)
            : launch_prep<int32_t, kPayloadSample>(a, pb, total_bags);
    else if (mode == kPayloadSampleW)
        i64 ? launch_prep<int64_t, kPayloadSampleW>(a, pb, total_bags)
            : launch_prep<int32_t, kPayloadSampleW>(a, pb, total_bags);
    else
        i64 ? launch_prep<int64_t, kPayloadMean>(a, pb, total_bags)
            : launch_prep<int32_t, kPayloadMean>(a, pb, total_bags);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    stage_mark(p, 1, a.stream);
    if (L.sort_tile == kSortThreads * kSortRoundsSmall)
        e = a.payload_pairs ? sort_passes<kSortRoundsSmall, uint2>(a)
                            : sort_passes<kSortRoundsSmall, uint32_t>(a);
    else
        e = a.payload_pairs ? sort_passes<kSortRounds, uint2>(a)
                            : sort_passes<kSortRounds, uint32_t>(a);
    if (e != hipSuccess) return e;
    stage_mark(p, 2, a.stream);

    const uint32_t* skeys = reinterpret_cast<const uint32_t*>(ws + L.off_keys[a.final_buf]);
    const uint32_t tau = static_cast<uint32_t>(p->tuning.tau);
    const uint32_t chunk = static_cast<uint32_t>(p->tuning.chunk);
    const uint32_t nt = static_cast<uint32_t>(L.rle_blocks);
    const bool sq = L.rle_tile == kRleThreads * kRleItemsSmall;
    auto kern = api_outputs ? (sq ? k_rle<true, 0, kRleItemsSmall> : k_rle<true, 0, kRleItems>)
              : a.payload_pairs
                  ? (sq ? k_rle<false, 2, kRleItemsSmall> : k_rle<false, 2, kRleItems>)
                  : (sq ? k_rle<false, 1, kRleItemsSmall> : k_rle<false, 1, kRleItems>);
    hipLaunchKernelGGL(kern, dim3(nt), dim3(kRleThreads), 0, a.stream, skeys,
                       static_cast<const void*>(ws + L.off_vals[a.final_buf]),
                       reinterpret_cast<uint2*>(ws + L.off_short_first), N, tau, chunk, nt,
                       reinterpret_cast<uint32_t*>(ws + L.off_rle_status), ctl + kCtlRleTicket,
                       ctl + kCtlError, p->d_hash_off, p->T,
                       reinterpret_cast<uint4*>(ws + L.off_short_info),
                       reinterpret_cast<uint4*>(ws + L.off_long_info), ctl + kCtlCounts,
                       ctl + kCtlMode, static_cast<uint32_t>(L.max_long),
                       L.seg ? nullptr : ctl + kCtlTotals + (L.npasses - 1) * kRadixMax,
                       reinterpret_cast<uint32_t*>(ws + L.off_unique),
                       reinterpret_cast<uint32_t*>(ws + L.off_run_start),
                       reinterpret_cast<uint32_t*>(ws + L.off_run_len),
                       reinterpret_cast<uint32_t*>(ws + L.off_short),
                       reinterpret_cast<uint32_t*>(ws + L.off_long),
                       reinterpret_cast<uint32_t*>(ws + L.off_tab_ranges),
                       reinterpret_cast<uint2*>(ws + L.off_chunk_info),
                       static_cast<uint32_t>(L.max_chunks));
    stage_mark(p, 3, a.stream);
    return hipGetLastError();
}

}  // namespace tbe

namespace tbe {
namespace {
__global__ void k_copy_word(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst)
{
    *dst = *src;
}
}  // namespace

hipError_t launch_workspace_init(void* ws, hipStream_t s)
{
    hipLaunchKernelGGL(k_fill_zero, dim3(1), dim3(1024), 0, s, static_cast<uint32_t*>(ws),
                       kCtlWords);
    return hipGetLastError();
}

hipError_t launch_workspace_status(const void* ws, uint32_t* out, hipStream_t s)
{
    hipLaunchKernelGGL(k_copy_word, dim3(1), dim3(1), 0, s,
                       static_cast<const uint32_t*>(ws) + kCtlError, out);
    return hipGetLastError();
}
}  // namespace tbe
