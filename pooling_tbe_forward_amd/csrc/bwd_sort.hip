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
// Kernels (caller's stream, no host synchronisation):
//   k_prep      per block of bags: key[j] and its payload (j itself for the
//               sort_rle entry point; the bag's sample id, plus the per-sample
//               weight when there is one, for the backward -- so the sorted
//               result needs no gather), digit histograms of every radix pass
//               (equal digits of a wavefront merged by ballots, then LDS, then
//               one global add per digit), and clears the look-back words
//   k_onesweep  one launch per radix pass (8-bit digits, only the
//               ceil(log2(sum rows)) key bits are sorted): a tile takes a
//               ticket in launch order, ranks its keys stably (wave ballots
//               find equal digits, per-wave LDS counters order them), looks
//               back over earlier tiles' published digit counts for its
//               offsets, and scatters key + payload
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
constexpr int kSortWaves = 4;
constexpr int kRleItems = 4;
constexpr int kRleTile = 256 * kRleItems;
constexpr uint32_t kFlagAgg = 1u << 30;
constexpr uint32_t kFlagInc = 2u << 30;
constexpr uint32_t kValMask = (1u << 30) - 1u;
constexpr uint32_t kSpinLimit = 1u << 24;
constexpr int kPrepMaxBags = 2048;   // bags per k_prep block (LDS offsets cache)
constexpr int kPrepKeys = 1024;      // target keys per k_prep block

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int sort_rounds(int64_t N) { return N > (int64_t(1) << 21) ? 16 : 8; }
}  // namespace

BwdLayout bwd_layout(const tbe_plan* p, int32_t B, int64_t N)
{
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
    const int64_t total_bags = int64_t(p->T) * B;
    int64_t pb = (N + kPrepKeys - 1) / kPrepKeys;   // ~kPrepKeys keys per k_prep block
    if (pb > 1024) pb = 1024;
    const int64_t need = (total_bags + kPrepMaxBags - 1) / kPrepMaxBags;
    if (pb < need) pb = need;
    if (pb > total_bags) pb = total_bags;
    if (pb < 1) pb = 1;
    L.prep_blocks = static_cast<int32_t>(pb);
    L.prep_bags = static_cast<int32_t>((total_bags + pb - 1) / pb);
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
    L.off_status = take(size_t(L.npasses) * kRadix * (L.sort_blocks > 0 ? L.sort_blocks : 1) * 4);
    L.off_rle_status = take(size_t(3) * (L.rle_blocks > 0 ? L.rle_blocks : 1) * 4);
    L.status_words = (L.off_rle_status - L.off_status) / 4 +
                     size_t(3) * (L.rle_blocks > 0 ? L.rle_blocks : 1);
    L.off_unique = take(n4);
    L.off_run_start = take(n4);
    L.off_run_len = take(n4);
    L.off_short = take(n4);
    L.off_long = take(n4);
    L.off_short_info = take(size_t(N + 1) * 16);
    L.off_long_info = take(size_t(ml + 1) * 16);
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
    st_rel(st + static_cast<size_t>(tile) * stride, kFlagAgg | value);
    uint32_t excl = 0;
    int64_t tp = static_cast<int64_t>(tile) - 1;
    uint32_t spins = 0;
    while (true) {
        uint32_t s[W];
#pragma unroll
        for (int i = 0; i < W; ++i)
            s[i] = (tp - i >= 0) ? ld_acq(st + static_cast<size_t>(tp - i) * stride) : kFlagInc;
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
                atomicOr(err, 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
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

// Add 1 per active lane to hist[d]: lanes with equal digits are found with
// nbits ballots and the lowest of them adds their count, so a hot digit (Zipf
// keys) costs one LDS atomic per wavefront instead of one per lane.
__device__ __forceinline__ void wave_hist_add(uint32_t* hist, uint32_t d, bool ok, int nbits,
                                              uint64_t lt)
{
    uint64_t peers = __ballot(ok);
    for (int bit = 0; bit < nbits; ++bit) {
        const bool on = (d >> bit) & 1u;
        const uint64_t bal = __ballot(on);
        peers &= on ? bal : ~bal;
    }
    if (ok && (peers & lt) == 0) atomicAdd(&hist[d], static_cast<uint32_t>(__popcll(peers)));
}

// Payload carried through the sort next to each key.
enum PayloadMode : int {
    kPayloadPos = 0,      // lookup position j (the sort_rle entry point)
    kPayloadSample = 1,   // sample id b of the lookup's bag
    kPayloadSampleW = 2,  // (b, per-sample weight bits) pair
};

template <typename IT, int MODE>
__global__ __launch_bounds__(256) void k_prep(
    const TableDesc* __restrict__ tables, uint32_t B, uint32_t total_bags, uint32_t bags_per_block,
    const IT* __restrict__ indices, const IT* __restrict__ offsets,
    const float* __restrict__ psw, uint32_t* __restrict__ keys, void* __restrict__ vals,
    uint32_t* __restrict__ totals, PassBits pb, uint32_t* __restrict__ status,
    size_t status_words)
{
    __shared__ uint32_t hist[4][kRadix];
    __shared__ int64_t boff[kPrepMaxBags + 1];
    __shared__ uint32_t hoff[kPrepMaxBags + 1];   // first key of each table the block touches
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (size_t i = blockIdx.x * 256ull + tid; i < status_words; i += gridDim.x * 256ull)
        status[i] = 0u;
    for (int i = tid; i < 4 * kRadix; i += 256) (&hist[0][0])[i] = 0u;
    const uint32_t g0 = blockIdx.x * bags_per_block;
    const uint32_t nb = g0 < total_bags ? min(bags_per_block, total_bags - g0) : 0u;
    const uint32_t t_first = nb ? g0 / B : 0;
    const uint32_t t_count = nb ? (g0 + nb - 1) / B - t_first + 1 : 0;   // <= nb
    for (uint32_t i = tid; i <= nb && nb > 0; i += 256) boff[i] = static_cast<int64_t>(offsets[g0 + i]);
    for (uint32_t i = tid; i < t_count; i += 256) hoff[i] = tables[t_first + i].hash_off;
    __syncthreads();
    const int64_t P0 = nb ? boff[0] : 0, P1 = nb ? boff[nb] : 0;
    constexpr int UN = 8;
    for (int64_t base = P0; base < P1; base += 256 * UN) {
        IT id[UN];
        float wv[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int64_t p = base + u * 256 + tid;
            id[u] = p < P1 ? indices[p] : IT(0);
            wv[u] = (MODE == kPayloadSampleW && p < P1) ? psw[p] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int64_t p = base + u * 256 + tid;
            const bool ok = p < P1;
            uint32_t key = 0;
            if (ok) {
                uint32_t lo = 0, hi = nb;  // boff[lo] <= p < boff[hi]
                while (hi - lo > 1) {
                    const uint32_t mid = (lo + hi) >> 1;
                    if (boff[mid] <= p) lo = mid; else hi = mid;
                }
                const uint32_t g = g0 + lo;
                const uint32_t t = g / B;
                key = hoff[t - t_first] + static_cast<uint32_t>(id[u]);
                keys[p] = key;
                const uint32_t b = g - t * B;
                if (MODE == kPayloadPos)
                    static_cast<uint32_t*>(vals)[p] = static_cast<uint32_t>(p);
                else if (MODE == kPayloadSample)
                    static_cast<uint32_t*>(vals)[p] = b;
                else
                    static_cast<uint2*>(vals)[p] = make_uint2(b, __float_as_uint(wv[u]));
            }
            for (int q = 0; q < pb.npasses; ++q)
                wave_hist_add(hist[q], (key >> pb.shift[q]) & pb.mask[q], ok, pb.bits[q], lt);
        }
    }
    __syncthreads();
    // digit totals are spread over kTotCopies copies (fewer adds per address)
    uint32_t* tcopy = totals + (blockIdx.x % kTotCopies) * (4 * kRadix);
    for (int q = 0; q < pb.npasses; ++q) {
        const uint32_t c = hist[q][tid];
        if (c) atomicAdd(&tcopy[q * kRadix + tid], c);
    }
}

// ---------------------------------------------------------------------------
template <int R, typename PT>
__global__ __launch_bounds__(256) void k_onesweep(
    const uint32_t* __restrict__ keys_in, const PT* __restrict__ vals_in,
    uint32_t* __restrict__ keys_out, PT* __restrict__ vals_out, uint32_t N, int shift,
    int nbits, const uint32_t* __restrict__ totals, uint32_t* __restrict__ status,
    uint32_t* __restrict__ ticket, uint32_t* __restrict__ err, uint32_t ntiles,
    uint32_t* __restrict__ prev_totals)
{
    __shared__ uint32_t wcnt[kSortWaves][kRadix];
    __shared__ uint32_t gofs[kRadix];
    __shared__ uint32_t wsum[kSortWaves];
    __shared__ uint32_t s_tile;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    if (tid == 0) s_tile = take_ticket(ticket, ntiles);
    for (int i = tid; i < kSortWaves * kRadix; i += 256) (&wcnt[0][0])[i] = 0u;
    // exclusive scan of the global digit totals: first position of each digit
    {
        uint32_t v = 0;
#pragma unroll
        for (int cp = 0; cp < kTotCopies; ++cp) v += totals[cp * 4 * kRadix + tid];
        const uint32_t inc = wave_incl_scan(v, lane);
        if (lane == 63) wsum[wave] = inc;
        __syncthreads();
        uint32_t pre = 0;
        for (int w = 0; w < wave; ++w) pre += wsum[w];
        gofs[tid] = pre + inc - v;
    }
    __syncthreads();
    const uint32_t tile = s_tile;
    if (tile >= ntiles) {          // only with an uninitialised control block
        if (tid == 0) atomicOr(err, 2u);
        return;
    }
    // the previous pass's digit totals are no longer needed: leave them zero
    if (tile == 0 && prev_totals)
#pragma unroll
        for (int cp = 0; cp < kTotCopies; ++cp) prev_totals[cp * 4 * kRadix + tid] = 0u;

    const uint32_t mask = (1u << nbits) - 1u;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const uint32_t wbase = tile * (256u * R) + static_cast<uint32_t>(wave) * (64u * R);
    uint32_t k[R], dg[R], rk[R];
    PT v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t i = wbase + r * 64u + lane;
        const bool ok = i < N;
        k[r] = ok ? keys_in[i] : 0u;
        if (ok) v[r] = vals_in[i];
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
        const int d = tid;
        uint32_t run = 0;
#pragma unroll
        for (int w = 0; w < kSortWaves; ++w) {
            const uint32_t c = wcnt[w][d];
            wcnt[w][d] = run;
            run += c;
        }
        const uint32_t excl = lookback<16>(status + d, kRadix, tile, run, err);
        gofs[d] += excl;
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

__device__ __forceinline__ int find_table_g(const uint32_t* __restrict__ hash_off, int T,
                                            uint32_t key)
{
    int lo = 0, hi = T;  // hash_off[lo] <= key < hash_off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (hash_off[mid] <= key) lo = mid; else hi = mid;
    }
    return lo;
}

template <bool API>
__global__ __launch_bounds__(256) void k_rle(
    const uint32_t* __restrict__ keys, uint32_t N, uint32_t tau, uint32_t chunk, uint32_t ntiles,
    uint32_t* __restrict__ rstatus, uint32_t* __restrict__ ticket, uint32_t* __restrict__ err,
    const uint32_t* __restrict__ hash_off, int32_t T, uint4* __restrict__ short_info,
    uint4* __restrict__ long_info, uint32_t* __restrict__ counts,
    uint32_t max_long, uint32_t* __restrict__ prev_totals,
    uint32_t* __restrict__ unique, uint32_t* __restrict__ run_start,
    uint32_t* __restrict__ run_len, uint32_t* __restrict__ short_ids,
    uint32_t* __restrict__ long_ids)
{
    __shared__ uint32_t wsum[3][4];
    __shared__ uint32_t texcl[3];
    __shared__ uint32_t s_tile;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    if (tid == 0) s_tile = take_ticket(ticket, ntiles);
    __syncthreads();
    const uint32_t tile = s_tile;
    if (tile >= ntiles) {          // only with an uninitialised control block
        if (tid == 0) atomicOr(err, 2u);
        return;
    }
    if (tile == 0 && prev_totals)   // the last radix pass is done with its totals
#pragma unroll
        for (int cp = 0; cp < kTotCopies; ++cp) prev_totals[cp * 4 * kRadix + tid] = 0u;
    const uint32_t i0 = tile * kRleTile + tid * kRleItems;

    uint32_t kk[kRleItems], len[kRleItems];
    uint32_t v[3] = {0, 0, 0};
#pragma unroll
    for (int q = 0; q < kRleItems; ++q) {
        const uint32_t i = i0 + q;
        len[q] = 0;
        kk[q] = 0;
        if (i < N) {
            kk[q] = keys[i];
            if (i == 0 || keys[i - 1] != kk[q]) {
                len[q] = run_length(keys, N, i, kk[q]);
                v[0] += 1;
                if (len[q] >= tau) {
                    v[1] += 1;
                    v[2] += (len[q] + chunk - 1) / chunk;
                }
            }
        }
    }
    uint32_t inc[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        inc[c] = wave_incl_scan(v[c], lane);
        if (lane == 63) wsum[c][wave] = inc[c];
    }
    __syncthreads();
    if (tid < 3) {
        const uint32_t tot = wsum[tid][0] + wsum[tid][1] + wsum[tid][2] + wsum[tid][3];
        const uint32_t ex =
            lookback<32>(rstatus + static_cast<size_t>(tid) * ntiles, 1, tile, tot, err);
        texcl[tid] = ex;
        if (tile == ntiles - 1) {
            // the last tile knows the totals
            counts[tid == 0 ? 0 : (tid == 1 ? 2 : 3)] = ex + tot;
        }
    }
    __syncthreads();
    uint32_t base[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        uint32_t pre = texcl[c];
        for (int w = 0; w < wave; ++w) pre += wsum[c][w];
        base[c] = pre + inc[c] - v[c];
    }
    if (tile == ntiles - 1 && tid == 255) {
        const uint32_t R = base[0] + v[0], Lg = base[1] + v[1];
        counts[1] = R - Lg;
        if (API) run_start[R] = N;
    }
    uint32_t r = base[0], lb = base[1], cb = base[2];
#pragma unroll
    for (int q = 0; q < kRleItems; ++q) {
        if (len[q] == 0) continue;
        if (r >= N || lb > r) break;  // guards: unreachable when consistent
        const uint32_t i = i0 + q;
        const uint32_t key = kk[q];
        if (API) {
            unique[r] = key;
            run_start[r] = i;
            run_len[r] = len[q];
        }
        if (len[q] >= tau) {
            if (lb < max_long) long_info[lb] = make_uint4(key, i, len[q], cb);
            if (API) long_ids[lb] = r;
            ++lb;
            cb += (len[q] + chunk - 1) / chunk;
        } else {
            const uint32_t t = static_cast<uint32_t>(find_table_g(hash_off, T, key));
            short_info[r - lb] = make_uint4(key, i, len[q], t);
            if (API) short_ids[r - lb] = r;
        }
        ++r;
    }
}

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
    for (int pass = 0; pass < L.npasses; ++pass) {
        const int nbits = L.digit_bits[pass];
        hipLaunchKernelGGL((k_onesweep<R, PT>), dim3(nb), dim3(256), 0, a.stream, keys[cur],
                           vals[cur], keys[cur ^ 1], vals[cur ^ 1], N, shift, nbits,
                           ctl + kCtlTotals + pass * kRadix,
                           status + static_cast<size_t>(pass) * kRadix * nb,
                           ctl + kCtlTicket + pass, ctl + kCtlError, nb,
                           pass > 0 ? ctl + kCtlTotals + (pass - 1) * kRadix : nullptr);
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
    hipLaunchKernelGGL((k_prep<IT, MODE>), dim3(L.prep_blocks), dim3(256), 0, a.stream,
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
    const int mode = api_outputs ? kPayloadPos : (a.psw ? kPayloadSampleW : kPayloadSample);
    a.payload_pairs = mode == kPayloadSampleW;
    const bool i64 = p->idtype == TBE_I64;
    if (mode == kPayloadPos)
        i64 ? launch_prep<int64_t, kPayloadPos>(a, pb, total_bags)
            : launch_prep<int32_t, kPayloadPos>(a, pb, total_bags);
    else if (mode == kPayloadSample)
        i64 ? launch_prep<int64_t, kPayloadSample>(a, pb, total_bags)
            : launch_prep<int32_t, kPayloadSample>(a, pb, total_bags);
    else
        i64 ? launch_prep<int64_t, kPayloadSampleW>(a, pb, total_bags)
            : launch_prep<int32_t, kPayloadSampleW>(a, pb, total_bags);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    stage_mark(p, 1, a.stream);
    const bool big = sort_rounds(L.N) == 16;
    if (mode == kPayloadSampleW)
        e = big ? sort_passes<16, uint2>(a) : sort_passes<8, uint2>(a);
    else
        e = big ? sort_passes<16, uint32_t>(a) : sort_passes<8, uint32_t>(a);
    if (e != hipSuccess) return e;
    stage_mark(p, 2, a.stream);

    const uint32_t* skeys = reinterpret_cast<const uint32_t*>(ws + L.off_keys[a.final_buf]);
    const uint32_t tau = static_cast<uint32_t>(p->tuning.tau);
    const uint32_t chunk = static_cast<uint32_t>(p->tuning.chunk);
    const uint32_t nt = static_cast<uint32_t>(L.rle_blocks);
    auto kern = api_outputs ? k_rle<true> : k_rle<false>;
    hipLaunchKernelGGL(kern, dim3(nt), dim3(256), 0, a.stream, skeys, N, tau, chunk, nt,
                       reinterpret_cast<uint32_t*>(ws + L.off_rle_status), ctl + kCtlRleTicket,
                       ctl + kCtlError, p->d_hash_off, p->T,
                       reinterpret_cast<uint4*>(ws + L.off_short_info),
                       reinterpret_cast<uint4*>(ws + L.off_long_info), ctl + kCtlCounts,
                       static_cast<uint32_t>(L.max_long),
                       ctl + kCtlTotals + (L.npasses - 1) * kRadix,
                       reinterpret_cast<uint32_t*>(ws + L.off_unique),
                       reinterpret_cast<uint32_t*>(ws + L.off_run_start),
                       reinterpret_cast<uint32_t*>(ws + L.off_run_len),
                       reinterpret_cast<uint32_t*>(ws + L.off_short),
                       reinterpret_cast<uint32_t*>(ws + L.off_long));
    stage_mark(p, 3, a.stream);
    return hipGetLastError();
}

}  // namespace tbe

namespace tbe {
hipError_t launch_workspace_init(void* ws, hipStream_t s)
{
    hipLaunchKernelGGL(k_fill_zero, dim3(1), dim3(1024), 0, s, static_cast<uint32_t*>(ws),
                       kCtlWords);
    return hipGetLastError();
}
}  // namespace tbe
