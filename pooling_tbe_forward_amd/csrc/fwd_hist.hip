// Forward pooled sum of small tables as (id counts) x (table) on MFMA.
//
// Section "The forward: a general gather and one clever special case" of the
// FBTriton TBE article: a pooled sum is a weighted sum of table rows where the
// weight is how often each row occurs in the bag, so when the whole table
// fits in a tile the pooled output of a group of bags is a [bags, rows] x
// [rows, D] matrix product; counts are exact in fp16 while they stay small.
//
// gfx950 design:
//  * a group is 16 consecutive bags of one eligible table (rows <= 256,
//    D <= 256, fp16 weights, no per-sample weights): the M rows of one MFMA
//    tile.  Workgroups (4 wavefronts) are persistent: as many as the chip
//    holds at once, shared evenly by the launch's tables, each taking every
//    k-th group of its table, so it loads that table's B operands once;
//  * a group is a short dependent chain (offsets, ids, counts, product,
//    store), so each step's loads go out one step early: the table before
//    the first offsets, the next group's offsets while this one is counted,
//    the next group's ids while this one is multiplied and stored.  Counts
//    and group records are double-buffered (two workgroup barriers a group);
//  * ids are counted into a [16, rows] LDS histogram (dynamic LDS sized by
//    the table's rows) with LDS atomics; ids out of range and lanes past the
//    end add to a discard word of their own, so the adds need no branch and
//    never pile onto one address.  A group's ids are one contiguous range of
//    the index array, loaded 16 per thread at once; an id's bag comes from
//    two wave ballots over the bag starts (a wave's 64 positions are
//    contiguous), not from a per-lane search;
//  * v_mfma_f32_16x16x16_f16 multiplies the counts (converted to fp16, exact
//    because a window holds at most 2048 ids of a bag) by the table.  A
//    lane's A operand (4 counts of one bag) is one 16-byte LDS read shared by
//    the wave's tiles; its B operand is 4 rows of one column of the table:
//      - small tables (at most 8 B operands per lane: rows <= 64 and D <= 128,
//        or rows <= 128 and D <= 64) keep their B operands in registers;
//      - larger ones are copied to LDS transposed (each column's rows
//        contiguous, at most 36864 halves) so a B operand is one 8-byte read;
//        beyond that they are read from global memory;
//    each wavefront owns 16-column output tiles and walks the rows in steps
//    of 16;
//  * bags longer than one window repeat count + multiply and keep
//    accumulating in the fp32 MFMA accumulators, so every id goes through the
//    matrix unit (no scalar tail).
#include "tbe_internal.h"

namespace tbe {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;                               // MFMA M = N = K
constexpr int kMaxTilesPerWave = kHistMaxD / kTile / 4;  // 256 columns over 4 waves
constexpr int kFlatIds = kHistBags * 256 / 256;   // ids per thread per chunk (16 bags x 256)
constexpr int kStageElems = 36864;   // transposed tables up to this many halves are staged in LDS
constexpr int kStageBatch = 4;       // 16-byte staging loads per thread in flight
constexpr int kRegFrags = 8;         // B operands a lane may hold in registers
static_assert(kHistBags == kTile, "a workgroup's bags are the M rows of one MFMA tile");

struct HistTables {
    int32_t n;
    int32_t t[16];
};

// Row stride (words) of the [16 bags][rows] count matrix: rows rounded up to
// the MFMA depth (the last k step reads up to there; those counts stay zero),
// plus 4, so the 16-byte A reads of 16 bags spread over the LDS banks.
__host__ __device__ inline int count_stride(int R) { return ((R + 15) & ~15) + 4; }
// Column stride (halves) of the transposed staged table: rows rounded up to 16
// plus 4 (4 mod 8 halves), so the 8-byte B reads of 16 consecutive columns
// fall in 16 different bank pairs.
__host__ __device__ inline int stage_stride(int R) { return ((R + 15) & ~15) + 4; }

// A value every lane holds the same copy of, moved to scalar registers.
__device__ inline int64_t uni64(int64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi =
        __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Per-group record written by wave 0: bag starts and ends, starts relative to
// the first (bags past the group's end start "at infinity", so no bag search
// counts them) and the longest bag's length.
struct GroupInfo {
    int64_t s[kHistBags];
    int64_t e[kHistBags];
    uint32_t rel[kHistBags];
    int32_t max_len;
    int32_t pad;
};

// KS > 0: B operands in registers, KS k steps (rows <= 16 KS) and TPW tiles
// per wave (D <= 64 TPW).  KS == 0: B operands from the LDS copy of the table
// (when stage_elems allows) or from global memory.
//
// Persistent: the blocks of a table (blocks_per_table of them, at most its
// number of groups) take its groups q, q + blocks_per_table, ..., so a block
// loads its table's B operands (or LDS copy) once.  While a group is counted,
// the next group's offsets are in flight; once it is counted, the next
// group's ids are issued, and stay in flight through the current group's
// product and stores.  Counts and group records are double-buffered, so a
// group costs two workgroup barriers.
template <typename IT, int KS, int TPW>
__global__ __launch_bounds__(256, KS > 0 ? 4 : 1) void k_fwd_hist(
    const TableDesc* __restrict__ tables, HistTables list, uint32_t B, uint32_t groups_per_table,
    int32_t sumD, const _Float16* __restrict__ weights, const IT* __restrict__ indices,
    const IT* __restrict__ offsets, float* __restrict__ out, int32_t stage_elems,
    int32_t cnt_off, int32_t cnt_buf_words, uint32_t blocks_per_table, int32_t mean)
{
    static_assert(KS * TPW <= kRegFrags && TPW <= kMaxTilesPerWave, "register B operands");
    constexpr int kTpw = KS > 0 ? TPW : kMaxTilesPerWave;   // accumulator tiles per wave
    // dynamic LDS: [stage_elems] fp16 staged table, then at byte cnt_off two
    // buffers of cnt_buf_words words: [kHistBags][count_stride(rows)] uint32
    // counts and 64 discard words
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
    _Float16* __restrict__ stab = reinterpret_cast<_Float16*>(dyn);
    uint32_t* __restrict__ cnt_base = reinterpret_cast<uint32_t*>(dyn + cnt_off);
    __shared__ GroupInfo info[2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int frag_row = lane & 15;        // A: bag row of this lane; B: output column
    const int frag_k = (lane >> 4) * 4;    // first of the 4 k values this lane holds
    // this block's table, and its first group of that table
    const uint32_t h = blockIdx.x / blocks_per_table;
    const int t = list.t[h];
    const TableDesc d = tables[t];

    // group (of this table) -> first bag, bag count, first offset index
    struct Grp {
        uint32_t b0;
        int nb;
        uint32_t g0;
    };
    auto group = [&](uint32_t q) {
        Grp r;
        r.b0 = q * kHistBags;
        r.nb = static_cast<int>(min(static_cast<uint32_t>(kHistBags), B - r.b0));
        r.g0 = static_cast<uint32_t>(t) * B + r.b0;
        return r;
    };
    // offsets i <= nb of a group (bag i spans [off_i, off_{i+1})); every wave
    // reads them (one cache line), wave 0 turns them into the group record
    auto read_offsets = [&](const Grp& g) { return offsets[g.g0 + min(lane, g.nb)]; };
    auto write_info = [&](IT oraw, const Grp& g, GroupInfo& gi) {
        const int64_t o = static_cast<int64_t>(oraw);
        const int64_t o1 = __shfl_down(o, 1);
        const bool bag = lane < g.nb;
        int32_t len = bag ? static_cast<int32_t>(o1 - o) : 0;
        const int64_t o0 = __shfl(o, 0);
        if (lane < kHistBags) {
            gi.s[lane] = bag ? o : 0;
            gi.e[lane] = bag ? o1 : 0;
            gi.rel[lane] = bag ? static_cast<uint32_t>(o - o0) : 0xFFFFFFFFu;
        }
#pragma unroll
        for (int m = 32; m > 0; m >>= 1) len = max(len, __shfl_xor(len, m));
        if (lane == 0) gi.max_len = len;
    };

    uint32_t qidx = blockIdx.x - h * blocks_per_table;
    Grp cur = group(qidx);
    IT oraw = read_offsets(cur);

    // Table loads, which do not depend on the offsets, go out behind them
    // (loads complete in order, so wave 0 can use the offsets while these are
    // in flight).  Register path: this lane's B operands, raw halves whose
    // addresses are clamped into the table (rows past R are zeroed when used).
    // LDS path: the first kStageBatch 16-byte pieces of the copy per thread.
    half4_t braw[KS > 0 ? TPW : 1][KS > 0 ? KS : 1];
    u32x4 tv[kStageBatch];
    auto load_b = [&](const TableDesc& td) {
        const _Float16* __restrict__ tb = weights + td.w_off;
        const int R = static_cast<int>(td.rows), D = td.D;
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int col = min((wave + 4 * m) * kTile + frag_row, D - 1);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int k = min(ks * kTile + frag_k + j, R - 1);
                    braw[m][ks][j] = tb[k * D + col];
                }
        }
    };
    // the LDS copy of a table: [D][kp] fp16 (rows of a column contiguous, pad
    // rows zero), so a lane's 4 k values of one column are one 8-byte read;
    // `first`: the first batch of loads is already in tv
    auto stage = [&](const TableDesc& td, bool first) {
        const _Float16* __restrict__ tb = weights + td.w_off;
        const int R = static_cast<int>(td.rows), D = td.D, kp = stage_stride(R);
        const int n8 = (R * D) / 8, rem = (R * D) % 8;
        auto put = [&](int e, const _Float16* v, int n) {
            int k = e / D, c = e - k * D;
            for (int j = 0; j < n; ++j) {
                stab[c * kp + k] = v[j];
                if (++c == D) { c = 0; ++k; }
            }
        };
        if ((reinterpret_cast<uintptr_t>(tb) & 15) == 0) {
            // kStageBatch loads per thread are in flight before any is stored
            for (int i0 = 0; i0 < n8; i0 += 256 * kStageBatch) {
                if (i0 || !first) {
#pragma unroll
                    for (int u = 0; u < kStageBatch; ++u) {
                        const int i = i0 + u * 256 + tid;
                        tv[u] = reinterpret_cast<const u32x4*>(tb)[i < n8 ? i : n8 - 1];
                    }
                }
#pragma unroll
                for (int u = 0; u < kStageBatch; ++u) {
                    // keeps the compiler from unpacking the halves (and so
                    // waiting for the loads) ahead of the offsets step
                    asm volatile("" : "+v"(tv[u]));
                    const int i = i0 + u * 256 + tid;
                    if (i < n8) put(8 * i, reinterpret_cast<const _Float16*>(&tv[u]), 8);
                }
            }
            for (int e = n8 * 8 + tid; e < n8 * 8 + rem; e += 256) put(e, tb + e, 1);
        } else {
#pragma unroll 1
            for (int e = tid; e < R * D; e += 256) put(e, tb + e, 1);
        }
        // rows R .. (R rounded up to 16) of every column are read by the last
        // k step: zero, so they add nothing (their counts are zero too)
        const int kz = ((R + kTile - 1) & ~(kTile - 1)) - R;
        for (int i = tid; i < kz * D; i += 256) {
            const int c = i / kz;
            stab[c * kp + R + (i - c * kz)] = static_cast<_Float16>(0.f);
        }
    };
    auto is_staged = [&](const TableDesc& td) {
        return KS == 0 && td.D * stage_stride(static_cast<int>(td.rows)) <= stage_elems;
    };
    const bool staged = is_staged(d);
    if constexpr (KS > 0) {
        load_b(d);
    } else {
        // (unconditional, so the wait below can leave them in flight: a block
        // that copies nothing reads the first descriptor instead, and drops it)
        const _Float16* __restrict__ tb = weights + d.w_off;
        const int n8 = (static_cast<int>(d.rows) * d.D) / 8;
        const bool pre = staged && (reinterpret_cast<uintptr_t>(tb) & 15) == 0 && n8 > 0;
        const u32x4* __restrict__ src =
            pre ? reinterpret_cast<const u32x4*>(tb) : reinterpret_cast<const u32x4*>(tables);
        const int lim = pre ? n8 - 1 : 0;
#pragma unroll
        for (int u = 0; u < kStageBatch; ++u) tv[u] = src[min(u * 256 + tid, lim)];
    }

    // the offsets are used only here, behind the table loads
    asm volatile("" : "+v"(oraw));
    if (wave == 0) write_info(oraw, cur, info[0]);
    __syncthreads();

    // The bags of a group are consecutive in the index array.  When each fits
    // one window, the group's ids are one contiguous range [P0, P0 + len):
    // every thread loads kFlatIds of them at once (coalesced, all in flight)
    // and finds each id's bag by a branch-free search over the bag starts.
    // Positions past the end re-read the last id and are dropped when
    // counted; a group with no ids (or not flat) reads its own first offset
    // instead (a valid address).  The first 256 x kFlatIds are loaded with no
    // branch (so the waits before the counting step can leave them in
    // flight); later ones skip steps wholly past the end.
    IT id[kFlatIds];
    uint32_t len = 0;
    const IT* __restrict__ ids = offsets;
    auto ids_of = [&](const Grp& g, const GroupInfo& gi) {
        const bool flat = gi.max_len <= kHistWindow;
        const int64_t P0 = uni64(gi.s[0]);
        len = flat ? static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
                         static_cast<int32_t>(gi.e[g.nb - 1] - P0)))   // <= 16 * 2048
                   : 0u;
        ids = len > 0 ? indices + P0 : offsets + g.g0;
    };
    auto load_ids = [&](uint32_t base, bool skip) {
        const uint32_t last = len > 0 ? len - 1 : 0;
#pragma unroll
        for (int u = 0; u < kFlatIds; ++u) {
            if (skip && base + u * 256 >= len) break;   // wave-uniform
            const uint32_t rp = min(base + u * 256 + tid, last);
            id[u] = *reinterpret_cast<const IT*>(reinterpret_cast<const char*>(ids) +
                                                 rp * static_cast<uint32_t>(sizeof(IT)));
        }
    };
    ids_of(cur, info[0]);
    load_ids(0, false);
    if (staged) stage(d, true);
    for (int i = tid; i < cnt_buf_words; i += 256) cnt_base[i] = 0u;

    int buf = 0;
    for (;;) {
        __syncthreads();   // counts zeroed, group record and staged table visible
        const GroupInfo& gi = info[buf];
        uint32_t* __restrict__ cnt = cnt_base + buf * cnt_buf_words;
        const int R = static_cast<int>(d.rows);
        const int D = d.D;
        const int cs = count_stride(R);
        const int sink = kHistBags * cs + lane;   // per-lane discard word
        const int ntiles = (D + kTile - 1) / kTile;
        const int ksteps = (R + kTile - 1) / kTile;
        const _Float16* __restrict__ tb = weights + d.w_off;
        const int kp = stage_stride(R);

        // the next group's offsets go out now and land during the counting
        const uint32_t nidx = qidx + blocks_per_table;
        const bool has_next = nidx < groups_per_table;
        const Grp nxt = group(has_next ? nidx : qidx);
        IT onext = read_offsets(nxt);

        floatx4 acc[kTpw];
#pragma unroll
        for (int m = 0; m < kTpw; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[m][v] = 0.f;
        // A: the lane's 4 counts (one 16-byte read, exact in fp16), shared by
        // the wave's tiles; B: registers, the LDS copy or global memory
        auto product = [&]() {
            auto a_frag = [&](int ks) {
                const u32x4 c4 =
                    *reinterpret_cast<const u32x4*>(&cnt[frag_row * cs + ks * kTile + frag_k]);
                half4_t a;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    a[j] = static_cast<_Float16>(static_cast<uint16_t>(c4[j]));
                return a;
            };
            if constexpr (KS > 0) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const half4_t a = a_frag(ks);
#pragma unroll
                    for (int m = 0; m < TPW; ++m) {
                        if (wave + 4 * m >= ntiles) continue;
                        // the loads are waited for here, not where they were issued
                        half4_t bf = braw[m][ks];
                        asm volatile("" : "+v"(bf));
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (ks * kTile + frag_k + j >= R) bf[j] = static_cast<_Float16>(0.f);
                        acc[m] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, bf, acc[m], 0, 0, 0);
                    }
                }
            } else if (staged) {
                for (int ks = 0; ks < ksteps; ++ks) {
                    const half4_t a = a_frag(ks);
#pragma unroll
                    for (int m = 0; m < kTpw; ++m) {
                        const int nt = wave + 4 * m;
                        if (nt >= ntiles) continue;
                        const int col = nt * kTile + frag_row;
                        const half4_t bf =
                            col < D ? *reinterpret_cast<const half4_t*>(
                                          &stab[col * kp + ks * kTile + frag_k])
                                    : half4_t{0, 0, 0, 0};
                        acc[m] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, bf, acc[m], 0, 0, 0);
                    }
                }
            } else {
                for (int ks = 0; ks < ksteps; ++ks) {
                    const half4_t a = a_frag(ks);
#pragma unroll 1
                    for (int m = 0; m < kTpw; ++m) {
                        const int nt = wave + 4 * m;
                        if (nt >= ntiles) break;
                        const int col = nt * kTile + frag_row;
                        half4_t bf;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int k = ks * kTile + frag_k + j;
                            bf[j] = k < R && col < D ? tb[static_cast<int64_t>(k) * D + col]
                                                     : static_cast<_Float16>(0.f);
                        }
                        acc[m] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, bf, acc[m], 0, 0, 0);
                    }
                }
            }
        };

        if (len > 0 || gi.max_len == 0) {
            // one window: the ids in registers (none for a group of empty bags)
            // this wave's copy of the bag starts: lane i < 16 holds bag i's
            const uint32_t rel_l = lane < kHistBags ? gi.rel[lane] : 0xFFFFFFFFu;
            for (uint32_t base = 0; base < len; base += 256 * kFlatIds) {
                if (base) load_ids(base, true);
                // A wave's 64 positions of a step are contiguous: the bag of
                // position rp (the last bag whose start is at or before it;
                // that bag is not empty) is the number of bag starts at or
                // before the span's first position, less one (one ballot),
                // plus the bag starts inside the span at or before rp (a
                // scan over those few, usually none or one).  Positions past
                // the end and ids out of range add to the lane's own word
                // past the counts (no two lanes share it, so they do not
                // serialize, and no product reads it).
#pragma unroll
                for (int u = 0; u < kFlatIds; ++u) {
                    if (base + u * 256 >= len) break;   // wave-uniform
                    const uint32_t p0 = base + u * 256 + wave * 64;
                    const uint32_t rp = p0 + lane;
                    int g = __popcll(__ballot(rel_l <= p0)) - 1;
                    const int gl = __popcll(__ballot(rel_l <= p0 + 63)) - 1;
                    for (int i = g + 1; i <= gl; ++i)
                        g += rp >= static_cast<uint32_t>(__builtin_amdgcn_readlane(
                                        static_cast<int>(rel_l), i))
                                 ? 1
                                 : 0;
                    const IT v = id[u];
                    const bool ok = rp < len && v >= 0 && v < R;
                    atomicAdd(&cnt[ok ? g * cs + static_cast<int>(v) : sink], 1u);
                }
            }
        } else {
            // Bags longer than one window: count + multiply per window, each
            // wave walking its bags' ids of the window.  Every window but the
            // last is multiplied here; the last one below.
            const int nwin = (gi.max_len + kHistWindow - 1) / kHistWindow;
            for (int win = 0; win < nwin; ++win) {
                for (int i = wave; i < cur.nb; i += 4) {
                    const int64_t s0 = gi.s[i] + static_cast<int64_t>(win) * kHistWindow;
                    const int64_t e0 = min(gi.e[i], s0 + kHistWindow);
                    for (int64_t p = s0 + lane; p < e0; p += 64) {
                        const int64_t v = static_cast<int64_t>(indices[p]);
                        if (v >= 0 && v < R) atomicAdd(&cnt[i * cs + v], 1u);
                    }
                }
                if (win + 1 < nwin) {
                    __syncthreads();
                    product();
                    __syncthreads();
                    for (int i = tid; i < kHistBags * cs; i += 256) cnt[i] = 0u;
                    __syncthreads();
                }
            }
        }
        if (has_next && wave == 0) {
            asm volatile("" : "+v"(onext));
            write_info(onext, nxt, info[buf ^ 1]);
        }
        __syncthreads();   // counts complete, the next group's record visible

        // the next group's ids go out now and stay in flight through this
        // group's product and stores
        if (has_next) {
            ids_of(nxt, info[buf ^ 1]);
            load_ids(0, false);
        }
        product();
        // the other count buffer was last read by the previous group's
        // product, which every wave finished before the barrier above
        uint32_t* __restrict__ cnt_other = cnt_base + (buf ^ 1) * cnt_buf_words;
        for (int i = tid; i < cnt_buf_words; i += 256) cnt_other[i] = 0u;

        // C layout of the 16x16 tile: lane l, register v -> row 4*(l/16) + v, column l%16
#pragma unroll
        for (int m = 0; m < kTpw; ++m) {
            const int nt = wave + 4 * m;
            const int col = nt * kTile + frag_row;
            if (nt >= ntiles || col >= D) continue;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = 4 * (lane >> 4) + v;
                float val = acc[m][v];
                if (mean) {   // one rounding of sum / length; an empty bag stays 0
                    const int64_t len = gi.e[row] - gi.s[row];
                    if (len > 0) val = val / static_cast<float>(len);
                }
                if (row < cur.nb)
                    out[static_cast<int64_t>(cur.b0 + row) * sumD + d.out_off + col] = val;
            }
        }
        if (!has_next) break;
        cur = nxt;
        qidx = nidx;
        buf ^= 1;
    }
}

// Workgroups of one launch: every group when there are fewer than the chip
// holds at once (a workgroup then takes one group), else as many as are
// resident (each takes several).  One cached occupancy per kernel and LDS size.
template <auto Kernel>
uint32_t resident_blocks(size_t lds)
{
    thread_local size_t c_lds = ~size_t(0);
    thread_local int c_val = 0;
    if (c_lds != lds) {
        int dev = 0, cus = 0, per = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, Kernel, 256, lds) != hipSuccess ||
            cus <= 0 || per <= 0)
            return 2048;
        c_lds = lds;
        c_val = cus * per;
    }
    return static_cast<uint32_t>(c_val);
}

template <typename IT, int KS, int TPW>
void launch_one(size_t lds, const tbe_plan* p, const HistTables& list, uint32_t B, uint32_t gpt,
                const FwdArgs& a, int32_t stage, int32_t cnt_off, int32_t cnt_buf_words)
{
    constexpr auto k = k_fwd_hist<IT, KS, TPW>;
    // the resident blocks, shared evenly by the launch's tables (each block
    // stays on one table), at most one block per group
    const uint32_t n = static_cast<uint32_t>(list.n);
    const uint32_t bpt = max(1u, min(gpt, (resident_blocks<k>(lds) + n - 1) / n));
    hipLaunchKernelGGL(k, dim3(bpt * n), dim3(256), lds, a.stream, p->d_tables, list, B, gpt,
                       p->sum_D, static_cast<const _Float16*>(a.weights),
                       static_cast<const IT*>(a.indices), static_cast<const IT*>(a.offsets), a.out,
                       stage, cnt_off, cnt_buf_words, bpt, a.mean ? 1 : 0);
}

// Register-operand shape (k steps, tiles per wave) for a launch whose tables
// have at most maxR rows and maxD columns, or {0, 0} for the LDS/global path.
void reg_shape(int maxR, int maxD, int& ks, int& tpw)
{
    ks = (maxR + kTile - 1) / kTile;
    ks = ks <= 1 ? 1 : ks <= 2 ? 2 : ks <= 4 ? 4 : ks <= 8 ? 8 : 0;
    tpw = ((maxD + kTile - 1) / kTile + 3) / 4;
    tpw = tpw <= 1 ? 1 : tpw <= 2 ? 2 : 0;
    if (ks == 0 || tpw == 0 || ks * tpw > kRegFrags) ks = tpw = 0;
}

template <typename IT, typename... Args>
void dispatch(int ks, int tpw, Args... args)
{
    switch (ks * 10 + tpw) {
    case 11: launch_one<IT, 1, 1>(args...); break;
    case 21: launch_one<IT, 2, 1>(args...); break;
    case 41: launch_one<IT, 4, 1>(args...); break;
    case 81: launch_one<IT, 8, 1>(args...); break;
    case 12: launch_one<IT, 1, 2>(args...); break;
    case 22: launch_one<IT, 2, 2>(args...); break;
    case 42: launch_one<IT, 4, 2>(args...); break;
    default: launch_one<IT, 0, 1>(args...); break;
    }
}

}  // namespace

hipError_t launch_fwd_hist(const FwdArgs& a)
{
    const tbe_plan* p = a.plan;
    HistTables list{};
    const uint32_t gpt = (static_cast<uint32_t>(a.B) + kHistBags - 1) / kHistBags;
    auto flush = [&]() -> hipError_t {
        if (list.n == 0) return hipSuccess;
        // Path and LDS for the largest tables of the launch: registers when
        // every B operand of a lane fits; else the LDS copy when every table's
        // transposed copy fits; then two count buffers sized for the table
        // with the most rows.
        int32_t stage = 0, cnt_buf_words = 0, maxR = 0, maxD = 0;
        for (int i = 0; i < list.n; ++i) {
            const TableDesc& d = p->h_tables[list.t[i]];
            maxR = max(maxR, static_cast<int32_t>(d.rows));
            maxD = max(maxD, d.D);
            stage = max(stage, d.D * stage_stride(static_cast<int>(d.rows)));
            cnt_buf_words = max(cnt_buf_words, kHistBags * count_stride(static_cast<int>(d.rows)) + 64);
        }
        int ks, tpw;
        reg_shape(maxR, maxD, ks, tpw);
        if (ks > 0 || stage > kStageElems) stage = 0;
        const int32_t cnt_off = (stage * static_cast<int32_t>(sizeof(_Float16)) + 15) & ~15;
        const size_t lds = static_cast<size_t>(cnt_off) + 2 * sizeof(uint32_t) * cnt_buf_words;
        const uint32_t B = static_cast<uint32_t>(a.B);
        if (p->idtype == TBE_I64)
            dispatch<int64_t>(ks, tpw, lds, p, list, B, gpt, a, stage, cnt_off, cnt_buf_words);
        else
            dispatch<int32_t>(ks, tpw, lds, p, list, B, gpt, a, stage, cnt_off, cnt_buf_words);
        list.n = 0;
        return hipGetLastError();
    };
    for (int t = 0; t < p->T; ++t) {
        const TableDesc& d = p->h_tables[t];
        if (!(d.flags & TD_HIST_OK)) continue;
        if (a.psw && (d.flags & TD_WEIGHTED)) continue;
        list.t[list.n++] = t;
        if (list.n == 16) {
            hipError_t e = flush();
            if (e != hipSuccess) return e;
        }
    }
    return flush();
}

}  // namespace tbe
