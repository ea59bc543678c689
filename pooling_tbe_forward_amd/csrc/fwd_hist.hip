// Forward pooled sum of small tables as (id counts) x (table) on MFMA.
//
// Section "The forward: a general gather and one clever special case" of the
// FBTriton TBE article: a pooled sum is a weighted sum of table rows where the
// weight is how often each row occurs in the bag, so when the whole table
// fits in a tile the pooled output of a group of bags is a [bags, rows] x
// [rows, D] matrix product; counts are exact in fp16 while they stay small.
//
// gfx950 design:
//  * one workgroup (4 wavefronts) owns 32 consecutive bags of one eligible
//    table (rows <= 256, D <= 256, fp16 weights, no per-sample weights);
//  * ids are counted into a [32, rows] LDS histogram with LDS atomics; the
//    block's ids are loaded many per thread at once (a block's bags are
//    consecutive in the index array);
//  * v_mfma_f32_32x32x8_f16 multiplies the counts (converted to fp16, exact
//    because a window holds at most 2048 ids of a bag) by the table (copied
//    to LDS once per block when it holds at most 32768 elements); each
//    wavefront owns 32-column output tiles and walks the rows in steps of 8;
//  * bags longer than one window repeat count + multiply and keep
//    accumulating in the fp32 MFMA accumulators, so every id goes through the
//    matrix unit (no scalar tail).
#include "tbe_internal.h"

namespace tbe {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kMaxTilesPerWave = kHistMaxD / 32 / 4;   // 256 columns over 4 waves
constexpr int kFlatIds = 32;   // ids per thread loaded together (contiguous-range counting)
constexpr int kStageElems = 32768;   // tables up to this many elements are staged in LDS
constexpr int kStageBatch = 4;       // 16-byte staging loads per thread in flight

struct HistTables {
    int32_t n;
    int32_t t[16];
};

template <typename IT>
__global__ __launch_bounds__(256) void k_fwd_hist(
    const TableDesc* __restrict__ tables, HistTables list, uint32_t B, uint32_t groups_per_table,
    int32_t sumD, const _Float16* __restrict__ weights, const IT* __restrict__ indices,
    const IT* __restrict__ offsets, float* __restrict__ out, int32_t stage_elems)
{
    // row stride kHistMaxRows + 1: the MFMA A operand reads one k of 32 bags
    // at once, which would all fall in one LDS bank with a stride of 256
    __shared__ uint32_t cnt[kHistBags][kHistMaxRows + 1];
    __shared__ int64_t bag_s[kHistBags];
    __shared__ int64_t bag_e[kHistBags];
    extern __shared__ __attribute__((aligned(16))) _Float16 stab[];   // staged table
    __shared__ uint32_t bag_rel[kHistBags];   // bag starts relative to the first
    __shared__ int32_t max_len;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t h = blockIdx.x / groups_per_table;
    const uint32_t q = blockIdx.x - h * groups_per_table;
    const int t = list.t[h];
    const TableDesc d = tables[t];
    const int R = static_cast<int>(d.rows);
    const int D = d.D;
    const uint32_t b0 = q * kHistBags;
    const int nb = static_cast<int>(min(static_cast<uint32_t>(kHistBags), B - b0));
    const uint32_t g0 = static_cast<uint32_t>(t) * B + b0;

    if (tid == 0) max_len = 0;
    __syncthreads();
    if (tid < kHistBags) {
        int64_t s = 0, e = 0;
        if (tid < nb) {
            s = static_cast<int64_t>(offsets[g0 + tid]);
            e = static_cast<int64_t>(offsets[g0 + tid + 1]);
        }
        bag_s[tid] = s;
        bag_e[tid] = e;
        atomicMax(&max_len, static_cast<int32_t>(e - s));
    }
    __syncthreads();
    // bags past nb start "at infinity", so the search below needs no bounds test
    if (tid < kHistBags)
        bag_rel[tid] = tid < nb ? static_cast<uint32_t>(bag_s[tid] - bag_s[0]) : 0xFFFFFFFFu;
    __syncthreads();
    const int nwin = (max_len + kHistWindow - 1) / kHistWindow;

    const int ksteps = (R + 7) / 8;
    const int ntiles = (D + 31) / 32;
    floatx16 acc[kMaxTilesPerWave];
#pragma unroll
    for (int m = 0; m < kMaxTilesPerWave; ++m)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[m][v] = 0.f;

    const _Float16* __restrict__ tb = weights + d.w_off;
    // a table of up to kStageElems elements is copied to LDS once per block
    // (16-byte loads), so the MFMA operands come from LDS
    const bool staged = R * D <= stage_elems;
    if (staged) {
        const int n8 = (R * D) / 8, rem = (R * D) % 8;
        const bool al = (reinterpret_cast<uintptr_t>(tb) & 15) == 0;
        if (al) {
            // kStageBatch loads per thread are issued before any is stored
            for (int i0 = 0; i0 < n8; i0 += 256 * kStageBatch) {
                uint4 v[kStageBatch];
                // indices past the end are clamped to the last element, which is
                // then written twice with the same value (no branch around the
                // loads, so they stay in flight together)
#pragma unroll
                for (int u = 0; u < kStageBatch; ++u) {
                    const int i = i0 + u * 256 + tid;
                    v[u] = reinterpret_cast<const uint4*>(tb)[i < n8 ? i : n8 - 1];
                }
#pragma unroll
                for (int u = 0; u < kStageBatch; ++u) {
                    const int i = i0 + u * 256 + tid;
                    reinterpret_cast<uint4*>(stab)[i < n8 ? i : n8 - 1] = v[u];
                }
            }
            for (int i = n8 * 8 + tid; i < n8 * 8 + rem; i += 256) stab[i] = tb[i];
        } else {
            for (int i = tid; i < R * D; i += 256) stab[i] = tb[i];
        }
    }
    const int frag_row = lane & 31;        // A: bag row of this lane; B: output column
    const int frag_k = (lane >> 5) * 4;    // first of the 4 k values this lane holds

    // The bags of a block are consecutive in the index array.  When each fits
    // one window, the block's ids are one contiguous range [P0, P1): every
    // thread loads kFlatIds of them at once (coalesced, all in flight) and finds
    // each id's bag by a branch-free search over the bag starts.
    const bool flat = nwin == 1;
    const int64_t P0 = bag_s[0];
    const int64_t P1 = bag_e[nb > 0 ? nb - 1 : 0];
    for (int win = 0; win < nwin; ++win) {
        for (int i = tid; i < kHistBags * (kHistMaxRows + 1); i += 256)
            (&cnt[0][0])[i] = 0u;
        __syncthreads();
        if (flat) {
            const uint32_t len = static_cast<uint32_t>(P1 - P0);   // <= kHistBags * kHistWindow
            for (uint32_t base = 0; base < len; base += 256 * kFlatIds) {
                uint32_t id[kFlatIds];   // row id, or R (out of range)
#pragma unroll
                for (int u = 0; u < kFlatIds; ++u) {
                    const uint32_t rp = base + u * 256 + tid;
                    const IT v = rp < len ? indices[P0 + rp] : IT(-1);
                    id[u] = (v >= 0 && v < R) ? static_cast<uint32_t>(v) : static_cast<uint32_t>(R);
                }
                // g[u]: the last bag whose start is <= the position (it is not
                // empty); all searches step together, then all adds.  An id
                // out of range (or a position past the end) counts into column
                // R, which the product never reads.
                int g[kFlatIds];
#pragma unroll
                for (int u = 0; u < kFlatIds; ++u) g[u] = 0;
#pragma unroll
                for (int st = kHistBags / 2; st > 0; st >>= 1)
#pragma unroll
                    for (int u = 0; u < kFlatIds; ++u) {
                        const uint32_t rp = base + u * 256 + tid;
                        g[u] = bag_rel[g[u] + st] <= rp ? g[u] + st : g[u];
                    }
#pragma unroll
                for (int u = 0; u < kFlatIds; ++u) atomicAdd(&cnt[g[u]][id[u]], 1u);
            }
        } else {
            for (int i = wave; i < nb; i += 4) {
                const int64_t s = bag_s[i] + static_cast<int64_t>(win) * kHistWindow;
                const int64_t e = min(bag_e[i], s + kHistWindow);
                for (int64_t p = s + lane; p < e; p += 64) {
                    const int64_t id = static_cast<int64_t>(indices[p]);
                    if (id >= 0 && id < R) atomicAdd(&cnt[i][id], 1u);
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < kMaxTilesPerWave; ++m) {
            const int nt = wave + 4 * m;
            if (nt >= ntiles) continue;
            const int col = nt * 32 + frag_row;
            for (int ks = 0; ks < ksteps; ++ks) {
                half4_t a, bf;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int k = ks * 8 + frag_k + j;
                    a[j] = static_cast<_Float16>(k < R ? static_cast<float>(cnt[frag_row][k]) : 0.f);
                    const bool ok = k < R && col < D;
                    if (staged)
                        bf[j] = ok ? stab[k * D + col] : static_cast<_Float16>(0.f);
                    else
                        bf[j] = ok ? tb[static_cast<int64_t>(k) * D + col]
                                   : static_cast<_Float16>(0.f);
                }
                acc[m] = __builtin_amdgcn_mfma_f32_32x32x8f16(a, bf, acc[m], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // C layout of the 32x32 tile: lane l, register v -> row 8*(v/4) + 4*(l/32) + v%4, column l%32
#pragma unroll
    for (int m = 0; m < kMaxTilesPerWave; ++m) {
        const int nt = wave + 4 * m;
        const int col = nt * 32 + frag_row;
        if (nt >= ntiles || col >= D) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int row = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (row < nb)
                out[static_cast<int64_t>(b0 + row) * sumD + d.out_off + col] = acc[m][v];
        }
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
        const dim3 grid(gpt * list.n);
        // LDS for the largest table of the launch, if every table fits
        int32_t stage = 0;
        for (int i = 0; i < list.n; ++i) {
            const TableDesc& d = p->h_tables[list.t[i]];
            stage = max(stage, static_cast<int32_t>(d.rows) * d.D);
        }
        if (stage > kStageElems) stage = 0;
        const size_t lds = static_cast<size_t>(stage) * sizeof(_Float16);
        if (p->idtype == TBE_I64)
            hipLaunchKernelGGL(k_fwd_hist<int64_t>, grid, dim3(256), lds, a.stream, p->d_tables,
                               list, static_cast<uint32_t>(a.B), gpt, p->sum_D,
                               static_cast<const _Float16*>(a.weights),
                               static_cast<const int64_t*>(a.indices),
                               static_cast<const int64_t*>(a.offsets), a.out, stage);
        else
            hipLaunchKernelGGL(k_fwd_hist<int32_t>, grid, dim3(256), lds, a.stream, p->d_tables,
                               list, static_cast<uint32_t>(a.B), gpt, p->sum_D,
                               static_cast<const _Float16*>(a.weights),
                               static_cast<const int32_t*>(a.indices),
                               static_cast<const int32_t*>(a.offsets), a.out, stage);
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
