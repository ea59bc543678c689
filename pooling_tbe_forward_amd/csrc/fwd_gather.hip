// Forward pooled gather-sum for gfx950.
//
// Operator: section "A lookup table that is most of the model" of the FBTriton
// TBE article -- bag (t, b) = indices[offsets[t*B+b] : offsets[t*B+b+1]], its
// rows (times the per-sample weight on weighted tables) summed into output row
// b at column D_offsets[t]; an empty bag writes zeros.
//
// Design (section "The forward: a general gather and one clever special case"
// describes the latency problem: a gather is a dependent chain, index then
// row, so several chains must be in flight):
//  * one 64-lane wavefront owns one bag at a time; a row of D elements is
//    covered by L = D/VEC lanes (16-byte loads), so the wave holds G = 64/L
//    row slots side by side and each lane keeps U independent row loads in
//    flight: G*U rows per wavefront per step;
//  * the bag's ids are fetched with one coalesced load per 64 ids and handed
//    to the row slots through cross-lane permutes, so the only serial chain is
//    offsets -> ids -> rows;
//  * accumulation in fp32 VGPRs; slots are folded with lane swaps at the end.
#include "tbe_internal.h"

namespace tbe {
namespace {

template <typename T, int N>
struct alignas(sizeof(T) * N) Pack {
    T v[N];
};

template <typename WT>
__device__ __forceinline__ float to_f32(WT x) { return static_cast<float>(x); }

// Streaming (non-temporal) store of an output slice: the pooled output is
// written once and not read again by this kernel, so it should not take cache
// lines from the rows being gathered (measured: mixed workload forward 281 ->
// 265 us; uniform unchanged).  P is a Pack of 4, 8, 16 or 32 bytes (the last
// as two 16-byte stores).
template <int BYTES>
struct RawVec;
template <> struct RawVec<16> { typedef uint32_t T __attribute__((ext_vector_type(4))); };
template <> struct RawVec<8> { typedef uint32_t T __attribute__((ext_vector_type(2))); };
template <> struct RawVec<4> { typedef uint32_t T; };

template <typename P>
__device__ __forceinline__ void stg_stream(P* p, const P& v)
{
#if __HIP_DEVICE_COMPILE__
    constexpr int kPiece = sizeof(P) < 16 ? sizeof(P) : 16;
    typedef typename RawVec<kPiece>::T R;
#pragma unroll
    for (int o = 0; o < static_cast<int>(sizeof(P)); o += kPiece) {
        R x;
        __builtin_memcpy(&x, reinterpret_cast<const char*>(&v) + o, kPiece);
        __builtin_nontemporal_store(
            x, (__attribute__((address_space(1))) R*)(reinterpret_cast<char*>(p) + o));
    }
#else
    *p = v;
#endif
}

template <typename IT>
__device__ __forceinline__ int64_t lane_bcast(IT v, int src) {
    return static_cast<int64_t>(__shfl(v, src));
}

// Issue the U row loads of one round: slot grp of row r0 + u*G + grp.  Slots
// past the end of the 64-id chunk read the chunk's last row again, and lanes
// past D read column 0 of their slot's row; both are masked out when summed,
// so every load is unconditional and all U stay in flight.  A repeated row is
// one this wave fetches anyway, so these loads add no new lines (pointing
// them at the table's first row sent about 30% of the mixed workload's row
// requests to the same few L2 lines; the time did not change measurably).
template <typename WT, typename IT, int VEC, int U>
__device__ __forceinline__ void issue_round(Pack<WT, VEC> (&v)[U], float (&w)[U], bool (&on)[U],
                                            const WT* tcol, int D, IT my_id,
                                            float my_w, int r0, int n, int g_log2, int grp,
                                            bool active, bool tw)
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int r = r0 + (u << g_log2) + grp;
        on[u] = r < n && active;
        const int src = r < n ? r : n - 1;  // n >= 1 inside a chunk
        const int64_t row = lane_bcast(my_id, src);
        w[u] = tw ? __shfl(my_w, src) : 1.f;
        v[u] = *reinterpret_cast<const Pack<WT, VEC>*>(tcol + row * D);
    }
}

// Nothing moves across this point: neither memory operations (the empty asm)
// nor arithmetic (the scheduling barrier).
__device__ __forceinline__ void issue_fence()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <typename WT, int VEC, int U>
__device__ __forceinline__ void sum_round(float (&acc)[VEC], const Pack<WT, VEC> (&v)[U],
                                          const float (&w)[U], const bool (&on)[U], bool tw)
{
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const float x = on[u] ? to_f32(v[u].v[k]) : 0.f;
            if (tw)
                acc[k] = fmaf(w[u], x, acc[k]);
            else
                acc[k] += x;
        }
}

template <typename WT, typename IT, int VEC, int U, bool WEIGHTED>
__global__ __launch_bounds__(64) void k_fwd_gather(
    const TableDesc* __restrict__ tables, uint32_t B, uint32_t total_bags, int32_t sumD,
    const WT* weights, const IT* __restrict__ indices,
    const IT* __restrict__ offsets, const float* __restrict__ psw, float* __restrict__ out,
    uint32_t bags_per_wave, int32_t hist_active, int32_t mean)
{
    const int lane = threadIdx.x & 63;
    const uint32_t wave = blockIdx.x;  // one wave per workgroup
    const uint32_t g0 = wave * bags_per_wave;
    if (g0 >= total_bags) return;
    const uint32_t g1 = min(g0 + bags_per_wave, total_bags);

    for (uint32_t g = g0; g < g1; ++g) {
        const uint32_t t = g / B;
        const uint32_t b = g - t * B;
        const IT s_raw = offsets[g];
        const IT e_raw = offsets[g + 1];
        const TableDesc d = tables[t];
        // the bag's bounds do not depend on its table's record: every field
        // used below is consumed here, before any branch or conversion, so the
        // wave waits once for both (the compiler would otherwise sink each
        // load to the block that uses it, making the chain record -> bounds ->
        // ids -> rows)
        asm volatile("" ::"s"(s_raw), "s"(e_raw), "s"(d.w_off), "s"(d.D), "s"(d.out_off),
                     "s"(d.flags));
        const int64_t s = static_cast<int64_t>(s_raw);
        const int64_t e = static_cast<int64_t>(e_raw);
        if (hist_active && (d.flags & TD_HIST_OK) && !(WEIGHTED && (d.flags & TD_WEIGHTED)))
            continue;  // pooled by the histogram kernel
        const bool tw = WEIGHTED && (d.flags & TD_WEIGHTED);
        const int D = d.D;
        const int lanes = D / VEC;
        const int lpr_log2 = lanes >= 64 ? 6 : (lanes <= 1 ? 0 : 32 - __builtin_clz(lanes - 1));
        const int g_log2 = 6 - lpr_log2;
        const int grp = lane >> lpr_log2;
        const int col = (lane & ((1 << lpr_log2) - 1)) * VEC;
        // (weights is not restrict-qualified: loads through it must stay
        // ordered by issue_fence)
        const WT* tb = weights + d.w_off;
        float* __restrict__ orow = out + static_cast<int64_t>(b) * sumD + d.out_off;

        for (int c0 = 0; c0 < D; c0 += 64 * VEC) {
            const int c = c0 + col;
            const bool active = c < D;
            float acc[VEC];
#pragma unroll
            for (int k = 0; k < VEC; ++k) acc[k] = 0.f;
            const WT* tcol = tb + (active ? c : 0);

            // ids of the next 64 lookups are fetched while the current ones are
            // gathered; row rounds are double-buffered (round r+1 is issued
            // before round r is summed), so 2*U row loads per lane are in flight
            IT nid = 0;
            float nw = 1.f;
            if (lane < e - s) {
                nid = indices[s + lane];
                if (tw) nw = psw[s + lane];
            }
            for (int64_t base = s; base < e; base += 64) {
                const int n = (e - base) < 64 ? static_cast<int>(e - base) : 64;
                const IT my_id = nid;
                const float my_w = nw;
                if (base + 64 + lane < e) {
                    nid = indices[base + 64 + lane];
                    if (tw) nw = psw[base + 64 + lane];
                }
                const int step = U << g_log2;
                Pack<WT, VEC> va[U], vb[U];
                float wa[U], wb[U];
                bool oa[U], ob[U];
                issue_round<WT, IT, VEC, U>(va, wa, oa, tcol, D, my_id, my_w, 0, n, g_log2, grp,
                                            active, tw);
                issue_fence();
                // the next round is always issued (past the end it re-reads a
                // row, masked): a load under a branch would make the compiler wait
                // for every outstanding load where the branches meet
                // (issue_fence keeps the compiler from moving a round's loads down
                // to their use, or a sum above the next round's loads, which
                // would undo the double buffering)
                for (int r0 = 0; r0 < n; r0 += 2 * step) {
                    issue_round<WT, IT, VEC, U>(vb, wb, ob, tcol, D, my_id, my_w, r0 + step, n,
                                                g_log2, grp, active, tw);
                    issue_fence();
                    sum_round<WT, VEC, U>(acc, va, wa, oa, tw);
                    if (r0 + step >= n) break;
                    issue_round<WT, IT, VEC, U>(va, wa, oa, tcol, D, my_id, my_w, r0 + 2 * step, n,
                                                g_log2, grp, active, tw);
                    issue_fence();
                    sum_round<WT, VEC, U>(acc, vb, wb, ob, tw);
                }
            }
            // fold the G row slots: lanes that differ only in the slot bits
            for (int m = 32; m >= (1 << lpr_log2); m >>= 1) {
#pragma unroll
                for (int k = 0; k < VEC; ++k) acc[k] += __shfl_xor(acc[k], m);
            }
            if (grp == 0 && active) {
                Pack<float, VEC> o;
                // mean pooling: one rounding of sum / length (an empty bag stays 0)
                const float len = mean && e > s ? static_cast<float>(e - s) : 1.f;
#pragma unroll
                for (int k = 0; k < VEC; ++k) o.v[k] = mean ? acc[k] / len : acc[k];
                stg_stream(reinterpret_cast<Pack<float, VEC>*>(orow + c), o);
            }
        }
    }
}

template <typename WT, typename IT, int VEC>
hipError_t launch_vec(const FwdArgs& a)
{
    const tbe_plan* p = a.plan;
    const uint32_t total = static_cast<uint32_t>(p->T) * static_cast<uint32_t>(a.B);
    const uint32_t bpw = static_cast<uint32_t>(max(1, p->tuning.fwd_bags_per_wave));
    const uint32_t waves = (total + bpw - 1) / bpw;
    // one-wave workgroups: the waves of a workgroup are placed one per SIMD of
    // a CU, so a four-wave workgroup waits for a free slot on all four SIMDs
    // at once, and with bags of unequal length that left about 5,300 of the
    // chip's 8,192 wave slots busy (mixed workload; about 7,250 with one-wave
    // workgroups, forward 236 -> 211 us)
    const uint32_t blocks = waves;
    if (blocks == 0) return hipSuccess;
    // rows per lane per round (2U in flight with the double buffer): 2 with
    // 16-byte loads, 8 with narrower ones.  The kernel is bound by how many
    // waves keep gathers in flight: U = 2 holds 8 waves per SIMD where U = 4
    // held 5 (fp16 weighted) or 6 (fp32), and measured faster on every
    // workload with hot rows (mixed forward 280 -> 235 us, stress 58 -> 52,
    // band 57 -> 50; uniform unchanged; U = 1 was slower on stress).
    constexpr int U = (VEC * sizeof(WT) >= 16) ? 2 : 8;
    const dim3 grid(blocks), block(64);
    const auto* w = static_cast<const WT*>(a.weights);
    const auto* ix = static_cast<const IT*>(a.indices);
    const auto* of = static_cast<const IT*>(a.offsets);
    const int ha = a.hist_active ? 1 : 0;
    const int mean = a.mean ? 1 : 0;
    const uint32_t Bu = static_cast<uint32_t>(a.B);
    if (a.psw)
        hipLaunchKernelGGL((k_fwd_gather<WT, IT, VEC, U, true>), grid, block, 0, a.stream,
                           p->d_tables, Bu, total, p->sum_D, w, ix, of, a.psw, a.out, bpw, ha,
                           mean);
    else
        hipLaunchKernelGGL((k_fwd_gather<WT, IT, VEC, U, false>), grid, block, 0, a.stream,
                           p->d_tables, Bu, total, p->sum_D, w, ix, of, a.psw, a.out, bpw, ha,
                           mean);
    return hipGetLastError();
}

template <typename WT, typename IT>
hipError_t launch_wt_it(const FwdArgs& a)
{
    switch (a.vec) {
    case 1: return launch_vec<WT, IT, 1>(a);
    case 2: return launch_vec<WT, IT, 2>(a);
    case 4: return launch_vec<WT, IT, 4>(a);
    case 8:
        if constexpr (sizeof(WT) == 2) return launch_vec<WT, IT, 8>(a);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_fwd_gather(const FwdArgs& a)
{
    const bool f16 = a.plan->wdtype == TBE_F16;
    const bool i64 = a.plan->idtype == TBE_I64;
    if (f16)
        return i64 ? launch_wt_it<_Float16, int64_t>(a) : launch_wt_it<_Float16, int32_t>(a);
    return i64 ? launch_wt_it<float, int64_t>(a) : launch_wt_it<float, int32_t>(a);
}

}  // namespace tbe
