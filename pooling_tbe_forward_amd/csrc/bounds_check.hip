// Device-side validation of the jagged inputs (the caller's preconditions of
// the operator in section "A lookup table that is most of the model" of the
// FBTriton TBE article: offsets start at 0, never decrease and end at the
// number of ids; every id of feature t lies in [0, rows[t])).  The article's
// section "Why the backward is the hard half" notes that bounds checking is a
// separate native op; here it counts violations instead of clamping.
//
// Reads stay in bounds even on bad input: an offset outside [0, num_indices]
// is counted and its bag is not walked.
#include "tbe_internal.h"

namespace tbe {
namespace {

__global__ void k_zero_i64(int64_t* p) { *p = 0; }

template <typename IT>
__global__ __launch_bounds__(256) void k_bounds_check(const TableDesc* __restrict__ tables,
                                                      uint32_t B, uint32_t total_bags,
                                                      const IT* __restrict__ indices, int64_t N,
                                                      const IT* __restrict__ offsets,
                                                      int64_t* __restrict__ err)
{
    const int lane = threadIdx.x & 63;
    const uint32_t nw = gridDim.x * (blockDim.x >> 6);
    unsigned long long bad = 0;
    for (uint32_t g = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x >> 6) +
                                                     (threadIdx.x >> 6));
         g < total_bags; g += nw) {
        const int64_t s = static_cast<int64_t>(offsets[g]);
        const int64_t e = static_cast<int64_t>(offsets[g + 1]);
        if (lane == 0) {
            if (g == 0 && s != 0) ++bad;
            if (g + 1 == total_bags && e != N) ++bad;
            if (e < s) ++bad;
        }
        if (s < 0 || e > N || e < s) {
            if (lane == 0 && (s < 0 || e > N)) ++bad;
            continue;
        }
        const uint32_t t = g / B;
        const int64_t rows = tables[t].rows;
        for (int64_t p = s + lane; p < e; p += 64) {
            const int64_t id = static_cast<int64_t>(indices[p]);
            if (id < 0 || id >= rows) ++bad;
        }
    }
    for (int m = 32; m >= 1; m >>= 1) bad += __shfl_xor(bad, m);
    if (lane == 0 && bad) atomicAdd(reinterpret_cast<unsigned long long*>(err), bad);
}

}  // namespace

hipError_t launch_bounds_check(const tbe_plan* p, int32_t B, const void* indices, int64_t N,
                               const void* offsets, int64_t* err, hipStream_t s)
{
    const uint32_t total = static_cast<uint32_t>(p->T) * static_cast<uint32_t>(B);
    hipLaunchKernelGGL(k_zero_i64, dim3(1), dim3(1), 0, s, err);
    if (total == 0) return hipGetLastError();
    const uint32_t waves = total < 65536u ? total : 65536u;
    const uint32_t blocks = (waves + 3) / 4;
    if (p->idtype == TBE_I64)
        hipLaunchKernelGGL(k_bounds_check<int64_t>, dim3(blocks), dim3(256), 0, s, p->d_tables,
                           static_cast<uint32_t>(B), total, static_cast<const int64_t*>(indices),
                           N, static_cast<const int64_t*>(offsets), err);
    else
        hipLaunchKernelGGL(k_bounds_check<int32_t>, dim3(blocks), dim3(256), 0, s, p->d_tables,
                           static_cast<uint32_t>(B), total, static_cast<const int32_t*>(indices),
                           N, static_cast<const int32_t*>(offsets), err);
    return hipGetLastError();
}

}  // namespace tbe
