// Device half of the seeded weight generator used for test and benchmark
// inputs (libtbe_datagen.so; not part of libtbe).
//
// Element e of a table gets two 32-bit words
//     h_i = lowbias32(lowbias32(lo32(e) ^ k_i) ^ hi32(e)),   i = 0, 1
// where lowbias32 is Chris Wellons' integer hash and k_0, k_1 are per-table
// stream keys computed on the host.  The words map to a value in double:
//   kind 0: an Irwin-Hall sum of four 16-bit uniforms, centred, times `scale`
//           (an approximately normal law);
//   kind 1: a 24-bit uniform on [-1, 1).
// The double is rounded once to fp32 and, for fp16 tables, once more to fp16,
// exactly as pooling_tbe_forward_amd/datagen.py does on the host, so the host
// can regenerate any row with the same bits.  One launch fills one table.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint32_t lowbias32(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

template <typename OT>
__global__ __launch_bounds__(256) void k_gen_weights(OT* __restrict__ out, int64_t n, uint32_t k0,
                                                     uint32_t k1, int32_t kind, double scale)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n;
         e += stride) {
        const uint32_t lo = static_cast<uint32_t>(e);
        const uint32_t hi = static_cast<uint32_t>(static_cast<uint64_t>(e) >> 32);
        const uint32_t h0 = lowbias32(lowbias32(lo ^ k0) ^ hi);
        double v;
        if (kind == 0) {
            const uint32_t h1 = lowbias32(lowbias32(lo ^ k1) ^ hi);
            const int32_t s = static_cast<int32_t>((h0 & 0xffffu) + (h0 >> 16) + (h1 & 0xffffu) +
                                                   (h1 >> 16)) - 131070;
            v = static_cast<double>(s) * scale;
        } else {
            const int32_t u = static_cast<int32_t>(h0 >> 8);
            v = static_cast<double>(2 * u - (1 << 24)) * 0x1p-24;
        }
        float f = static_cast<float>(v);   // round to nearest even
        // The fp32 value must exist: without this the compiler folds the two
        // conversions into one direct double -> fp16 rounding, which differs
        // from rounding twice by one fp16 ulp near ties (measured: about 1 in
        // 30,000 elements of the fp16 tables).
        asm volatile("" : "+v"(f));
        out[e] = static_cast<OT>(f);       // fp16: one more rounding, nearest even
    }
}

}  // namespace

// Fill out[0 .. n) (device pointer, fp32 when f16 == 0, else fp16) with one
// table's generated weights on `stream` (a hipStream_t; NULL = default).
// Returns 0, or a hipError_t code.
extern "C" int tbe_datagen_fill(void* out, int64_t n, int32_t f16, uint32_t k0, uint32_t k1,
                                int32_t kind, double scale, void* stream)
{
    if (n <= 0) return 0;
    if (!out || (kind != 0 && kind != 1)) return static_cast<int>(hipErrorInvalidValue);
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (f16)
        hipLaunchKernelGGL(k_gen_weights<_Float16>, dim3(static_cast<uint32_t>(blocks)), dim3(256),
                           0, s, static_cast<_Float16*>(out), n, k0, k1, kind, scale);
    else
        hipLaunchKernelGGL(k_gen_weights<float>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                           s, static_cast<float*>(out), n, k0, k1, kind, scale);
    return static_cast<int>(hipGetLastError());
}
