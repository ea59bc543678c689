// Internal definitions shared by the HIP sources of libtbe (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "tbe.h"

namespace tbe {

constexpr int kWave = 64;

// Per-table descriptor read by every kernel (32 bytes, device resident).
enum : int32_t {
    TD_WEIGHTED = 1,   // per-sample weights apply to this table when given
    TD_HIST_OK = 2,    // shape and dtype allow the histogram x table path
};

struct TableDesc {
    int64_t w_off;      // element offset of the table in the packed weights
    uint32_t hash_off;  // hash_size_cumsum[t]: first linearized key of the table
    uint32_t rows;
    int32_t D;
    int32_t out_off;    // D_offsets[t]: first output column of the table
    int32_t flags;      // TD_*
    int32_t pad;
};
static_assert(sizeof(TableDesc) == 32, "descriptor layout");

// Histogram path limits: table rows (the contraction depth) and width.
constexpr int kHistMaxRows = 256;
constexpr int kHistMaxD = 256;
constexpr int kHistBags = 32;        // bags per MFMA tile (M)
constexpr int kHistWindow = 2048;    // ids counted per window: counts stay exact in fp16

}  // namespace tbe

struct tbe_plan {
    int32_t T = 0;
    int32_t wdtype = 0;
    int32_t idtype = 0;
    int32_t sum_D = 0;
    int32_t max_D = 0;
    int64_t sum_rows = 0;
    std::vector<int64_t> rows, w_off, D_off, hash_off;
    std::vector<int32_t> dims;
    std::vector<uint8_t> weighted;
    std::vector<tbe::TableDesc> h_tables;
    tbe::TableDesc* d_tables = nullptr;   // device [T]
    uint32_t* d_hash_off = nullptr;       // device [T+1]
    tbe_tuning tuning{};
    int device = 0;
};

namespace tbe {

// ---- forward -------------------------------------------------------------
struct FwdArgs {
    const tbe_plan* plan;
    int32_t B;
    const void* weights;
    const void* indices;
    const void* offsets;
    const float* psw;
    float* out;
    int vec;            // elements per lane load (power of two)
    bool hist_active;   // eligible tables go through the histogram kernel
    hipStream_t stream;
};
hipError_t launch_fwd_gather(const FwdArgs& a);
hipError_t launch_fwd_hist(const FwdArgs& a);

// ---- backward --------------------------------------------------------------
// Workspace carve-up (byte offsets), computed on the host.
struct BwdLayout {
    int64_t N = 0;
    int32_t nbits = 0;          // key bits to sort
    int32_t npasses = 0;
    int32_t digit_bits[4] = {0, 0, 0, 0};
    int32_t sort_tile = 0;      // keys per sort block
    int32_t sort_blocks = 0;
    int32_t rle_tile = 0;
    int32_t rle_blocks = 0;
    int64_t max_chunks = 0;     // bound on long-run chunks
    size_t off_keys[2], off_vals[2];
    size_t off_sample, off_sorted_sample, off_sorted_psw;
    size_t off_hist;            // [sort_blocks * 256] digit counts
    size_t off_unique, off_run_start, off_run_len, off_short, off_long;
    size_t off_long_chunk;      // [N+1] first chunk of each long run
    size_t off_tile_counts;     // [rle_blocks * 4]
    size_t off_counts;          // [16]
    size_t off_partials;        // [max_chunks * max_D] (fp64 or fp32)
    size_t total = 0;
};
BwdLayout bwd_layout(const tbe_plan* p, int32_t B, int64_t N);

struct BwdArgs {
    const tbe_plan* plan;
    int32_t B;
    int64_t N;
    const void* indices;
    const void* offsets;
    const float* psw;
    const float* grad;
    void* weights;
    float lr;
    char* ws;
    BwdLayout L;
    hipStream_t stream;
    // filled by run_sort_rle: which ping-pong buffer holds the sorted result
    int final_buf;
};
hipError_t run_sort_rle(BwdArgs& a);
hipError_t run_segment_sgd(const BwdArgs& a);

hipError_t launch_bounds_check(const tbe_plan* p, int32_t B, const void* indices,
                               int64_t N, const void* offsets, int64_t* err, hipStream_t s);

}  // namespace tbe
