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
constexpr int kHistBags = 16;        // bags per workgroup = M of the MFMA tile
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
    int32_t pooling = 0;                  // TBE_POOL_SUM or TBE_POOL_MEAN
    int device = 0;
    // one-shot stage events of the next call (tbe_set_stage_events)
    hipEvent_t stage_ev[8] = {};
    int32_t n_stage_ev = 0;
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
    bool mean;          // mean pooling: each bag's sum divided by its length
    hipStream_t stream;
};
hipError_t launch_fwd_gather(const FwdArgs& a);
hipError_t launch_fwd_hist(const FwdArgs& a);

// ---- backward --------------------------------------------------------------
// Control block at offset 0 of every backward workspace.  It must be zero when
// a call starts (tbe_workspace_init), and every call leaves it zero again:
// tile tickets reset themselves, each pass's digit totals are cleared by the
// next kernel.  Counts, the payload mode and the error word are outputs.
constexpr int kCtlTicket = 0;      // [4] tile tickets of the radix passes
constexpr int kCtlRleTicket = 4;   // tile ticket of the run-length encode
constexpr int kCtlError = 12;      // error word, sticky until tbe_workspace_init (kErr* bits)
constexpr int kCtlMode = 13;       // payload of the last integer stage (kMode*); an output
constexpr int kCtlCounts = 8;      // [4] runs, short runs, long runs, long-run chunks

// Bits of the error word (tbe_workspace_status).
constexpr uint32_t kErrLookback = 1u;     // a look-back wait gave up: results invalid
constexpr uint32_t kErrControl = 2u;      // the control block was not initialised
constexpr uint32_t kErrPayload = 4u;      // apply found another payload than it was told
// Payload the integer stage left in the workspace (kCtlMode).
constexpr uint32_t kModeNone = 0u;        // none yet, or tbe_sort_rle's lookup positions
constexpr uint32_t kModeSample = 1u;      // sample ids
constexpr uint32_t kModePairs = 2u;       // (sample id, weight) pairs
constexpr int kTotCopies = 8;      // digit totals are kept in this many copies
constexpr int kRadixMax = 512;     // digit counters of the widest radix pass (9-bit digits)
constexpr int kCtlTotals = 16;     // [kTotCopies][4][kRadixMax] digit totals of every radix pass
constexpr int kCtlWords = 16 + kTotCopies * 4 * kRadixMax;

// Workspace carve-up (byte offsets), computed on the host.
struct BwdLayout {
    int64_t N = 0;
    int32_t nbits = 0;          // key bits to sort
    int32_t npasses = 0;
    int32_t digit_bits[4] = {0, 0, 0, 0};
    int32_t sort_tile = 0;      // keys per sort tile
    int32_t sort_blocks = 0;
    int32_t rle_tile = 0;
    int32_t rle_blocks = 0;
    int32_t prep_blocks = 0;
    int32_t prep_bags = 0;      // bags per k_prep block
    int64_t max_chunks = 0;     // bound on long-run chunks
    int64_t max_long = 0;       // bound on long runs
    size_t off_keys[2], off_vals[2];
    size_t off_status;          // [npasses][sort_blocks][256] look-back words
    size_t off_rle_status;      // [3][rle_blocks]
    size_t status_words = 0;    // words cleared by k_prep from off_status on
    size_t off_ctl;             // [kCtlWords]
    size_t off_unique, off_run_start, off_run_len, off_short, off_long;
    size_t off_short_info;      // [N] {key, start, len, table}
    size_t off_short_first;     // [N] {sample, per-sample weight bits} of each short run's first lookup
    size_t off_long_info;       // [max_long] {key, start, len, first chunk}
    size_t off_tab_ranges;      // [3][T+1] per table: first short run, first long run, first chunk
    size_t off_chunk_info;      // [max_chunks] {first sorted position, length} of each chunk
    size_t off_partials;        // [max_chunks * max_D] (fp64 or fp32)
    // Segmented sort (seg): each table's keys are sorted within the table's
    // own segment of lookup positions, on the widest table's row bits.
    bool seg = false;
    int32_t prep_bpt = 0;       // k_prep blocks per table (segmented sort)
    int32_t seg_copies = 0;     // copies of each table's digit counts (fewer adds per address)
    size_t off_tab_tot = 0;     // [T][seg_copies][npasses][kRadixMax] digit counts of each table
    size_t off_seg_tiles = 0;   // [sort_blocks] {first position, end, table's first position, table}
    size_t off_tile_bag = 0;    // [sort_blocks] bag (within its table) of each tile's first position
    size_t off_seg_first = 0;   // [T + 1] each table's first tile slot
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
    // row-wise Adagrad (state != nullptr): one fp32 state value per row,
    // indexed by the row's key; eps is added after the square root
    float* state;
    float eps;
    char* ws;
    BwdLayout L;
    hipStream_t stream;
    // filled by run_sort_rle: which ping-pong buffer holds the sorted result,
    // and whether its payload is (sample, weight) pairs or sample ids
    int final_buf;
    int payload_pairs;
    // the payload's kind (the first radix pass of a per-table sort makes it)
    int payload_mode;
};
// api_outputs: also write unique keys, run starts / lengths and run-id lists.
hipError_t run_sort_rle(BwdArgs& a, bool api_outputs);
// Segment reduce and the row update: exact SGD, or row-wise Adagrad when
// a.state is set (then every table must fit one worker slab: see
// adagrad_supported).
hipError_t run_segment_sgd(const BwdArgs& a);
// Whether the row-wise Adagrad kernels cover this plan and buffers: the
// update needs a row's whole sum of squares inside one worker.
bool adagrad_supported(const BwdArgs& a);

// Record stage event k of the next call, if the caller asked for it.
inline void stage_mark(const tbe_plan* p, int k, hipStream_t s)
{
    if (k < p->n_stage_ev && p->stage_ev[k]) (void)hipEventRecord(p->stage_ev[k], s);
}

// Zero the control block (first kCtlWords words) of a fresh workspace.
hipError_t launch_workspace_init(void* ws, hipStream_t s);
// Copy the workspace's error word to a caller's device word.
hipError_t launch_workspace_status(const void* ws, uint32_t* out, hipStream_t s);

hipError_t launch_bounds_check(const tbe_plan* p, int32_t B, const void* indices,
                               int64_t N, const void* offsets, int64_t* err, hipStream_t s);

}  // namespace tbe
