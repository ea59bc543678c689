/*
 * tbe.h -- C ABI of the MI355X (gfx950) table-batched embedding-bag library.
 *
 * The operator is the one described in "FBTriton table-batched embeddings:
 * the backward win is a threshold moved from 32 to 256" (ai.thesatyajit.com):
 *
 *  - Section "A lookup table that is most of the model": every table is packed
 *    into one weight buffer; all ids go into one flat indices array; offsets
 *    are feature-major, so bag (t, b) is indices[offsets[t*B+b] :
 *    offsets[t*B+b+1]]; the forward writes a [B, sum D] output with table t's
 *    pooled vector at its own column offset.  Pooling is a sum.
 *  - Section "Why the backward is the hard half": a read row's gradient is
 *    the sum of the output gradients of the bags that read it; the backward
 *    linearizes (table, row) into hash_size_cumsum[t] + row, sorts, run-length
 *    encodes, and applies exact SGD to each row once its sum is finished.
 *  - Section "Three tiers, routed by run length": runs are routed by length
 *    against a threshold into a short-run path and a split long-run path.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless the argument says "host".
 *  - The caller allocates and owns every device buffer.  The library
 *    allocates device memory only inside tbe_plan_create (three small
 *    per-table arrays) and frees it in tbe_plan_destroy.  Forward and
 *    backward never allocate; the backward uses the caller's workspace.
 *  - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *    enqueued on it; no call synchronises the host or reads device memory
 *    back, so results are ready when the stream says so.
 *  - Host-checkable problems return an error before anything is enqueued.
 *    Device-resident preconditions are the caller's (offsets[0] = 0,
 *    nondecreasing offsets, offsets[T*B] = num_indices, 0 <= id < rows[t]);
 *    tbe_bounds_check verifies them on the device.
 *  - Layout: table t, row r, column d is weights[weights_offsets[t] +
 *    r*D_t + d] with weights_offsets[t] = sum_{t'<t} rows[t']*D[t']; output
 *    column D_offsets[t] + d; linearized key hash_size_cumsum[t] + r.
 *  - Limits: sum(rows) < 2^32, num_indices < 2^30, T*B < 2^31, D_t <= 4096.
 *  - No exceptions cross this boundary.
 */
#ifndef TBE_H
#define TBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TBE_OK = 0,
    TBE_EINVAL = 1,   /* bad argument (NULL pointer, negative size, bad enum, small workspace) */
    TBE_ERANGE = 2,   /* a size exceeds the limits above */
    TBE_ENOMEM = 3,   /* device allocation in tbe_plan_create failed */
    TBE_EHIP = 4,     /* a HIP runtime call or kernel launch failed */
    TBE_ENOTSUP = 5   /* a valid but unsupported combination */
} tbe_status;

typedef enum { TBE_F32 = 0, TBE_F16 = 1 } tbe_fp;   /* weight storage type */
typedef enum { TBE_I32 = 0, TBE_I64 = 1 } tbe_int;  /* applies to indices AND offsets */
typedef enum { TBE_POOL_SUM = 0, TBE_POOL_MEAN = 1 } tbe_pooling;

typedef struct tbe_plan tbe_plan;  /* opaque; immutable after create except tuning and pooling */

/* Launch knobs.  Defaults come from measurements on MI355X; tbe_set_tuning
 * exists for sweeps and for tests that force a path. */
typedef struct {
    int32_t tau;               /* runs with length >= tau take the long (split) path */
    int32_t chunk;             /* lookups per long-run chunk (split-K) */
    int32_t hist_mode;         /* 0 auto, 1 never, 2 always for eligible tables */
    int32_t hist_min_mean_len; /* auto: histogram path when N/(T*B) >= this */
    int32_t fwd_bags_per_wave; /* forward: consecutive bags handled by one wavefront */
    int32_t seg_slab_kib;      /* backward: target size (KiB) of the grad_output slab of one
                                  column block of a table, B x columns x 4 bytes; rows
                                  wider than that are reduced in column blocks of at least
                                  16 lanes' loads (0 = whole rows) */
    int32_t sort_mode;         /* backward sort: 0 auto, 1 one sort over every table's keys,
                                  2 per table (each table's lookups sorted on their rows
                                  inside the table's own positions; up to 1024 tables,
                                  else as 1) */
    int32_t reserved[9];
} tbe_tuning;

/* Bits of a backward workspace's error word (tbe_workspace_status; also
 * counts[4] of tbe_sort_view).  The word is sticky: a bit stays set until
 * tbe_workspace_init.  Any bit set means that the calls made on the workspace
 * since then may have left invalid results (weights, state, sort outputs). */
#define TBE_WS_ERR_LOOKBACK 1u  /* a look-back wait of the sort or run-length encode
                                   gave up (a predecessor never published) */
#define TBE_WS_ERR_CONTROL 2u   /* a call found the control block uninitialised */
#define TBE_WS_ERR_PAYLOAD 4u   /* tbe_backward_apply(_adagrad) was told `weighted`
                                   unlike what tbe_backward_prepare stored; that
                                   apply did nothing */

/* Device pointers into a backward workspace (valid until the workspace is
 * reused).  Every count lives in device memory: counts[0] = number of runs,
 * counts[1] = short runs, counts[2] = long runs, counts[3] = long-run chunks,
 * counts[4] = error word (TBE_WS_ERR_* bits), counts[5] = payload mode of the
 * last integer stage (library-internal). */
typedef struct {
    uint32_t* sorted_keys;   /* [N]   keys ascending; ties keep lookup order        */
    uint32_t* sorted_pos;    /* [N]   lookup position j of each sorted entry        */
    uint32_t* unique_keys;   /* [N]   first counts[0] valid, strictly ascending     */
    uint32_t* run_start;     /* [N+1] first sorted position of each run             */
    uint32_t* run_len;       /* [N]   lookups in each run                           */
    uint32_t* short_runs;    /* [N]   run ids with len < tau, ascending             */
    uint32_t* long_runs;     /* [N]   run ids with len >= tau, ascending            */
    uint32_t* counts;        /* [6]                                                 */
} tbe_sort_view;

/*
 * Create a plan for T tables.  rows/dims (host [T]): rows and width of each
 * table (rows >= 0, 1 <= D <= 4096).  weight_dtype: tbe_fp.  index_dtype:
 * tbe_int.  weighted (host [T] or NULL): which tables apply per-sample
 * weights when a call passes them (NULL = every table).  On success *out owns
 * three small device arrays (per-table descriptors) on the current device.
 * Errors: TBE_EINVAL, TBE_ERANGE, TBE_ENOMEM, TBE_EHIP.
 */
tbe_status tbe_plan_create(int32_t T, const int64_t* rows, const int32_t* dims,
                           int32_t weight_dtype, int32_t index_dtype,
                           const uint8_t* weighted, tbe_plan** out);

/* Free the plan and its device arrays.  NULL is a no-op.  The caller must
 * make sure no enqueued work still uses the plan. */
void tbe_plan_destroy(tbe_plan* plan);

/* Host copies of the layout prefix sums: weights_offsets [T] (elements),
 * D_offsets [T+1], hash_size_cumsum [T+1].  Any pointer may be NULL. */
tbe_status tbe_plan_layout(const tbe_plan* plan, int64_t* weights_offsets,
                           int64_t* D_offsets, int64_t* hash_size_cumsum);

/*
 * Forward pooled sum (section "A lookup table that is most of the model";
 * the small-table path is section "The forward: a general gather and one
 * clever special case").
 *   weights  [sum rows*D] of weight_dtype (read only)
 *   indices  [num_indices] of index_dtype
 *   offsets  [T*B+1] of index_dtype, feature-major
 *   per_sample_weights [num_indices] fp32 or NULL (applied on weighted tables)
 *   output   [B, sum D] fp32; every element is written (empty bags -> 0)
 * Accumulation is fp32.  B = 0 is a no-op.
 */
tbe_status tbe_forward(const tbe_plan* plan, int32_t B, const void* weights,
                       const void* indices, int64_t num_indices, const void* offsets,
                       const float* per_sample_weights, float* output, void* stream);

/* Bytes of workspace tbe_backward_sgd / tbe_sort_rle need for (B,
 * num_indices) under the plan's current tuning.  0 on invalid arguments. */
size_t tbe_backward_workspace_bytes(const tbe_plan* plan, int32_t B, int64_t num_indices);

/*
 * Prepare a backward workspace before its first use (enqueued on `stream`).
 * The first 65600 bytes of a workspace are a control block (tile tickets and
 * digit totals of the sort, counts, an error word) that must be zero when a
 * call starts; every tbe_backward_sgd / tbe_sort_rle call leaves it zero
 * again, so one init per allocation is enough, whatever plan, B or
 * num_indices later calls use.  A zero-filled allocation is also initialised.
 * Errors: TBE_EINVAL (NULL, not 256-byte aligned, fewer than 65600 bytes),
 * TBE_EHIP.
 */
tbe_status tbe_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward + exact SGD, in place (section "Why the backward is the hard
 * half"; routing by run length from section "Three tiers, routed by run
 * length").  For every row r of table t read by some lookup,
 *   W_t[r] <- W_t[r] - lr * sum_{lookups j of (t, r)} w_j * grad_output[b(j), D_offsets[t] : +D_t]
 * with w_j the per-sample weight (1 on unweighted tables or when NULL).
 * Rows nobody read are not touched.  grad_output is [B, sum D] fp32.
 * Accumulation is fp64 for fp32 tables and fp32 for fp16 tables; the update
 * is rounded once to the storage type.  The result is deterministic.
 * workspace: device buffer of at least tbe_backward_workspace_bytes bytes,
 * 256-byte aligned, initialised once by tbe_workspace_init.  Calls that
 * share a workspace must not overlap (same stream, or ordered by events).
 */
tbe_status tbe_backward_sgd(const tbe_plan* plan, int32_t B, void* weights,
                            const void* indices, int64_t num_indices, const void* offsets,
                            const float* per_sample_weights, const float* grad_output,
                            float lr, void* workspace, size_t workspace_bytes, void* stream);

/*
 * tbe_backward_sgd without a caller workspace, for callers that cannot
 * allocate device memory or pass a workspace (code under stream capture,
 * serving loops, harnesses that forbid allocation).  The same kernels and the
 * same result as tbe_backward_sgd; the workspace is a 64 MiB array inside the
 * library, one copy per GPU, held until the process ends.  Nothing is
 * allocated per call.
 *   error_word: device uint32 (4-byte aligned) or NULL; when given, it
 *               receives the call's workspace error word (TBE_WS_ERR_* bits,
 *               0 = valid) on `stream` after the update.
 * Each call clears the array's control block first, so a call never sees an
 * earlier call's state.  Every call on one GPU shares the array: calls that
 * may overlap on one GPU (different streams, or several host threads) race
 * and must be serialised by the caller.
 * Errors: as for tbe_backward_sgd, and TBE_ERANGE when the call needs more
 * workspace than the array holds (tbe_backward_workspace_bytes(plan, B,
 * num_indices) > tbe_backward_noalloc_max_bytes(); about 830K lookups for
 * fp32 tables of D = 128 -- a batch of 328K such lookups needs 25 MB).
 */
tbe_status tbe_backward_sgd_noalloc(const tbe_plan* plan, int32_t B, void* weights,
                                    const void* indices, int64_t num_indices,
                                    const void* offsets, const float* per_sample_weights,
                                    const float* grad_output, float lr, uint32_t* error_word,
                                    void* stream);

/* Size in bytes of tbe_backward_sgd_noalloc's per-GPU workspace array. */
size_t tbe_backward_noalloc_max_bytes(void);

/*
 * The backward in two halves, for callers that overlap its integer stage with
 * other work.  The integer stage reads only indices, offsets and per-sample
 * weights, so it can run on a second stream while the forward of the same
 * batch runs; tbe_backward_sgd is exactly prepare followed by apply on one
 * stream.
 *
 * tbe_backward_prepare: linearize, stable radix sort (payload: sample id and
 * per-sample weight), run-length encode and classify runs, into the
 * workspace (section "Why the backward is the hard half"; classification
 * from section "Three tiers, routed by run length").  Arguments as for
 * tbe_backward_sgd.
 *
 * tbe_backward_apply: segment reduce + exact SGD from a workspace that
 * tbe_backward_prepare filled for the same plan, B and num_indices, with the
 * plan's tuning unchanged in between.  weighted: nonzero iff prepare was
 * given per-sample weights.  The workspace records which payload prepare
 * stored; if `weighted` disagrees with it (or no prepare ran since
 * tbe_workspace_init), apply updates nothing and sets TBE_WS_ERR_PAYLOAD in
 * the workspace's error word (tbe_workspace_status).  The caller orders apply
 * after prepare (same stream, or an event); errors as for tbe_backward_sgd.
 */
tbe_status tbe_backward_prepare(const tbe_plan* plan, int32_t B, const void* indices,
                                int64_t num_indices, const void* offsets,
                                const float* per_sample_weights, void* workspace,
                                size_t workspace_bytes, void* stream);
tbe_status tbe_backward_apply(const tbe_plan* plan, int32_t B, int64_t num_indices,
                              int32_t weighted, void* weights, const float* grad_output,
                              float lr, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward + exact row-wise Adagrad, in place (section "Why the backward is
 * the hard half", where the article reads the update out of the Triton
 * kernel).  For every row r of table t read by some lookup, with g the same
 * finished row gradient as in tbe_backward_sgd:
 *   state[k] <- state[k] + (1/D_t) * sum_d g[d]^2   (rounded once to fp32)
 *   W_t[r]   <- W_t[r] - lr / (sqrt(state[k]) + eps) * g
 * where k = hash_size_cumsum[t] + r (tbe_plan_layout) indexes `state`, a
 * caller-owned device array of sum(rows) fp32 values (zero before the first
 * step), 4-byte aligned.  eps >= 0 (the pages do not give a value; 1e-8 is
 * this library's suggestion).  Rows nobody read keep their weights and
 * state.  Accumulation as for tbe_backward_sgd; the state step and the rate
 * are computed in the accumulator type.  The update needs a row's whole sum
 * of squares inside one group of lanes, so every table needs D <= 64 * v,
 * where v (1, 2 or 4) is the widest vector width that every D, grad_output
 * and the weights are aligned to: TBE_ENOTSUP otherwise.  TBE_EINVAL also
 * for a NULL or misaligned state and for eps < 0 or NaN.  Workspace and
 * ordering rules as for tbe_backward_sgd.
 *
 * tbe_backward_apply_adagrad: the same update from a workspace that
 * tbe_backward_prepare filled (see tbe_backward_apply).
 */
tbe_status tbe_backward_adagrad(const tbe_plan* plan, int32_t B, void* weights, float* state,
                                const void* indices, int64_t num_indices, const void* offsets,
                                const float* per_sample_weights, const float* grad_output,
                                float lr, float eps, void* workspace, size_t workspace_bytes,
                                void* stream);
tbe_status tbe_backward_apply_adagrad(const tbe_plan* plan, int32_t B, int64_t num_indices,
                                      int32_t weighted, void* weights, float* state,
                                      const float* grad_output, float lr, float eps,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * The backward's integer stage alone (section "Why the backward is the hard
 * half": the backward inverts the batch -- every lookup gets the key
 * hash_size_cumsum[t] + row, the keys are sorted so each row's contributors
 * sit next to each other, and a run-length encode makes each row one unit of
 * work; the article's Triton backward gets this from one native op that
 * linearizes, radix-sorts and run-length encodes.  The split of runs by length
 * is section "Three tiers, routed by run length").  The sort is stable (ties
 * in lookup order) and its payload is the lookup position j, so sorted_pos is
 * the stable permutation.  Arguments as for tbe_backward_sgd; fills *view
 * (host struct) with device pointers into the workspace, valid until the
 * workspace is used again.  Runs with length >= tuning.tau are listed as long.
 * Errors: TBE_EINVAL (NULL view, or as for tbe_backward_sgd), TBE_ERANGE,
 * TBE_EHIP.  Device-side failures set the error word (counts[4]).
 */
tbe_status tbe_sort_rle(const tbe_plan* plan, int32_t B, const void* indices,
                        int64_t num_indices, const void* offsets, void* workspace,
                        size_t workspace_bytes, tbe_sort_view* view, void* stream);

/*
 * Device-side input check (section "Why the backward is the hard half" names
 * bounds checking of the indices as a separate native op run outside the
 * fused path; the preconditions are those of the input format in section "A
 * lookup table that is most of the model").  *error_count (device int64,
 * caller-owned, overwritten) receives the number of violations:
 * offsets[0] != 0, a decreasing offset step, offsets[T*B] != num_indices, and
 * each id outside [0, rows[t]).  Nothing is clamped or skipped, and every
 * read stays in bounds even on bad input.  The caller syncs the stream to read
 * the count.  Errors: TBE_EINVAL (NULL plan or error_count, negative sizes,
 * NULL indices/offsets where needed), TBE_ERANGE, TBE_EHIP.
 */
tbe_status tbe_bounds_check(const tbe_plan* plan, int32_t B, const void* indices,
                            int64_t num_indices, const void* offsets,
                            int64_t* error_count, void* stream);

/*
 * Error word of a backward workspace (TBE_WS_ERR_* bits; 0 = every call on
 * the workspace since tbe_workspace_init ran normally), copied to
 * *error_word, a caller-owned 4-byte-aligned device uint32, on `stream`, after
 * the work already enqueued there; the caller syncs to read it.  The word
 * itself sits at byte offset 48 of the workspace.  Nothing is cleared.
 * Errors: TBE_EINVAL (NULL or misaligned pointers, a workspace smaller than
 * its control block), TBE_EHIP.
 */
tbe_status tbe_workspace_status(const void* workspace, size_t workspace_bytes,
                                uint32_t* error_word, void* stream);

/* Read / replace the plan's launch knobs (values are validated). */
tbe_status tbe_get_tuning(const tbe_plan* plan, tbe_tuning* tuning);
tbe_status tbe_set_tuning(tbe_plan* plan, const tbe_tuning* tuning);

/*
 * Pooling of a bag (section "A lookup table that is most of the model" gives
 * the sum as the usual pooling).  TBE_POOL_SUM (the default): the
 * (per-sample-weighted) sum of the bag's rows.  TBE_POOL_MEAN: that sum
 * divided by the bag's length; an empty bag still pools to zero.  The
 * backward of a mean-pooled plan divides each lookup's contribution by the
 * length of its bag.  Applies to every later call on the plan (the
 * histogram path, where it applies, divides its sums the same way).  Errors:
 * TBE_EINVAL (NULL plan, unknown mode).
 */
tbe_status tbe_plan_set_pooling(tbe_plan* plan, int32_t pooling);

/*
 * Optional per-stage timing, for profilers and benchmarks.  events: host array
 * of n hipEvent_t handles (NULL entries allowed) the caller created; the NEXT
 * call on this plan records them on its stream at its stage boundaries, then
 * forgets them (one-shot).  Forward: [0] before its first kernel, [1] after
 * its last.  Backward: [0] start, [1] after the key/payload pass, [2] after
 * the radix passes, [3] after run-length encoding, [4] after the
 * segment-reduce + SGD kernel, [5] after the long-run combine;
 * tbe_backward_prepare records [0]-[3], tbe_backward_apply [4]-[5].  Events
 * beyond n are not recorded.  events = NULL (or n = 0) clears.  Not for plans
 * shared by concurrent calls.
 */
tbe_status tbe_set_stage_events(tbe_plan* plan, void* const* events, int32_t n);

/* Static English text for a status code. */
const char* tbe_status_string(tbe_status status);

/* ABI version (major*10000 + minor*100 + patch). */
int32_t tbe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TBE_H */
