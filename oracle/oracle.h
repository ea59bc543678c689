/*
 * CPU oracle for the table-batched embedding-bag (TBE) operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or helper with the
 * HIP library.
 *
 * What it computes is the plain definition of the operator described in the
 * FBTriton TBE article (ai.thesatyajit.com, "FBTriton table-batched
 * embeddings: the backward win is a threshold moved from 32 to 256"):
 *
 *  - forward, section "A lookup table that is most of the model": bag (t, b)
 *    is indices[offsets[t*B+b] : offsets[t*B+b+1]]; its pooled vector is the
 *    (optionally per-sample-weighted) sum of the rows it names, written to
 *    output row b at table t's column offset; an empty bag pools to zero and
 *    a repeated id counts twice; mean pooling (the same section gives the sum
 *    as the usual pooling, so the mean is the other common mode) divides a
 *    bag's sum by its length;
 *  - integer stage, section "Why the backward is the hard half": the key of a
 *    lookup is hash_size_cumsum[t] + row, keys are sorted (ties kept in lookup
 *    order), run-length encoded; section "Three tiers, routed by run length":
 *    runs are split into short (< tau) and long (>= tau) lists;
 *  - backward, section "Why the backward is the hard half": a read row's
 *    gradient is the sum of the output gradients of every bag that read it
 *    (times the per-sample weight; with mean pooling, also divided by the
 *    bag's length), and exact SGD applies w <- w - lr * g once
 *    the sum is finished; exact row-wise Adagrad (same section) keeps one
 *    fp32 state value per row, raises it by the row's mean squared gradient
 *    and steps the row by lr / (sqrt(state) + eps) times the gradient.
 *
 * All accumulation is in double precision.  fp16 storage is IEEE binary16,
 * decoded exactly and re-encoded with round-to-nearest-even.
 *
 * Status codes: 0 = ok, 1 = invalid argument, 2 = input out of range
 * (bad offsets or ids), 3 = a requested row is not held by a sparse table.
 */
#ifndef TBE_ORACLE_H
#define TBE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_F16 = 1 };
/* Pooling of a bag: the (weighted) sum of its rows, or that sum divided by
 * the bag's length (an empty bag pools to zero either way). */
enum { ORACLE_POOL_SUM = 0, ORACLE_POOL_MEAN = 1 };

/* Rows of one table held on the host.  ids == NULL: dense, row r is at
 * data + r*D.  Otherwise ids[0..n) is strictly ascending and row ids[i] is at
 * data + i*D (a sparse subset, for checks on multi-GB tables). */
typedef struct {
    int64_t n;
    const int64_t* ids;
    void* data;
} oracle_table;

int oracle_layout(int32_t T, const int64_t* rows, const int32_t* dims,
                  int64_t* weights_offsets /*[T]*/, int64_t* D_offsets /*[T+1]*/,
                  int64_t* hash_size_cumsum /*[T+1]*/);

/* bag_list == NULL: every bag, out is [B, sum D].
 * Otherwise out is [nbags, Dmax] and row k is bag bag_list[k] (= t*B + b). */
int oracle_forward(int32_t T, int32_t B, const int64_t* rows, const int32_t* dims,
                   int32_t wdtype, const oracle_table* tables,
                   const int64_t* indices, const int64_t* offsets,
                   const float* psw, const uint8_t* weighted,
                   const int64_t* bag_list, int64_t nbags, double* out, int32_t pooling);

/* Arrays are caller-allocated with N = offsets[T*B] entries each. */
int oracle_sort_rle(int32_t T, int32_t B, const int64_t* rows,
                    const int64_t* indices, const int64_t* offsets, int64_t tau,
                    int64_t* sorted_keys, int64_t* sorted_pos, int64_t* unique_keys,
                    int64_t* run_start, int64_t* run_len, int64_t* num_runs,
                    int64_t* short_runs, int64_t* num_short,
                    int64_t* long_runs, int64_t* num_long);

/* keys[0..nkeys) strictly ascending linearized keys whose rows to update.
 * grad_rows / new_rows: optional [nkeys, Dmax] double outputs (the finished
 * row gradient and the exact updated row).  write_back != 0 stores the
 * updated rows, rounded to the storage dtype, into tables[t].data. */
int oracle_backward_sgd(int32_t T, int32_t B, const int64_t* rows, const int32_t* dims,
                        int32_t wdtype, oracle_table* tables,
                        const int64_t* indices, const int64_t* offsets,
                        const float* psw, const uint8_t* weighted,
                        const float* grad_output, float lr,
                        const int64_t* keys, int64_t nkeys,
                        double* grad_rows, double* new_rows, int32_t write_back,
                        int32_t pooling);

/* Backward + exact row-wise Adagrad for keys[0..nkeys) (strictly ascending).
 * state_in[k] is the fp32 state of key k's row before the step, state_out[k]
 * receives the new one: state_in + mean_d(G[d]^2), rounded once to fp32.
 * The row steps by lr / (sqrt(new state) + eps) * G.  grad_rows, new_rows and
 * write_back as for oracle_backward_sgd.  Section "Why the backward is the
 * hard half" (the update read out of the Triton kernel; eps is the caller's). */
int oracle_backward_adagrad(int32_t T, int32_t B, const int64_t* rows, const int32_t* dims,
                            int32_t wdtype, oracle_table* tables,
                            const int64_t* indices, const int64_t* offsets,
                            const float* psw, const uint8_t* weighted,
                            const float* grad_output, float lr, float eps,
                            const int64_t* keys, int64_t nkeys,
                            const float* state_in, float* state_out,
                            double* grad_rows, double* new_rows, int32_t write_back,
                            int32_t pooling);

/* Host threads used by oracle_forward (bags split among threads) and
 * oracle_backward_sgd / oracle_backward_adagrad (the requested keys split into
 * ranges; each range's rows summed by one thread).  Every output element is
 * still accumulated by one thread in lookup order, so results are the same
 * bits for any count.  n < 1 means 1; the default is 1.  Returns the count
 * now in force (1 when the library was built without OpenMP). */
int oracle_set_threads(int n);

/* IEEE binary16 helpers (exposed so the tests can pin them). */
double   oracle_half_to_double(uint16_t h);
uint16_t oracle_double_to_half(double x);

#ifdef __cplusplus
}
#endif
#endif
