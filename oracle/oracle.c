/*
 * CPU oracle for the table-batched embedding-bag operator: plain loops, double
 * accumulation.  TEST INFRASTRUCTURE ONLY (see oracle.h for the contract and
 * the passages of the FBTriton TBE article each function follows).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 1;

int oracle_set_threads(int n)
{
#ifdef _OPENMP
    g_threads = n < 1 ? 1 : n;
#else
    (void)n;
    g_threads = 1;
#endif
    return g_threads;
}

/* ---------------------------------------------------------------------- */
/* IEEE 754 binary16 (1 sign bit, 5 exponent bits with bias 15, 10 fraction
 * bits).  Decoding is exact; encoding rounds to nearest, ties to even,
 * keeps subnormals and overflows to infinity. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* zero or subnormal */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* 1.f * 2^(e-15) */
    return sign ? -v : v;
}

uint16_t oracle_double_to_half(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return 0x7e00;
    double a = fabs(x);
    /* Largest finite half is 65504; the midpoint to the next (2^16) is 65520
     * and ties go to the even significand, i.e. to infinity. */
    if (a >= 65520.0)
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: units of 2^-24 */
        double q = nearbyint(ldexp(a, 24));
        return sign | (uint16_t)q;                 /* q == 1024 encodes 2^-14 */
    }
    int E;
    frexp(a, &E);                                  /* a = m * 2^E, m in [0.5, 1) */
    int p = E - 1;                                 /* a in [2^p, 2^(p+1)) */
    double q = nearbyint(ldexp(a, 10 - p));        /* significand in [1024, 2048] */
    uint32_t bits = (uint32_t)(p + 15) << 10;
    bits += (uint32_t)q - 1024;                    /* q == 2048 carries into the exponent */
    return sign | (uint16_t)bits;
}

static double load_elem(const void* base, int64_t i, int32_t wdtype)
{
    if (wdtype == ORACLE_F32)
        return (double)((const float*)base)[i];
    return oracle_half_to_double(((const uint16_t*)base)[i]);
}

static void store_elem(void* base, int64_t i, int32_t wdtype, double v)
{
    if (wdtype == ORACLE_F32)
        ((float*)base)[i] = (float)v;              /* C conversion: nearest-even */
    else
        ((uint16_t*)base)[i] = oracle_double_to_half(v);
}

/* Position of row r inside a held table, or -1 when it is not held. */
static int64_t held_row(const oracle_table* tb, int64_t r)
{
    if (tb->ids == NULL)
        return (r >= 0 && r < tb->n) ? r : -1;
    int64_t lo = 0, hi = tb->n;
    while (lo < hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if (tb->ids[mid] < r)
            lo = mid + 1;
        else
            hi = mid;
    }
    return (lo < tb->n && tb->ids[lo] == r) ? lo : -1;
}

/* ---------------------------------------------------------------------- */
/* Per-table prefix sums of the packed input format: table t's rows start at
 * element weights_offsets[t] = sum_{t'<t} rows*D, its output columns at
 * D_offsets[t] = sum_{t'<t} D, its keys at hash_size_cumsum[t] = sum rows. */
int oracle_layout(int32_t T, const int64_t* rows, const int32_t* dims,
                  int64_t* weights_offsets, int64_t* D_offsets, int64_t* hash_size_cumsum)
{
    if (T < 1 || !rows || !dims)
        return 1;
    int64_t w = 0, d = 0, h = 0;
    for (int32_t t = 0; t < T; ++t) {
        if (rows[t] < 0 || dims[t] < 1)
            return 1;
        if (weights_offsets) weights_offsets[t] = w;
        if (D_offsets) D_offsets[t] = d;
        if (hash_size_cumsum) hash_size_cumsum[t] = h;
        w += rows[t] * (int64_t)dims[t];
        d += dims[t];
        h += rows[t];
    }
    if (D_offsets) D_offsets[T] = d;
    if (hash_size_cumsum) hash_size_cumsum[T] = h;
    return 0;
}

static int check_inputs(int32_t T, int32_t B, const int64_t* rows,
                        const int64_t* indices, const int64_t* offsets)
{
    if (T < 1 || B < 0 || !rows || !offsets)
        return 1;
    int64_t nb = (int64_t)T * B;
    if (offsets[0] != 0)
        return 2;
    for (int64_t k = 0; k < nb; ++k)
        if (offsets[k + 1] < offsets[k])
            return 2;
    if (offsets[nb] > 0 && !indices)
        return 1;
    for (int32_t t = 0; t < T; ++t)
        for (int64_t j = offsets[(int64_t)t * B]; j < offsets[(int64_t)(t + 1) * B]; ++j)
            if (indices[j] < 0 || indices[j] >= rows[t])
                return 2;
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Forward: pooled sum of each bag (pooling 1: the sum divided by the bag's
 * length; an empty bag stays zero), written at the table's column offset. */
int oracle_forward(int32_t T, int32_t B, const int64_t* rows, const int32_t* dims,
                   int32_t wdtype, const oracle_table* tables,
                   const int64_t* indices, const int64_t* offsets,
                   const float* psw, const uint8_t* weighted,
                   const int64_t* bag_list, int64_t nbags, double* out, int32_t pooling)
{
    int rc = check_inputs(T, B, rows, indices, offsets);
    if (rc) return rc;
    if (!dims || !tables || !out || (wdtype != ORACLE_F32 && wdtype != ORACLE_F16))
        return 1;
    int64_t* Doff = (int64_t*)malloc(sizeof(int64_t) * (T + 1));
    oracle_layout(T, rows, dims, NULL, Doff, NULL);
    int32_t Dmax = 0;
    for (int32_t t = 0; t < T; ++t)
        if (dims[t] > Dmax) Dmax = dims[t];
    int64_t sumD = Doff[T];

    int64_t count = bag_list ? nbags : (int64_t)T * B;
    for (int64_t k = 0; k < count; ++k) {
        int64_t bag = bag_list ? bag_list[k] : k;
        if (bag < 0 || bag >= (int64_t)T * B) { free(Doff); return 1; }
    }
    int err = 0;
    /* bags are independent: each output element is written by one thread */
#pragma omp parallel for schedule(dynamic, 64) num_threads(g_threads) if (g_threads > 1)
    for (int64_t k = 0; k < count; ++k) {
        int64_t bag = bag_list ? bag_list[k] : k;
        int32_t t = (int32_t)(bag / B);
        int64_t b = bag % B;
        int32_t D = dims[t];
        double* dst = bag_list ? out + k * Dmax : out + b * sumD + Doff[t];
        for (int32_t d = 0; d < D; ++d)
            dst[d] = 0.0;                              /* an empty bag pools to zero */
        for (int64_t j = offsets[bag]; j < offsets[bag + 1]; ++j) {
            int64_t pos = held_row(&tables[t], indices[j]);
            if (pos < 0) {
#pragma omp atomic write
                err = 3;
                break;
            }
            double w = (psw && (!weighted || weighted[t])) ? (double)psw[j] : 1.0;
            for (int32_t d = 0; d < D; ++d)
                dst[d] += w * load_elem(tables[t].data, pos * D + d, wdtype);
        }
        int64_t len = offsets[bag + 1] - offsets[bag];
        if (pooling == ORACLE_POOL_MEAN && len > 0)
            for (int32_t d = 0; d < D; ++d)
                dst[d] /= (double)len;
    }
    free(Doff);
    return err;
}

/* ---------------------------------------------------------------------- */
/* Integer stage: linearized keys, sort by (key, lookup position), RLE,
 * classification into short and long runs. */
typedef struct { int64_t key, pos; } kp_t;

static int cmp_kp(const void* a, const void* b)
{
    const kp_t* x = (const kp_t*)a;
    const kp_t* y = (const kp_t*)b;
    if (x->key != y->key) return x->key < y->key ? -1 : 1;
    if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;
    return 0;
}

/* keys[j] = hash_size_cumsum[t(j)] + indices[j] for every lookup j. */
static void linear_keys(int32_t T, int32_t B, const int64_t* rows, const int64_t* indices,
                        const int64_t* offsets, int64_t* keys)
{
    int64_t base = 0;
    for (int32_t t = 0; t < T; ++t) {
        for (int64_t j = offsets[(int64_t)t * B]; j < offsets[(int64_t)(t + 1) * B]; ++j)
            keys[j] = base + indices[j];
        base += rows[t];
    }
}

int oracle_sort_rle(int32_t T, int32_t B, const int64_t* rows,
                    const int64_t* indices, const int64_t* offsets, int64_t tau,
                    int64_t* sorted_keys, int64_t* sorted_pos, int64_t* unique_keys,
                    int64_t* run_start, int64_t* run_len, int64_t* num_runs,
                    int64_t* short_runs, int64_t* num_short,
                    int64_t* long_runs, int64_t* num_long)
{
    int rc = check_inputs(T, B, rows, indices, offsets);
    if (rc) return rc;
    int64_t N = offsets[(int64_t)T * B];
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (N ? N : 1));
    kp_t* kp = (kp_t*)malloc(sizeof(kp_t) * (N ? N : 1));
    linear_keys(T, B, rows, indices, offsets, keys);
    for (int64_t j = 0; j < N; ++j) {
        kp[j].key = keys[j];
        kp[j].pos = j;
    }
    qsort(kp, (size_t)N, sizeof(kp_t), cmp_kp);
    int64_t* starts = (int64_t*)malloc(sizeof(int64_t) * (N + 1));
    int64_t R = 0, ns = 0, nl = 0;
    for (int64_t i = 0; i < N; ++i) {
        if (sorted_keys) sorted_keys[i] = kp[i].key;
        if (sorted_pos) sorted_pos[i] = kp[i].pos;
        if (i == 0 || kp[i].key != kp[i - 1].key) {
            if (unique_keys) unique_keys[R] = kp[i].key;
            starts[R] = i;
            ++R;
        }
    }
    starts[R] = N;
    for (int64_t r = 0; r < R; ++r) {
        /* run r spans from its first element to the next run's first */
        int64_t len = starts[r + 1] - starts[r];
        if (run_start) run_start[r] = starts[r];
        if (run_len) run_len[r] = len;
        if (len >= tau) {
            if (long_runs) long_runs[nl] = r;
            ++nl;
        } else {
            if (short_runs) short_runs[ns] = r;
            ++ns;
        }
    }
    if (num_runs) *num_runs = R;
    if (num_short) *num_short = ns;
    if (num_long) *num_long = nl;
    free(starts);
    free(kp);
    free(keys);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Backward + exact SGD for the requested rows: G = sum over lookups j of the
 * row of w_j * grad_output[b(j), D_offsets[t] : +D_t], accumulated in lookup
 * order (pooling 1: w_j divided by the length of j's bag, the derivative of
 * the mean); new = W[r] - lr * G. */
int oracle_backward_sgd(int32_t T, int32_t B, const int64_t* rows, const int32_t* dims,
                        int32_t wdtype, oracle_table* tables,
                        const int64_t* indices, const int64_t* offsets,
                        const float* psw, const uint8_t* weighted,
                        const float* grad_output, float lr,
                        const int64_t* keys, int64_t nkeys,
                        double* grad_rows, double* new_rows, int32_t write_back,
                        int32_t pooling)
{
    int rc = check_inputs(T, B, rows, indices, offsets);
    if (rc) return rc;
    if (!dims || !tables || (nkeys > 0 && (!keys || !grad_output)) ||
        (wdtype != ORACLE_F32 && wdtype != ORACLE_F16) || nkeys < 0)
        return 1;
    for (int64_t k = 1; k < nkeys; ++k)
        if (keys[k] <= keys[k - 1])
            return 1;
    int64_t* Doff = (int64_t*)malloc(sizeof(int64_t) * (T + 1));
    int64_t* hcs = (int64_t*)malloc(sizeof(int64_t) * (T + 1));
    oracle_layout(T, rows, dims, NULL, Doff, hcs);
    int32_t Dmax = 0;
    for (int32_t t = 0; t < T; ++t)
        if (dims[t] > Dmax) Dmax = dims[t];
    int64_t sumD = Doff[T];
    double* G = (double*)calloc((size_t)(nkeys ? nkeys : 1) * Dmax, sizeof(double));

    /* Every bag adds each of its lookups' weighted output-gradient slices into
     * the row the lookup read.  The requested keys are split into contiguous
     * ranges; a range's rows are summed by one thread, which walks, in lookup
     * order, the lookups of the tables the range touches (one range = the
     * whole loop when single-threaded), so every row's sum is in lookup order
     * whatever the thread count. */
    int64_t nranges = g_threads > 1 ? (int64_t)g_threads * 8 : 1;
    if (nranges > nkeys) nranges = nkeys > 0 ? nkeys : 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(g_threads) if (g_threads > 1)
    for (int64_t q = 0; q < nranges; ++q) {
        int64_t k0 = nkeys * q / nranges, k1 = nkeys * (q + 1) / nranges;
        if (k0 >= k1)
            continue;
        for (int32_t t = 0; t < T; ++t) {
            if (hcs[t + 1] <= keys[k0] || hcs[t] > keys[k1 - 1])
                continue;                            /* no key of this range in table t */
            int32_t D = dims[t];
            for (int64_t b = 0; b < B; ++b) {
                int64_t bag = (int64_t)t * B + b;
                for (int64_t j = offsets[bag]; j < offsets[bag + 1]; ++j) {
                    int64_t key = hcs[t] + indices[j];
                    int64_t lo = k0, hi = k1;        /* find key among this range's */
                    while (lo < hi) {
                        int64_t mid = lo + (hi - lo) / 2;
                        if (keys[mid] < key) lo = mid + 1; else hi = mid;
                    }
                    if (lo >= k1 || keys[lo] != key)
                        continue;
                    double w = (psw && (!weighted || weighted[t])) ? (double)psw[j] : 1.0;
                    if (pooling == ORACLE_POOL_MEAN)
                        w /= (double)(offsets[bag + 1] - offsets[bag]);
                    const float* g = grad_output + b * sumD + Doff[t];
                    double* acc = G + lo * Dmax;
                    for (int32_t d = 0; d < D; ++d)
                        acc[d] += w * (double)g[d];
                }
            }
        }
    }

    rc = 0;
    for (int64_t k = 0; k < nkeys; ++k)
        if (keys[k] < 0 || keys[k] >= hcs[T]) { rc = 1; break; }
    /* each key's row is updated on its own (rows are distinct) */
#pragma omp parallel for schedule(dynamic, 256) num_threads(g_threads) if (g_threads > 1 && rc == 0)
    for (int64_t k = 0; k < (rc == 0 ? nkeys : 0); ++k) {
        /* table of the key: the last t with hash_size_cumsum[t] <= key */
        int32_t t = 0;
        while (t + 1 < T && hcs[t + 1] <= keys[k])
            ++t;
        int64_t r = keys[k] - hcs[t];
        int64_t pos = held_row(&tables[t], r);
        if (pos < 0) {
#pragma omp atomic write
            rc = 3;
            continue;
        }
        int32_t D = dims[t];
        for (int32_t d = 0; d < D; ++d) {
            double g = G[k * Dmax + d];
            double w_new = load_elem(tables[t].data, pos * D + d, wdtype) - (double)lr * g;
            if (grad_rows) grad_rows[k * Dmax + d] = g;
            if (new_rows) new_rows[k * Dmax + d] = w_new;
            if (write_back) store_elem(tables[t].data, pos * D + d, wdtype, w_new);
        }
    }
    free(G);
    free(hcs);
    free(Doff);
    return rc;
}

/* ---------------------------------------------------------------------- */
/* Backward + exact row-wise Adagrad for the requested rows (section "Why the
 * backward is the hard half", where the article reads the update out of the
 * Triton kernel).  The row gradient G is the same finished sum as for SGD.
 * The row's one state value is raised by the mean over its D elements of
 * G[d]^2; that new value is kept in fp32 (the state's storage type, rounded
 * once) and the row steps by lr / (sqrt(state) + eps) times G.  eps is not
 * given on the pages; the caller passes it. */
int oracle_backward_adagrad(int32_t T, int32_t B, const int64_t* rows, const int32_t* dims,
                            int32_t wdtype, oracle_table* tables,
                            const int64_t* indices, const int64_t* offsets,
                            const float* psw, const uint8_t* weighted,
                            const float* grad_output, float lr, float eps,
                            const int64_t* keys, int64_t nkeys,
                            const float* state_in, float* state_out,
                            double* grad_rows, double* new_rows, int32_t write_back,
                            int32_t pooling)
{
    if (nkeys > 0 && (!state_in || !state_out))
        return 1;
    int32_t Dmax = 0;
    for (int32_t t = 0; dims && t < T; ++t)
        if (dims[t] > Dmax) Dmax = dims[t];
    /* the finished row gradients, exactly as the SGD definition sums them
     * (lr = 0 there: nothing is written back, only G is wanted) */
    double* G = (double*)calloc((size_t)(nkeys ? nkeys : 1) * (Dmax ? Dmax : 1), sizeof(double));
    int rc = oracle_backward_sgd(T, B, rows, dims, wdtype, tables, indices, offsets, psw,
                                 weighted, grad_output, 0.0f, keys, nkeys, G, NULL, 0, pooling);
    if (rc) { free(G); return rc; }
    int64_t* hcs = (int64_t*)malloc(sizeof(int64_t) * (T + 1));
    oracle_layout(T, rows, dims, NULL, NULL, hcs);
    for (int64_t k = 0; k < nkeys && rc == 0; ++k) {
        int32_t t = 0;
        while (t + 1 < T && hcs[t + 1] <= keys[k])
            ++t;
        int64_t pos = held_row(&tables[t], keys[k] - hcs[t]);
        if (pos < 0) { rc = 3; break; }
        int32_t D = dims[t];
        double sq = 0.0;
        for (int32_t d = 0; d < D; ++d)
            sq += G[k * Dmax + d] * G[k * Dmax + d];
        float state = (float)((double)state_in[k] + sq / (double)D);
        state_out[k] = state;
        double rate = (double)lr / (sqrt((double)state) + (double)eps);
        for (int32_t d = 0; d < D; ++d) {
            double g = G[k * Dmax + d];
            double w_new = load_elem(tables[t].data, pos * D + d, wdtype) - rate * g;
            if (grad_rows) grad_rows[k * Dmax + d] = g;
            if (new_rows) new_rows[k * Dmax + d] = w_new;
            if (write_back) store_elem(tables[t].data, pos * D + d, wdtype, w_new);
        }
    }
    free(hcs);
    free(G);
    return rc;
}
