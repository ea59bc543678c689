// C ABI of libtbe: argument validation, plan construction, kernel dispatch.
// Every entry point is declared and documented in include/tbe.h.
#include <mutex>
#include <new>

#include "tbe_internal.h"

using namespace tbe;

// Scratch of tbe_backward_sgd_noalloc: the backward's workspace for callers
// that cannot allocate.  Every GPU the library runs on holds its own copy
// until the process ends; all calls on one GPU share it.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int64_t kMaxD = 4096;

tbe_tuning default_tuning()
{
    tbe_tuning t{};
    t.tau = 64;               // long-run threshold (runs >= tau are split); measured
    t.chunk = 256;            // lookups per long-run chunk
    t.hist_mode = 0;          // auto
    t.hist_min_mean_len = 64; // histogram path pays once bags are this long
    t.fwd_bags_per_wave = 1;
    t.seg_slab_kib = 1024;   // grad_output slab per column block: a quarter of an XCD's L2
    t.sort_mode = 0;         // auto
    return t;
}

bool valid_dtype(int32_t wd, int32_t id)
{
    return (wd == TBE_F32 || wd == TBE_F16) && (id == TBE_I32 || id == TBE_I64);
}

tbe_status check_call(const tbe_plan* p, int32_t B, int64_t num_indices, const void* indices,
                      const void* offsets)
{
    if (!p || B < 0 || num_indices < 0) return TBE_EINVAL;
    if (B > 0 && !offsets) return TBE_EINVAL;
    if (num_indices > 0 && !indices) return TBE_EINVAL;
    if (num_indices >= (int64_t(1) << 30)) return TBE_ERANGE;
    if (int64_t(p->T) * B >= (int64_t(1) << 31)) return TBE_ERANGE;
    return TBE_OK;
}

bool use_hist(const tbe_plan* p, int32_t B, int64_t N)
{
    // a speed path: the gather kernel gives the same results (sum and mean)
    if (p->tuning.hist_mode == 1) return false;
    bool any = false;
    for (int t = 0; t < p->T; ++t) any |= (p->h_tables[t].flags & TD_HIST_OK) != 0;
    if (!any) return false;
    if (p->tuning.hist_mode == 2) return true;
    const int64_t bags = int64_t(p->T) * B;
    return bags > 0 && N >= int64_t(p->tuning.hist_min_mean_len) * bags;
}

}  // namespace

extern "C" {

int32_t tbe_version(void) { return 101; }

const char* tbe_status_string(tbe_status s)
{
    switch (s) {
    case TBE_OK: return "ok";
    case TBE_EINVAL: return "invalid argument";
    case TBE_ERANGE: return "size out of supported range";
    case TBE_ENOMEM: return "device allocation failed";
    case TBE_EHIP: return "HIP runtime error";
    case TBE_ENOTSUP: return "unsupported combination";
    }
    return "unknown status";
}

tbe_status tbe_plan_create(int32_t T, const int64_t* rows, const int32_t* dims,
                           int32_t weight_dtype, int32_t index_dtype, const uint8_t* weighted,
                           tbe_plan** out)
{
    if (!out) return TBE_EINVAL;
    *out = nullptr;
    if (T < 1 || !rows || !dims || !valid_dtype(weight_dtype, index_dtype)) return TBE_EINVAL;
    tbe_plan* p = new (std::nothrow) tbe_plan();
    if (!p) return TBE_ENOMEM;
    p->T = T;
    p->wdtype = weight_dtype;
    p->idtype = index_dtype;
    p->tuning = default_tuning();
    int64_t w = 0, dsum = 0, h = 0;
    for (int t = 0; t < T; ++t) {
        if (rows[t] < 0 || dims[t] < 1) { delete p; return TBE_EINVAL; }
        if (dims[t] > kMaxD) { delete p; return TBE_ERANGE; }
        p->rows.push_back(rows[t]);
        p->dims.push_back(dims[t]);
        p->weighted.push_back(weighted ? (weighted[t] ? 1 : 0) : 1);
        p->w_off.push_back(w);
        p->D_off.push_back(dsum);
        p->hash_off.push_back(h);
        w += rows[t] * dims[t];
        dsum += dims[t];
        h += rows[t];
        if (dims[t] > p->max_D) p->max_D = dims[t];
    }
    p->D_off.push_back(dsum);
    p->hash_off.push_back(h);
    if (h >= (int64_t(1) << 32) || dsum >= (int64_t(1) << 31)) { delete p; return TBE_ERANGE; }
    p->sum_rows = h;
    p->sum_D = static_cast<int32_t>(dsum);

    p->h_tables.resize(T);
    std::vector<uint32_t> hoff(T + 1);
    for (int t = 0; t < T; ++t) {
        TableDesc& d = p->h_tables[t];
        d.w_off = p->w_off[t];
        d.hash_off = static_cast<uint32_t>(p->hash_off[t]);
        d.rows = static_cast<uint32_t>(p->rows[t]);
        d.D = p->dims[t];
        d.out_off = static_cast<int32_t>(p->D_off[t]);
        d.flags = 0;
        if (p->weighted[t]) d.flags |= TD_WEIGHTED;
        if (weight_dtype == TBE_F16 && p->rows[t] >= 1 && p->rows[t] <= kHistMaxRows &&
            p->dims[t] <= kHistMaxD)
            d.flags |= TD_HIST_OK;
        d.pad = 0;
        hoff[t] = static_cast<uint32_t>(p->hash_off[t]);
    }
    hoff[T] = static_cast<uint32_t>(h);
    if (hipGetDevice(&p->device) != hipSuccess) { delete p; return TBE_EHIP; }
    if (hipMalloc(&p->d_tables, sizeof(TableDesc) * T) != hipSuccess) {
        delete p;
        return TBE_ENOMEM;
    }
    if (hipMalloc(&p->d_hash_off, sizeof(uint32_t) * (T + 1)) != hipSuccess) {
        (void)hipFree(p->d_tables);
        delete p;
        return TBE_ENOMEM;
    }
    if (hipMemcpy(p->d_tables, p->h_tables.data(), sizeof(TableDesc) * T,
                  hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(p->d_hash_off, hoff.data(), sizeof(uint32_t) * (T + 1),
                  hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(p->d_tables);
        (void)hipFree(p->d_hash_off);
        delete p;
        return TBE_EHIP;
    }
    *out = p;
    return TBE_OK;
}

void tbe_plan_destroy(tbe_plan* p)
{
    if (!p) return;
    (void)hipFree(p->d_tables);
    (void)hipFree(p->d_hash_off);
    delete p;
}

tbe_status tbe_plan_layout(const tbe_plan* p, int64_t* weights_offsets, int64_t* D_offsets,
                           int64_t* hash_size_cumsum)
{
    if (!p) return TBE_EINVAL;
    for (int t = 0; t <= p->T; ++t) {
        if (weights_offsets && t < p->T) weights_offsets[t] = p->w_off[t];
        if (D_offsets) D_offsets[t] = p->D_off[t];
        if (hash_size_cumsum) hash_size_cumsum[t] = p->hash_off[t];
    }
    return TBE_OK;
}

tbe_status tbe_get_tuning(const tbe_plan* p, tbe_tuning* t)
{
    if (!p || !t) return TBE_EINVAL;
    *t = p->tuning;
    return TBE_OK;
}

tbe_status tbe_plan_set_pooling(tbe_plan* p, int32_t pooling)
{
    if (!p || (pooling != TBE_POOL_SUM && pooling != TBE_POOL_MEAN)) return TBE_EINVAL;
    p->pooling = pooling;
    return TBE_OK;
}

tbe_status tbe_set_tuning(tbe_plan* p, const tbe_tuning* t)
{
    if (!p || !t) return TBE_EINVAL;
    if (t->tau < 1 || t->chunk < 1 || t->hist_mode < 0 || t->hist_mode > 2 ||
        t->hist_min_mean_len < 0 || t->fwd_bags_per_wave < 1 || t->fwd_bags_per_wave > 1024 ||
        t->seg_slab_kib < 0 || t->sort_mode < 0 || t->sort_mode > 2)
        return TBE_EINVAL;
    p->tuning = *t;
    return TBE_OK;
}

tbe_status tbe_forward(const tbe_plan* p, int32_t B, const void* weights, const void* indices,
                       int64_t num_indices, const void* offsets, const float* psw, float* output,
                       void* stream)
{
    tbe_status st = check_call(p, B, num_indices, indices, offsets);
    if (st != TBE_OK) return st;
    if (B == 0) return TBE_OK;
    if (!weights || !output) return TBE_EINVAL;
    const size_t wbytes = p->wdtype == TBE_F32 ? 4 : 2;
    int vec = static_cast<int>(16 / wbytes);
    for (int t = 0; t < p->T; ++t)
        while (p->dims[t] % vec) vec >>= 1;
    while (vec > 1 && (reinterpret_cast<uintptr_t>(weights) % (vec * wbytes) ||
                       reinterpret_cast<uintptr_t>(output) % (vec * 4)))
        vec >>= 1;
    FwdArgs a{p, B, weights, indices, offsets, psw, output, vec, use_hist(p, B, num_indices),
              p->pooling == TBE_POOL_MEAN, static_cast<hipStream_t>(stream)};
    stage_mark(p, 0, a.stream);
    tbe_status st2 = TBE_OK;
    // the gather kernel is launched only if some table is not pooled by the
    // histogram kernel (the same routing as in both kernels)
    bool gather = !a.hist_active;
    for (int t = 0; t < p->T && !gather; ++t) {
        const int32_t f = p->h_tables[t].flags;
        gather = !(f & TD_HIST_OK) || (psw && (f & TD_WEIGHTED));
    }
    if (a.hist_active && launch_fwd_hist(a) != hipSuccess) st2 = TBE_EHIP;
    if (st2 == TBE_OK && gather && launch_fwd_gather(a) != hipSuccess) st2 = TBE_EHIP;
    stage_mark(p, 1, a.stream);
    const_cast<tbe_plan*>(p)->n_stage_ev = 0;
    return st2;
}

size_t tbe_backward_workspace_bytes(const tbe_plan* p, int32_t B, int64_t num_indices)
{
    if (check_call(p, B, num_indices, reinterpret_cast<const void*>(1),
                   reinterpret_cast<const void*>(1)) != TBE_OK)
        return 0;
    return bwd_layout(p, B, num_indices).total;
}

static tbe_status prepare_bwd(const tbe_plan* p, int32_t B, const void* indices,
                              int64_t num_indices, const void* offsets, void* workspace,
                              size_t workspace_bytes, void* stream, BwdArgs& a)
{
    tbe_status st = check_call(p, B, num_indices, indices, offsets);
    if (st != TBE_OK) return st;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255)) return TBE_EINVAL;
    a.plan = p;
    a.B = B;
    a.N = num_indices;
    a.indices = indices;
    a.offsets = offsets;
    a.psw = nullptr;
    a.grad = nullptr;
    a.weights = nullptr;
    a.lr = 0.f;
    a.state = nullptr;
    a.eps = 0.f;
    a.ws = static_cast<char*>(workspace);
    a.L = bwd_layout(p, B, num_indices);
    a.stream = static_cast<hipStream_t>(stream);
    a.final_buf = 0;
    a.payload_pairs = 0;
    if (workspace_bytes < a.L.total) return TBE_EINVAL;
    return TBE_OK;
}

tbe_status tbe_backward_prepare(const tbe_plan* p, int32_t B, const void* indices,
                                int64_t num_indices, const void* offsets, const float* psw,
                                void* workspace, size_t workspace_bytes, void* stream)
{
    if (p && B == 0 && num_indices >= 0) return TBE_OK;
    BwdArgs a;
    tbe_status st = prepare_bwd(p, B, indices, num_indices, offsets, workspace,
                                workspace_bytes, stream, a);
    if (st != TBE_OK) return st;
    if (num_indices == 0) return TBE_OK;
    a.psw = psw;
    stage_mark(p, 0, a.stream);
    st = run_sort_rle(a, false) == hipSuccess ? TBE_OK : TBE_EHIP;
    const_cast<tbe_plan*>(p)->n_stage_ev = 0;
    return st;
}

// The update's own arguments: SGD (state == nullptr) or row-wise Adagrad.
static tbe_status set_update(BwdArgs& a, void* weights, const float* grad_output, float lr,
                             float* state, float eps, bool adagrad)
{
    if (!weights || !grad_output) return TBE_EINVAL;
    a.grad = grad_output;
    a.weights = weights;
    a.lr = lr;
    if (!adagrad) return TBE_OK;
    if (!state || (reinterpret_cast<uintptr_t>(state) & 3) || !(eps >= 0.f)) return TBE_EINVAL;
    a.state = state;
    a.eps = eps;
    return adagrad_supported(a) ? TBE_OK : TBE_ENOTSUP;
}

static tbe_status apply_half(const tbe_plan* p, int32_t B, int64_t num_indices, int32_t weighted,
                             void* weights, float* state, const float* grad_output, float lr,
                             float eps, bool adagrad, void* workspace, size_t workspace_bytes,
                             void* stream)
{
    if (p && B == 0 && num_indices >= 0) return TBE_OK;
    BwdArgs a;
    // indices / offsets are not read here; any non-null stand-in passes the checks
    tbe_status st = prepare_bwd(p, B, workspace, num_indices, workspace, workspace,
                                workspace_bytes, stream, a);
    if (st != TBE_OK) return st;
    st = set_update(a, weights, grad_output, lr, state, eps, adagrad);
    if (st != TBE_OK) return st;
    if (num_indices == 0) return TBE_OK;
    a.final_buf = a.L.npasses & 1;   // each radix pass swaps the ping-pong buffers
    // (sample, weight) payload: per-sample weights, or mean pooling's 1 / length
    a.payload_pairs = weighted != 0 || p->pooling == TBE_POOL_MEAN;
    st = run_segment_sgd(a) == hipSuccess ? TBE_OK : TBE_EHIP;
    const_cast<tbe_plan*>(p)->n_stage_ev = 0;
    return st;
}

static tbe_status backward_whole(const tbe_plan* p, int32_t B, void* weights, float* state,
                                 const void* indices, int64_t num_indices, const void* offsets,
                                 const float* psw, const float* grad_output, float lr, float eps,
                                 bool adagrad, void* workspace, size_t workspace_bytes,
                                 void* stream)
{
    if (p && B == 0 && num_indices >= 0) return TBE_OK;
    BwdArgs a;
    tbe_status st = prepare_bwd(p, B, indices, num_indices, offsets, workspace,
                                workspace_bytes, stream, a);
    if (st != TBE_OK) return st;
    st = set_update(a, weights, grad_output, lr, state, eps, adagrad);
    if (st != TBE_OK) return st;
    if (num_indices == 0) return TBE_OK;
    a.psw = psw;
    stage_mark(p, 0, a.stream);
    tbe_status st2 = TBE_OK;
    if (run_sort_rle(a, false) != hipSuccess) st2 = TBE_EHIP;
    else if (run_segment_sgd(a) != hipSuccess) st2 = TBE_EHIP;
    const_cast<tbe_plan*>(p)->n_stage_ev = 0;
    return st2;
}

tbe_status tbe_backward_apply(const tbe_plan* p, int32_t B, int64_t num_indices, int32_t weighted,
                              void* weights, const float* grad_output, float lr,
                              void* workspace, size_t workspace_bytes, void* stream)
{
    return apply_half(p, B, num_indices, weighted, weights, nullptr, grad_output, lr, 0.f, false,
                      workspace, workspace_bytes, stream);
}

tbe_status tbe_backward_apply_adagrad(const tbe_plan* p, int32_t B, int64_t num_indices,
                                      int32_t weighted, void* weights, float* state,
                                      const float* grad_output, float lr, float eps,
                                      void* workspace, size_t workspace_bytes, void* stream)
{
    return apply_half(p, B, num_indices, weighted, weights, state, grad_output, lr, eps, true,
                      workspace, workspace_bytes, stream);
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch copy, looked up once per device with
// that device current (the host-side name `scratch` is not a device address).
tbe_status scratch_on_current_device(void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TBE_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return TBE_EHIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return TBE_OK;
}
}  // namespace

tbe_status tbe_backward_sgd_noalloc(const tbe_plan* p, int32_t B, void* weights,
                                    const void* indices, int64_t num_indices, const void* offsets,
                                    const float* psw, const float* grad_output, float lr,
                                    uint32_t* error_word, void* stream)
{
    tbe_status st = check_call(p, B, num_indices, indices, offsets);
    if (st != TBE_OK) return st;
    if (!weights || !grad_output || (reinterpret_cast<uintptr_t>(error_word) & 3))
        return TBE_EINVAL;
    if (bwd_layout(p, B, num_indices).total > kScratchBytes) return TBE_ERANGE;
    if (B == 0 || num_indices == 0) {
        // nothing to update; the caller's error word still gets a value
        if (error_word) {
            void* ws = nullptr;
            st = scratch_on_current_device(&ws);
            if (st != TBE_OK) return st;
            const hipStream_t s = static_cast<hipStream_t>(stream);
            if (launch_workspace_init(ws, s) != hipSuccess ||
                launch_workspace_status(ws, error_word, s) != hipSuccess)
                return TBE_EHIP;
        }
        return TBE_OK;
    }
    void* ws = nullptr;
    st = scratch_on_current_device(&ws);
    if (st != TBE_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // the control block must start at zero: the previous call on this GPU may
    // have left its error word set (a fill kernel, so a captured graph holds
    // no memset node)
    if (launch_workspace_init(ws, s) != hipSuccess) return TBE_EHIP;
    st = backward_whole(p, B, weights, nullptr, indices, num_indices, offsets, psw, grad_output,
                        lr, 0.f, false, ws, kScratchBytes, stream);
    if (st == TBE_OK && error_word && launch_workspace_status(ws, error_word, s) != hipSuccess)
        st = TBE_EHIP;
    return st;
}

size_t tbe_backward_noalloc_max_bytes(void) { return kScratchBytes; }

tbe_status tbe_backward_sgd(const tbe_plan* p, int32_t B, void* weights, const void* indices,
                            int64_t num_indices, const void* offsets, const float* psw,
                            const float* grad_output, float lr, void* workspace,
                            size_t workspace_bytes, void* stream)
{
    return backward_whole(p, B, weights, nullptr, indices, num_indices, offsets, psw, grad_output,
                          lr, 0.f, false, workspace, workspace_bytes, stream);
}

tbe_status tbe_backward_adagrad(const tbe_plan* p, int32_t B, void* weights, float* state,
                                const void* indices, int64_t num_indices, const void* offsets,
                                const float* psw, const float* grad_output, float lr, float eps,
                                void* workspace, size_t workspace_bytes, void* stream)
{
    return backward_whole(p, B, weights, state, indices, num_indices, offsets, psw, grad_output,
                          lr, eps, true, workspace, workspace_bytes, stream);
}

tbe_status tbe_sort_rle(const tbe_plan* p, int32_t B, const void* indices, int64_t num_indices,
                        const void* offsets, void* workspace, size_t workspace_bytes,
                        tbe_sort_view* view, void* stream)
{
    if (!view) return TBE_EINVAL;
    BwdArgs a;
    tbe_status st = prepare_bwd(p, B, indices, num_indices, offsets, workspace,
                                workspace_bytes, stream, a);
    if (st != TBE_OK) return st;
    const hipError_t e = run_sort_rle(a, true);
    const_cast<tbe_plan*>(p)->n_stage_ev = 0;
    if (e != hipSuccess) return TBE_EHIP;
    char* ws = a.ws;
    const BwdLayout& L = a.L;
    view->sorted_keys = reinterpret_cast<uint32_t*>(ws + L.off_keys[a.final_buf]);
    view->sorted_pos = reinterpret_cast<uint32_t*>(ws + L.off_vals[a.final_buf]);
    view->unique_keys = reinterpret_cast<uint32_t*>(ws + L.off_unique);
    view->run_start = reinterpret_cast<uint32_t*>(ws + L.off_run_start);
    view->run_len = reinterpret_cast<uint32_t*>(ws + L.off_run_len);
    view->short_runs = reinterpret_cast<uint32_t*>(ws + L.off_short);
    view->long_runs = reinterpret_cast<uint32_t*>(ws + L.off_long);
    view->counts = reinterpret_cast<uint32_t*>(ws + L.off_ctl) + kCtlCounts;
    return TBE_OK;
}

tbe_status tbe_set_stage_events(tbe_plan* p, void* const* events, int32_t n)
{
    if (!p || n < 0) return TBE_EINVAL;
    if (!events) n = 0;
    if (n > 8) n = 8;
    for (int k = 0; k < 8; ++k) p->stage_ev[k] = k < n ? static_cast<hipEvent_t>(events[k]) : nullptr;
    p->n_stage_ev = n;
    return TBE_OK;
}

tbe_status tbe_workspace_init(void* workspace, size_t workspace_bytes, void* stream)
{
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255) ||
        workspace_bytes < size_t(kCtlWords) * 4)
        return TBE_EINVAL;
    if (launch_workspace_init(workspace, static_cast<hipStream_t>(stream)) != hipSuccess)
        return TBE_EHIP;
    return TBE_OK;
}

tbe_status tbe_workspace_status(const void* workspace, size_t workspace_bytes,
                                uint32_t* error_word, void* stream)
{
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255) ||
        workspace_bytes < size_t(kCtlWords) * 4 || !error_word ||
        (reinterpret_cast<uintptr_t>(error_word) & 3))
        return TBE_EINVAL;
    if (launch_workspace_status(workspace, error_word, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return TBE_EHIP;
    return TBE_OK;
}

tbe_status tbe_bounds_check(const tbe_plan* p, int32_t B, const void* indices,
                            int64_t num_indices, const void* offsets, int64_t* error_count,
                            void* stream)
{
    tbe_status st = check_call(p, B, num_indices, indices, offsets);
    if (st != TBE_OK) return st;
    if (!error_count) return TBE_EINVAL;
    if (launch_bounds_check(p, B, indices, num_indices, offsets, error_count,
                            static_cast<hipStream_t>(stream)) != hipSuccess)
        return TBE_EHIP;
    return TBE_OK;
}

}  // extern "C"
