// C-ABI front end of the q4gsw library: validation, route selection and launches.
//
// Validation runs on the host before any HIP call, so every error path can be
// exercised without a GPU.  Route selection follows the pages' pattern of a
// geometry predicate with a fallback to the ordinary route (WebGPU BK64 QKV PR
// body) and of route attestation for test harnesses (the WebGPU SDPA routing PR
// body in the same stack): q4gsw_route reports the route a call takes.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "../../include/q4gsw.h"
#include "internal.h"

using namespace q4gsw;

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 30;
constexpr int64_t kMaxM = int64_t(1) << 23;

// Per-call choices (q4gsw_options), validated: route family, forward block rows, K splits.
struct Opts {
    int32_t route = Q4GSW_ROUTE_NONE;
    int32_t rows = 0;
    int32_t splits = 0;
};

q4gsw_status read_opts(const q4gsw_options* o, Opts* out) {
    *out = Opts{};
    if (!o) return Q4GSW_OK;
    if (o->route < Q4GSW_ROUTE_NONE || o->route > Q4GSW_ROUTE_DQ8CA) return Q4GSW_E_ROUTE;
    if (o->tile_rows != 0 && o->tile_rows != 64 && o->tile_rows != 128) return Q4GSW_E_SHAPE;
    if (o->splits < 0 || o->splits > 64) return Q4GSW_E_SHAPE;
    out->route = o->route;
    out->rows = o->tile_rows;
    out->splits = o->splits;
    return Q4GSW_OK;
}

int esize(int32_t dt) { return dt == Q4GSW_F32 ? 4 : 2; }
bool act_dtype_ok(int32_t dt) { return dt == Q4GSW_F32 || dt == Q4GSW_F16 || dt == Q4GSW_BF16; }
bool scale_dtype_ok(int32_t dt) { return dt == Q4GSW_F32 || dt == Q4GSW_F16; }

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};
Range range_of(const void* p, uint64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

q4gsw_status check_desc(const q4gsw_weight* w) {
    if (!w) return Q4GSW_E_NULL;
    if (w->magic != Q4GSW_MAGIC || w->version != Q4GSW_LAYOUT_VERSION) return Q4GSW_E_DESC;
    if (w->N < 1 || w->K < 1 || w->N > kMaxDim || w->K > kMaxDim || w->group_size < 1 ||
        w->K % w->group_size != 0)
        return Q4GSW_E_DESC;
    if (!scale_dtype_ok(w->scale_dtype)) return Q4GSW_E_DESC;
    const Layout L = make_layout(w->N, w->K, w->group_size, esize(w->scale_dtype));
    if (w->n_pad != L.n_pad || w->k_pad != L.k_pad || w->g_pad != L.g_pad || w->nibble_offset != L.nibble_offset ||
        w->scale_offset != L.scale_offset || w->bytes < L.total)
        return Q4GSW_E_DESC;
    if (!w->data) return Q4GSW_E_NULL;
    return Q4GSW_OK;
}

WView view_of(const q4gsw_weight* w) {
    WView v;
    v.nib = static_cast<const uint8_t*>(w->data) + w->nibble_offset;
    v.scales = static_cast<const uint8_t*>(w->data) + w->scale_offset;
    v.scale_f16 = w->scale_dtype == Q4GSW_F16;
    v.N = w->N;
    v.K = w->K;
    v.gs = w->group_size;
    v.n_pad = w->n_pad;
    v.k_pad = w->k_pad;
    v.g_pad = w->g_pad;
    return v;
}

bool fold_ok(const q4gsw_weight* w) { return (w->flags & Q4GSW_FLAG_FOLD_F16) != 0; }

enum Kind { kGeneric, kSmallM, kMfma };

Kind route_kind(int32_t route) {
    switch (route) {
        case Q4GSW_ROUTE_GENERIC: return kGeneric;
        case Q4GSW_ROUTE_GEMV:
        case Q4GSW_ROUTE_BWD_GEMV: return kSmallM;
        default: return kMfma;
    }
}

// Route of a forward (or QKV) call; Q4GSW_ROUTE_NONE with *err set when a forced route cannot serve it.
int32_t pick_fwd(const q4gsw_weight* w, int64_t M, int32_t dt, bool qkv, int32_t forced, q4gsw_status* err) {
    const WView v = view_of(w);
    const bool small_ok = M <= 8 && w->group_size % 8 == 0;
    const bool mfma_ok = gemm_fwd_supported(v, dt, fold_ok(w));
    auto mfma_route = [&]() -> int32_t {
        if (qkv) return Q4GSW_ROUTE_QKV_FUSED;
        if (dt == Q4GSW_F32) return Q4GSW_ROUTE_GEMM_SPLIT;
        if (dt == Q4GSW_F16 && w->scale_dtype == Q4GSW_F16 && fold_ok(w)) return Q4GSW_ROUTE_GEMM_FOLD;
        return Q4GSW_ROUTE_GEMM_GROUP;
    };
    *err = Q4GSW_OK;
    if (forced != Q4GSW_ROUTE_NONE) {
        switch (route_kind(forced)) {
            case kGeneric: return Q4GSW_ROUTE_GENERIC;
            case kSmallM:
                if (small_ok) return Q4GSW_ROUTE_GEMV;
                break;
            case kMfma:
                if (mfma_ok) return mfma_route();
                break;
        }
        *err = Q4GSW_E_ROUTE;
        return Q4GSW_ROUTE_NONE;
    }
    if (small_ok) return Q4GSW_ROUTE_GEMV;
    if (mfma_ok) return mfma_route();
    return Q4GSW_ROUTE_GENERIC;
}

int32_t pick_bwd(const q4gsw_weight* w, int64_t M, int32_t dt, int32_t forced, q4gsw_status* err) {
    const WView v = view_of(w);
    const bool small_ok = M <= 8 && w->group_size % 8 == 0;
    const bool mfma_ok = gemm_bwd_supported(v, dt, fold_ok(w));
    int32_t mfma_route = Q4GSW_ROUTE_NONE;
    if (mfma_ok) {
        const BwdPlan bp = plan_gemm_bwd(v, dt, fold_ok(w), M);
        mfma_route = (bp.v1 || bp.mode == kModeFold) ? Q4GSW_ROUTE_BWD_FOLD
                     : bp.mode == kModeBSplit         ? Q4GSW_ROUTE_BWD_BSPLIT
                                                      : Q4GSW_ROUTE_BWD_SPLIT;
    }
    *err = Q4GSW_OK;
    if (forced != Q4GSW_ROUTE_NONE) {
        switch (route_kind(forced)) {
            case kGeneric: return Q4GSW_ROUTE_GENERIC;
            case kSmallM:
                if (small_ok) return Q4GSW_ROUTE_BWD_GEMV;
                break;
            case kMfma:
                if (mfma_ok) return mfma_route;
                break;
        }
        *err = Q4GSW_E_ROUTE;
        return Q4GSW_ROUTE_NONE;
    }
    if (small_ok) return Q4GSW_ROUTE_BWD_GEMV;
    if (mfma_ok) return mfma_route;
    return Q4GSW_ROUTE_GENERIC;
}

uint64_t fwd_ws_bytes(const q4gsw_weight* w, int64_t M, int32_t dt, int32_t route, const Opts& o) {
    const WView v = view_of(w);
    if (route == Q4GSW_ROUTE_GEMV) {
        const int s = gemv_fwd_splits(v, M);
        return s > 1 ? (uint64_t)s * M * v.n_pad * 4 : 0;
    }
    if (route == Q4GSW_ROUTE_GEMM_FOLD || route == Q4GSW_ROUTE_GEMM_GROUP || route == Q4GSW_ROUTE_GEMM_SPLIT) {
        FwdSeg seg{v, nullptr};
        return (uint64_t)plan_gemm_fwd(&seg, 1, dt, fold_ok(w), M, o.rows, o.splits).ws_bytes;
    }
    return 0;
}

uint64_t bwd_ws_bytes(const q4gsw_weight* w, int64_t M, int32_t dt, int32_t route, const Opts& o) {
    const WView v = view_of(w);
    if (route == Q4GSW_ROUTE_BWD_GEMV) {
        const int s = gemv_bwd_splits(v, M);
        return s > 1 ? (uint64_t)s * M * v.k_pad * 4 : 0;
    }
    if (route == Q4GSW_ROUTE_BWD_FOLD || route == Q4GSW_ROUTE_BWD_SPLIT || route == Q4GSW_ROUTE_BWD_BSPLIT)
        return (uint64_t)plan_gemm_bwd(v, dt, fold_ok(w), M, o.splits).ws_bytes;
    return 0;
}

q4gsw_status check_qkv_descs(const q4gsw_weight* wq, const q4gsw_weight* wk, const q4gsw_weight* wv) {
    q4gsw_status st;
    if ((st = check_desc(wq)) != Q4GSW_OK) return st;
    if ((st = check_desc(wk)) != Q4GSW_OK) return st;
    if ((st = check_desc(wv)) != Q4GSW_OK) return st;
    const q4gsw_weight* ws[3] = {wq, wk, wv};
    for (int i = 1; i < 3; ++i) {
        if (ws[i]->K != wq->K || ws[i]->group_size != wq->group_size || ws[i]->scale_dtype != wq->scale_dtype ||
            fold_ok(ws[i]) != fold_ok(wq))
            return Q4GSW_E_DESC;
    }
    return Q4GSW_OK;
}

uint64_t qkv_ws_bytes(const q4gsw_weight* const w[3], int64_t M, int32_t dt, int32_t route, const Opts& o) {
    if (route == Q4GSW_ROUTE_QKV_FUSED) {
        FwdSeg segs[3];
        for (int i = 0; i < 3; ++i) segs[i] = FwdSeg{view_of(w[i]), nullptr};
        return (uint64_t)plan_gemm_fwd(segs, 3, dt, fold_ok(w[0]), M, o.rows, o.splits).ws_bytes;
    }
    uint64_t b = 0;
    for (int i = 0; i < 3; ++i) {
        const uint64_t x = fwd_ws_bytes(w[i], M, dt, route, o);
        b = x > b ? x : b;
    }
    return b;
}

q4gsw_status hip_status(hipError_t e) { return e == hipSuccess ? Q4GSW_OK : Q4GSW_E_HIP; }

// epi: a low-rank term the MFMA route adds in its reduction or epilogue; *epi_done tells whether
// this call applied it (the other routes leave it to the caller).
q4gsw_status run_fwd(const q4gsw_weight* w, const void* x, int32_t dt, int64_t M, float* y, void* ws,
                     int32_t route, const Opts& o, hipStream_t s, const LowRankEpi* epi = nullptr,
                     bool* epi_done = nullptr) {
    if (epi_done) *epi_done = false;
    const WView v = view_of(w);
    switch (route) {
        case Q4GSW_ROUTE_GENERIC: return hip_status(launch_generic_fwd(v, x, dt, M, y, s));
        case Q4GSW_ROUTE_GEMV: {
            const int splits = gemv_fwd_splits(v, M);
            if (splits == 1) return hip_status(launch_gemv_fwd(v, x, dt, M, y, 1, s));
            float* part = static_cast<float*>(ws);
            hipError_t e = launch_gemv_fwd(v, x, dt, M, part, splits, s);
            if (e == hipSuccess) e = launch_reduce_splits(part, splits, M, v.N, v.n_pad, y, v.N, s);
            return hip_status(e);
        }
        default: {
            FwdSeg seg{v, y};
            const FwdPlan plan = plan_gemm_fwd(&seg, 1, dt, fold_ok(w), M, o.rows, o.splits);
            return hip_status(launch_gemm_fwd(&seg, 1, x, dt, M, plan, static_cast<float*>(ws), s, epi, epi_done));
        }
    }
}

// epi: a low-rank term for the split reduction of the MFMA routes; *epi_done tells whether this
// call applied it (routes and plans without that reduction leave it to the caller).
q4gsw_status run_bwd(const q4gsw_weight* w, const void* d_out, int32_t g_dtype, int64_t M, float* d_x, void* ws,
                     int32_t route, const Opts& o, hipStream_t s, const LowRankEpi* epi = nullptr,
                     bool* epi_done = nullptr) {
    if (epi_done) *epi_done = false;
    const WView v = view_of(w);
    switch (route) {
        case Q4GSW_ROUTE_GENERIC: return hip_status(launch_generic_bwd(v, d_out, g_dtype, M, d_x, s));
        case Q4GSW_ROUTE_BWD_GEMV: {
            const int splits = gemv_bwd_splits(v, M);
            if (splits == 1) return hip_status(launch_gemv_bwd(v, d_out, g_dtype, M, d_x, 1, s));
            float* part = static_cast<float*>(ws);
            hipError_t e = launch_gemv_bwd(v, d_out, g_dtype, M, part, splits, s);
            if (e == hipSuccess) e = launch_reduce_splits(part, splits, M, v.K, v.k_pad, d_x, v.K, s);
            return hip_status(e);
        }
        default: {
            const BwdPlan plan = plan_gemm_bwd(v, g_dtype, fold_ok(w), M, o.splits);
            const bool fuse = epi && !plan.v1 && plan.splits > 1;
            if (fuse && epi_done) *epi_done = true;
            return hip_status(launch_gemm_bwd(v, d_out, g_dtype, M, d_x, plan, static_cast<float*>(ws), s,
                                              fuse ? epi : nullptr));
        }
    }
}

bool ws_ok(const void* ws, uint64_t ws_bytes, uint64_t need) {
    return need == 0 || (ws && ws_bytes >= need && (reinterpret_cast<uintptr_t>(ws) & 255u) == 0);
}

// Forward validation shared by q4gsw_linear_fwd_ex and the allocation-free forward: descriptor,
// pointers, sizes, dtype and route; *route and *need are set on success.
q4gsw_status prepare_fwd(const q4gsw_weight* w, const void* x, int32_t x_dtype, int64_t M, const float* y,
                         const Opts& o, int32_t* route, uint64_t* need) {
    q4gsw_status st = check_desc(w);
    if (st != Q4GSW_OK) return st;
    if (!x || !y) return Q4GSW_E_NULL;
    if (M < 1 || M > kMaxM) return Q4GSW_E_SHAPE;
    if (!act_dtype_ok(x_dtype)) return Q4GSW_E_DTYPE;
    *route = pick_fwd(w, M, x_dtype, false, o.route, &st);
    if (st != Q4GSW_OK) return st;
    *need = fwd_ws_bytes(w, M, x_dtype, *route, o);
    return Q4GSW_OK;
}

// Overlap checks of a forward call whose workspace is ws[0, need).
q4gsw_status fwd_alias(const q4gsw_weight* w, const void* x, int32_t x_dtype, int64_t M, const float* y,
                       const void* ws, uint64_t need) {
    const Range yr = range_of(y, (uint64_t)M * w->N * 4);
    const Range xr = range_of(x, (uint64_t)M * w->K * esize(x_dtype));
    const Range wr = range_of(w->data, w->bytes);
    if (overlap(yr, xr) || overlap(yr, wr)) return Q4GSW_E_ALIAS;
    if (need > 0) {
        const Range sr = range_of(ws, need);
        if (overlap(yr, sr) || overlap(sr, wr) || overlap(sr, xr)) return Q4GSW_E_ALIAS;
    }
    return Q4GSW_OK;
}

// ---- the allocation-free forward's scratch ----------------------------------------------------
// One buffer per device, held from module load until the process ends.  Host code never uses the
// symbol itself (on the host it only names the device variable): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and every launch gets it.
static __device__ __align__(256) uint8_t scratch[Q4GSW_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (null when it cannot be had).
void* scratch_of_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) p = nullptr;
        g_scratch_ptr[dev] = p;
    });
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

q4gsw_status q4gsw_packed_bytes(int64_t N, int64_t K, int64_t group_size, int32_t scale_dtype, uint64_t* bytes) {
    if (!bytes) return Q4GSW_E_NULL;
    if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return Q4GSW_E_SHAPE;
    if (group_size < 1 || K % group_size != 0) return Q4GSW_E_GROUP;
    if (!scale_dtype_ok(scale_dtype)) return Q4GSW_E_DTYPE;
    *bytes = make_layout(N, K, group_size, esize(scale_dtype)).total;
    return Q4GSW_OK;
}

q4gsw_status q4gsw_pack(const uint8_t* codes, const void* scales, int32_t scale_dtype, int64_t N, int64_t K,
                        int64_t group_size, void* packed, uint64_t packed_bytes, void* stream, q4gsw_weight* out) {
    if (!codes || !scales || !packed || !out) return Q4GSW_E_NULL;
    uint64_t need = 0;
    q4gsw_status st = q4gsw_packed_bytes(N, K, group_size, scale_dtype, &need);
    if (st != Q4GSW_OK) return st;
    if (packed_bytes < need) return Q4GSW_E_BUFFER;
    const Range pr = range_of(packed, need);
    if (overlap(pr, range_of(codes, (uint64_t)N * K)) ||
        overlap(pr, range_of(scales, (uint64_t)(K / group_size) * N * esize(scale_dtype))))
        return Q4GSW_E_ALIAS;
    const Layout L = make_layout(N, K, group_size, esize(scale_dtype));
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_pack(codes, scales, scale_dtype == Q4GSW_F16, N, K, group_size, L,
                               static_cast<uint8_t*>(packed), s);
    uint32_t hdr[2] = {0u, 0u};
    if (e == hipSuccess) e = hipMemcpyAsync(hdr, packed, sizeof(hdr), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return Q4GSW_E_HIP;
    if (hdr[kHdrBadCode]) return Q4GSW_E_CODE_RANGE;
    q4gsw_weight w;
    std::memset(&w, 0, sizeof(w));
    w.magic = Q4GSW_MAGIC;
    w.version = Q4GSW_LAYOUT_VERSION;
    w.N = N;
    w.K = K;
    w.group_size = group_size;
    w.n_pad = L.n_pad;
    w.k_pad = L.k_pad;
    w.g_pad = L.g_pad;
    w.scale_dtype = scale_dtype;
    w.flags = (scale_dtype == Q4GSW_F16 && !hdr[kHdrNoFold]) ? Q4GSW_FLAG_FOLD_F16 : 0u;
    w.data = packed;
    w.bytes = L.total;
    w.nibble_offset = L.nibble_offset;
    w.scale_offset = L.scale_offset;
    *out = w;
    return Q4GSW_OK;
}

q4gsw_status q4gsw_unpack(const q4gsw_weight* w, uint8_t* codes, void* scales, void* stream) {
    q4gsw_status st = check_desc(w);
    if (st != Q4GSW_OK) return st;
    if (!codes || !scales) return Q4GSW_E_NULL;
    const Range wr = range_of(w->data, w->bytes);
    const Range cr = range_of(codes, (uint64_t)w->N * w->K);
    const Range sr = range_of(scales, (uint64_t)(w->K / w->group_size) * w->N * esize(w->scale_dtype));
    if (overlap(wr, cr) || overlap(wr, sr) || overlap(cr, sr)) return Q4GSW_E_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_unpack(view_of(w), codes, scales, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return hip_status(e);
}

q4gsw_status q4gsw_workspace_bytes_ex(int32_t op, const q4gsw_weight* w, int64_t M, int32_t act_dtype,
                                      const q4gsw_options* opts, uint64_t* bytes) {
    if (!bytes) return Q4GSW_E_NULL;
    q4gsw_status st = check_desc(w);
    if (st != Q4GSW_OK) return st;
    if (M < 1 || M > kMaxM) return Q4GSW_E_SHAPE;
    if (!act_dtype_ok(act_dtype)) return Q4GSW_E_DTYPE;
    Opts o;
    if ((st = read_opts(opts, &o)) != Q4GSW_OK) return st;
    if (op == Q4GSW_OP_FWD) {
        const int32_t r = pick_fwd(w, M, act_dtype, false, o.route, &st);
        if (st != Q4GSW_OK) return st;
        *bytes = fwd_ws_bytes(w, M, act_dtype, r, o);
        return Q4GSW_OK;
    }
    if (op == Q4GSW_OP_BWD_INPUT) {
        const int32_t r = pick_bwd(w, M, act_dtype, o.route, &st);
        if (st != Q4GSW_OK) return st;
        *bytes = bwd_ws_bytes(w, M, act_dtype, r, o);
        return Q4GSW_OK;
    }
    if (op == Q4GSW_OP_DQ8CA) {
        const WView v = view_of(w);
        if (!dq8ca_supported(v)) return Q4GSW_E_GROUP;
        *bytes = (uint64_t)plan_dq8ca(v, M, o.splits).ws_bytes;
        return Q4GSW_OK;
    }
    return Q4GSW_E_SHAPE;
}

q4gsw_status q4gsw_workspace_bytes(int32_t op, const q4gsw_weight* w, int64_t M, int32_t act_dtype, uint64_t* bytes) {
    return q4gsw_workspace_bytes_ex(op, w, M, act_dtype, nullptr, bytes);
}

q4gsw_status q4gsw_qkv_workspace_bytes_ex(const q4gsw_weight* wq, const q4gsw_weight* wk, const q4gsw_weight* wv,
                                          int64_t M, int32_t x_dtype, const q4gsw_options* opts, uint64_t* bytes) {
    if (!bytes) return Q4GSW_E_NULL;
    q4gsw_status st = check_qkv_descs(wq, wk, wv);
    if (st != Q4GSW_OK) return st;
    if (M < 1 || M > kMaxM) return Q4GSW_E_SHAPE;
    if (!act_dtype_ok(x_dtype)) return Q4GSW_E_DTYPE;
    Opts o;
    if ((st = read_opts(opts, &o)) != Q4GSW_OK) return st;
    const int32_t r = pick_fwd(wq, M, x_dtype, true, o.route, &st);
    if (st != Q4GSW_OK) return st;
    const q4gsw_weight* w3[3] = {wq, wk, wv};
    *bytes = qkv_ws_bytes(w3, M, x_dtype, r, o);
    return Q4GSW_OK;
}

q4gsw_status q4gsw_qkv_workspace_bytes(const q4gsw_weight* wq, const q4gsw_weight* wk, const q4gsw_weight* wv,
                                       int64_t M, int32_t x_dtype, uint64_t* bytes) {
    return q4gsw_qkv_workspace_bytes_ex(wq, wk, wv, M, x_dtype, nullptr, bytes);
}

q4gsw_status q4gsw_linear_fwd_ex(const q4gsw_weight* w, const void* x, int32_t x_dtype, int64_t M, float* y,
                                 void* ws, uint64_t ws_bytes, const q4gsw_options* opts, void* stream) {
    Opts o;
    q4gsw_status st = read_opts(opts, &o);
    if (st != Q4GSW_OK) return st;
    int32_t route = Q4GSW_ROUTE_NONE;
    uint64_t need = 0;
    if ((st = prepare_fwd(w, x, x_dtype, M, y, o, &route, &need)) != Q4GSW_OK) return st;
    if (!ws_ok(ws, ws_bytes, need)) return Q4GSW_E_WORKSPACE;
    if ((st = fwd_alias(w, x, x_dtype, M, y, ws, need)) != Q4GSW_OK) return st;
    return run_fwd(w, x, x_dtype, M, y, ws, route, o, static_cast<hipStream_t>(stream));
}

q4gsw_status q4gsw_linear_fwd(const q4gsw_weight* w, const void* x, int32_t x_dtype, int64_t M, float* y, void* ws,
                              uint64_t ws_bytes, void* stream) {
    return q4gsw_linear_fwd_ex(w, x, x_dtype, M, y, ws, ws_bytes, nullptr, stream);
}

q4gsw_status q4gsw_linear_fwd_noalloc(const q4gsw_weight* w, const void* x, int32_t x_dtype, int64_t M, float* y,
                                      void* stream) {
    const Opts o;
    int32_t route = Q4GSW_ROUTE_NONE;
    uint64_t need = 0;
    q4gsw_status st = prepare_fwd(w, x, x_dtype, M, y, o, &route, &need);
    if (st != Q4GSW_OK) return st;
    if (need > Q4GSW_SCRATCH_BYTES) return Q4GSW_E_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        ws = scratch_of_current_device();
        if (!ws) return Q4GSW_E_HIP;
    }
    if ((st = fwd_alias(w, x, x_dtype, M, y, ws, need)) != Q4GSW_OK) return st;
    return run_fwd(w, x, x_dtype, M, y, ws, route, o, static_cast<hipStream_t>(stream));
}

q4gsw_status q4gsw_linear_bwd_input_ex(const q4gsw_weight* w, const void* d_out, int32_t g_dtype, int64_t M,
                                       float* d_x, void* ws, uint64_t ws_bytes, const q4gsw_options* opts,
                                       void* stream) {
    q4gsw_status st = check_desc(w);
    if (st != Q4GSW_OK) return st;
    if (!d_out || !d_x) return Q4GSW_E_NULL;
    if (M < 1 || M > kMaxM) return Q4GSW_E_SHAPE;
    if (!act_dtype_ok(g_dtype)) return Q4GSW_E_DTYPE;
    Opts o;
    if ((st = read_opts(opts, &o)) != Q4GSW_OK) return st;
    const int32_t route = pick_bwd(w, M, g_dtype, o.route, &st);
    if (st != Q4GSW_OK) return st;
    const uint64_t need = bwd_ws_bytes(w, M, g_dtype, route, o);
    if (!ws_ok(ws, ws_bytes, need)) return Q4GSW_E_WORKSPACE;
    const Range xr = range_of(d_x, (uint64_t)M * w->K * 4);
    const Range gr = range_of(d_out, (uint64_t)M * w->N * esize(g_dtype));
    if (overlap(xr, gr) || overlap(xr, range_of(w->data, w->bytes)) ||
        (need > 0 && (overlap(xr, range_of(ws, need)) || overlap(range_of(ws, need), gr) ||
                      overlap(range_of(ws, need), range_of(w->data, w->bytes)))))
        return Q4GSW_E_ALIAS;
    return run_bwd(w, d_out, g_dtype, M, d_x, ws, route, o, static_cast<hipStream_t>(stream));
}

q4gsw_status q4gsw_linear_bwd_input(const q4gsw_weight* w, const void* d_out, int32_t g_dtype, int64_t M, float* d_x,
                                    void* ws, uint64_t ws_bytes, void* stream) {
    return q4gsw_linear_bwd_input_ex(w, d_out, g_dtype, M, d_x, ws, ws_bytes, nullptr, stream);
}

q4gsw_status q4gsw_dq8ca_quantize(const void* x, int32_t x_dtype, int64_t M, int64_t K, int8_t* q, float* scale,
                                  int32_t* zero_point, void* stream) {
    if (!x || !q || !scale || !zero_point) return Q4GSW_E_NULL;
    if (M < 1 || M > kMaxM || K < 1 || K > kMaxDim) return Q4GSW_E_SHAPE;
    if (!act_dtype_ok(x_dtype)) return Q4GSW_E_DTYPE;
    const Range xr = range_of(x, (uint64_t)M * K * esize(x_dtype));
    const Range qr = range_of(q, (uint64_t)M * K);
    const Range sr = range_of(scale, (uint64_t)M * 4);
    const Range zr = range_of(zero_point, (uint64_t)M * 4);
    if (overlap(qr, xr) || overlap(sr, xr) || overlap(zr, xr) || overlap(qr, sr) || overlap(qr, zr) || overlap(sr, zr))
        return Q4GSW_E_ALIAS;
    return hip_status(launch_dq8ca_quantize(x, x_dtype, M, K, q, scale, zero_point, static_cast<hipStream_t>(stream)));
}

q4gsw_status q4gsw_linear_dq8ca_ex(const q4gsw_weight* w, const void* x, int32_t x_dtype, int64_t M, float* y,
                                   void* ws, uint64_t ws_bytes, const q4gsw_options* opts, void* stream) {
    q4gsw_status st = check_desc(w);
    if (st != Q4GSW_OK) return st;
    if (!x || !y) return Q4GSW_E_NULL;
    if (M < 1 || M > kMaxM) return Q4GSW_E_SHAPE;
    if (!act_dtype_ok(x_dtype)) return Q4GSW_E_DTYPE;
    Opts o;
    if ((st = read_opts(opts, &o)) != Q4GSW_OK) return st;
    const WView v = view_of(w);
    if (!dq8ca_supported(v)) return Q4GSW_E_GROUP;
    const Dq8caPlan plan = plan_dq8ca(v, M, o.splits);
    const uint64_t need = (uint64_t)plan.ws_bytes;
    if (!ws_ok(ws, ws_bytes, need)) return Q4GSW_E_WORKSPACE;
    if ((st = fwd_alias(w, x, x_dtype, M, y, ws, need)) != Q4GSW_OK) return st;
    return hip_status(launch_dq8ca(v, x, x_dtype, M, y, plan, ws, static_cast<hipStream_t>(stream)));
}

q4gsw_status q4gsw_linear_dq8ca(const q4gsw_weight* w, const void* x, int32_t x_dtype, int64_t M, float* y, void* ws,
                                uint64_t ws_bytes, void* stream) {
    return q4gsw_linear_dq8ca_ex(w, x, x_dtype, M, y, ws, ws_bytes, nullptr, stream);
}

q4gsw_status q4gsw_qkv_fused_ex(const q4gsw_weight* wq, const q4gsw_weight* wk, const q4gsw_weight* wv, const void* x,
                                int32_t x_dtype, int64_t M, float* q, float* k, float* v, void* ws, uint64_t ws_bytes,
                                const q4gsw_options* opts, void* stream) {
    q4gsw_status st = check_qkv_descs(wq, wk, wv);
    if (st != Q4GSW_OK) return st;
    if (!x || !q || !k || !v) return Q4GSW_E_NULL;
    if (M < 1 || M > kMaxM) return Q4GSW_E_SHAPE;
    if (!act_dtype_ok(x_dtype)) return Q4GSW_E_DTYPE;
    Opts o;
    if ((st = read_opts(opts, &o)) != Q4GSW_OK) return st;
    const int32_t route = pick_fwd(wq, M, x_dtype, true, o.route, &st);
    if (st != Q4GSW_OK) return st;
    const q4gsw_weight* w3[3] = {wq, wk, wv};
    float* o3[3] = {q, k, v};
    const uint64_t need = qkv_ws_bytes(w3, M, x_dtype, route, o);
    if (!ws_ok(ws, ws_bytes, need)) return Q4GSW_E_WORKSPACE;
    Range outs[3];
    for (int i = 0; i < 3; ++i) outs[i] = range_of(o3[i], (uint64_t)M * w3[i]->N * 4);
    const Range xr = range_of(x, (uint64_t)M * wq->K * esize(x_dtype));
    for (int i = 0; i < 3; ++i) {
        if (overlap(outs[i], xr)) return Q4GSW_E_ALIAS;
        for (int j = 0; j < 3; ++j) {
            if (j > i && overlap(outs[i], outs[j])) return Q4GSW_E_ALIAS;
            if (overlap(outs[i], range_of(w3[j]->data, w3[j]->bytes))) return Q4GSW_E_ALIAS;
        }
        if (need > 0 && overlap(outs[i], range_of(ws, need))) return Q4GSW_E_ALIAS;
    }
    if (need > 0) {
        if (overlap(range_of(ws, need), xr)) return Q4GSW_E_ALIAS;
        for (int j = 0; j < 3; ++j)
            if (overlap(range_of(ws, need), range_of(w3[j]->data, w3[j]->bytes))) return Q4GSW_E_ALIAS;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (route == Q4GSW_ROUTE_QKV_FUSED) {
        FwdSeg segs[3];
        for (int i = 0; i < 3; ++i) segs[i] = FwdSeg{view_of(w3[i]), o3[i]};
        const FwdPlan plan = plan_gemm_fwd(segs, 3, x_dtype, fold_ok(wq), M, o.rows, o.splits);
        return hip_status(launch_gemm_fwd(segs, 3, x, x_dtype, M, plan, static_cast<float*>(ws), s));
    }
    // Decode shapes (M <= 8): the three streaming GEMVs in one launch when none of them splits K,
    // each weight with the per-row work of its own call, so the outputs equal three separate
    // forwards bit for bit.
    if (route == Q4GSW_ROUTE_GEMV) {
        const WView v3[3] = {view_of(wq), view_of(wk), view_of(wv)};
        if (gemv_fwd_splits(v3[0], M) == 1 && gemv_fwd_splits(v3[1], M) == 1 && gemv_fwd_splits(v3[2], M) == 1)
            return hip_status(launch_gemv_fwd_multi(v3, o3, 3, x, x_dtype, M, s));
    }
    // Fallback outside the fused predicate: three forwards on the same stream (same contract).
    for (int i = 0; i < 3; ++i) {
        st = run_fwd(w3[i], x, x_dtype, M, o3[i], ws, route, o, s);
        if (st != Q4GSW_OK) return st;
    }
    return Q4GSW_OK;
}

q4gsw_status q4gsw_qkv_fused(const q4gsw_weight* wq, const q4gsw_weight* wk, const q4gsw_weight* wv, const void* x,
                             int32_t x_dtype, int64_t M, float* q, float* k, float* v, void* ws, uint64_t ws_bytes,
                             void* stream) {
    return q4gsw_qkv_fused_ex(wq, wk, wv, x, x_dtype, M, q, k, v, ws, ws_bytes, nullptr, stream);
}

// ---- the adapter step around the frozen base ----------------------------------------------------
static bool finite_f(double v) { return v == v && v - v == 0.0; }

q4gsw_status q4gsw_adapter_workspace_bytes(int32_t op, const q4gsw_weight* w, int64_t M, int32_t act_dtype,
                                           int32_t rank, uint64_t* bytes) {
    if (!bytes) return Q4GSW_E_NULL;
    *bytes = 0;
    q4gsw_status st = check_desc(w);
    if (st != Q4GSW_OK) return st;
    if (M < 1 || M > kMaxM || rank < 1 || rank > adapter_rank_max() || !adapter_shape_ok(M, w->N, w->K, rank))
        return Q4GSW_E_SHAPE;
    if (!act_dtype_ok(act_dtype)) return Q4GSW_E_DTYPE;
    const Opts o;
    if (op == Q4GSW_OP_FWD) {
        const int32_t route = pick_fwd(w, M, act_dtype, false, o.route, &st);
        if (st != Q4GSW_OK) return st;
        *bytes = round_up((int64_t)fwd_ws_bytes(w, M, act_dtype, route, o), 256) +
                 adapter_fwd_terms_ws_bytes(M, w->N, w->K, rank);
        return Q4GSW_OK;
    }
    if (op == Q4GSW_OP_BWD_INPUT) {
        const int32_t route = pick_bwd(w, M, act_dtype, o.route, &st);
        if (st != Q4GSW_OK) return st;
        *bytes = round_up((int64_t)bwd_ws_bytes(w, M, act_dtype, route, o), 256) +
                 adapter_bwd_terms_ws_bytes(M, w->N, w->K, rank);
        return Q4GSW_OK;
    }
    return Q4GSW_E_SHAPE;
}

q4gsw_status q4gsw_adapter_fwd(const q4gsw_weight* w, const void* x, int32_t x_dtype, int64_t M, const float* A,
                               const float* B, int32_t rank, float alpha, float* y, float* t, void* ws,
                               uint64_t ws_bytes, void* stream) {
    const Opts o;
    int32_t route = Q4GSW_ROUTE_NONE;
    uint64_t base = 0;
    q4gsw_status st = prepare_fwd(w, x, x_dtype, M, y, o, &route, &base);
    if (st != Q4GSW_OK) return st;
    if (!A || !B || !t) return Q4GSW_E_NULL;
    if (rank < 1 || rank > adapter_rank_max() || !adapter_shape_ok(M, w->N, w->K, rank)) return Q4GSW_E_SHAPE;
    if (!finite_f(alpha)) return Q4GSW_E_SHAPE;
    // the forward's workspace, then the column-chunk sums of t
    base = round_up((int64_t)base, 256);
    const uint64_t need = base + adapter_fwd_terms_ws_bytes(M, w->N, w->K, rank);
    if (!ws_ok(ws, ws_bytes, need)) return Q4GSW_E_WORKSPACE;
    if ((st = fwd_alias(w, x, x_dtype, M, y, ws, need)) != Q4GSW_OK) return st;
    // the outputs y and t against every input and each other; the workspace against t and the factors
    const Range yr = range_of(y, (uint64_t)M * w->N * 4), tr = range_of(t, (uint64_t)M * rank * 4);
    const Range ar = range_of(A, (uint64_t)rank * w->K * 4), br = range_of(B, (uint64_t)w->N * rank * 4);
    const Range xr = range_of(x, (uint64_t)M * w->K * esize(x_dtype)), wr = range_of(w->data, w->bytes);
    const Range sr = range_of(ws, need);
    if (overlap(yr, ar) || overlap(yr, br) || overlap(yr, tr) || overlap(tr, xr) || overlap(tr, ar) ||
        overlap(tr, br) || overlap(tr, wr) || overlap(sr, tr) || overlap(sr, ar) || overlap(sr, br))
        return Q4GSW_E_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* tws = static_cast<uint8_t*>(ws) + base;
    if ((st = hip_status(launch_adapter_fwd_t(x, x_dtype, M, w->K, A, rank, tws, s))) != Q4GSW_OK) return st;
    const LowRankEpi epi = adapter_fwd_epi(M, w->K, B, rank, alpha, t, tws);
    bool done = false;
    if ((st = run_fwd(w, x, x_dtype, M, y, ws, route, o, s, &epi, &done)) != Q4GSW_OK) return st;
    if (done) return Q4GSW_OK;
    return hip_status(launch_adapter_fwd_expand(y, M, w->N, w->K, B, rank, alpha, t, tws, s));
}

q4gsw_status q4gsw_adapter_bwd(const q4gsw_weight* w, const void* x, const void* d_out, int32_t dtype, int64_t M,
                               const float* A, const float* B, int32_t rank, float alpha, const float* t, float* d_x,
                               float* d_A, float* d_B, void* ws, uint64_t ws_bytes, void* stream) {
    q4gsw_status st = check_desc(w);
    if (st != Q4GSW_OK) return st;
    if (!x || !d_out || !A || !B || !t || !d_x || !d_A || !d_B) return Q4GSW_E_NULL;
    if (M < 1 || M > kMaxM || rank < 1 || rank > adapter_rank_max() || !finite_f(alpha) ||
        !adapter_shape_ok(M, w->N, w->K, rank))
        return Q4GSW_E_SHAPE;
    if (!act_dtype_ok(dtype)) return Q4GSW_E_DTYPE;
    const Opts o;
    const int32_t route = pick_bwd(w, M, dtype, o.route, &st);
    if (st != Q4GSW_OK) return st;
    const uint64_t base = round_up((int64_t)bwd_ws_bytes(w, M, dtype, route, o), 256);
    const uint64_t need = base + adapter_bwd_terms_ws_bytes(M, w->N, w->K, rank);
    if (!ws_ok(ws, ws_bytes, need)) return Q4GSW_E_WORKSPACE;
    const int64_t N = w->N, K = w->K;
    const Range outs[3] = {range_of(d_x, (uint64_t)M * K * 4), range_of(d_A, (uint64_t)rank * K * 4),
                           range_of(d_B, (uint64_t)N * rank * 4)};
    const Range ins[6] = {range_of(x, (uint64_t)M * K * esize(dtype)), range_of(d_out, (uint64_t)M * N * esize(dtype)),
                          range_of(A, (uint64_t)rank * K * 4), range_of(B, (uint64_t)N * rank * 4),
                          range_of(t, (uint64_t)M * rank * 4), range_of(w->data, w->bytes)};
    const Range sr = range_of(ws, need);
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlap(outs[i], ins[j])) return Q4GSW_E_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return Q4GSW_E_ALIAS;
        if (overlap(outs[i], sr)) return Q4GSW_E_ALIAS;
    }
    for (int j = 0; j < 6; ++j)
        if (overlap(sr, ins[j])) return Q4GSW_E_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the chunk sums of u first, so that the input gradient's split reduction can add alpha u A
    void* terms = static_cast<uint8_t*>(ws) + base;
    if ((st = hip_status(launch_adapter_bwd_u(d_out, dtype, M, N, K, B, rank, terms, s))) != Q4GSW_OK) return st;
    const LowRankEpi epi = adapter_bwd_epi(M, N, K, A, rank, alpha, terms);
    bool dx_done = false;
    if ((st = run_bwd(w, d_out, dtype, M, d_x, ws, route, o, s, &epi, &dx_done)) != Q4GSW_OK) return st;
    return hip_status(launch_adapter_bwd_rest(x, d_out, dtype, M, N, K, A, rank, alpha, t, d_x, dx_done, d_A, d_B,
                                              terms, s));
}

q4gsw_status q4gsw_adamw_step(float* param, const float* grad, float* exp_avg, float* exp_avg_sq, int64_t n,
                              const q4gsw_adamw_params* hp, int64_t step, void* stream) {
    if (!hp) return Q4GSW_E_NULL;
    if (n < 0 || step < 1) return Q4GSW_E_SHAPE;
    if (!(finite_f(hp->lr) && hp->lr >= 0 && finite_f(hp->weight_decay) && hp->weight_decay >= 0 &&
          hp->beta1 >= 0 && hp->beta1 < 1 && hp->beta2 >= 0 && hp->beta2 < 1 && finite_f(hp->eps) && hp->eps > 0))
        return Q4GSW_E_SHAPE;
    if (n == 0) return Q4GSW_OK;
    if (!param || !grad || !exp_avg || !exp_avg_sq) return Q4GSW_E_NULL;
    const uint64_t b = (uint64_t)n * 4;
    const Range r[4] = {range_of(param, b), range_of(grad, b), range_of(exp_avg, b), range_of(exp_avg_sq, b)};
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (overlap(r[i], r[j])) return Q4GSW_E_ALIAS;
    return hip_status(launch_adamw(param, grad, exp_avg, exp_avg_sq, n, hp->lr, hp->beta1, hp->beta2, hp->eps,
                                   hp->weight_decay, step, static_cast<hipStream_t>(stream)));
}

int32_t q4gsw_route(int32_t op, const q4gsw_weight* w, int64_t M, int32_t act_dtype) {
    if (check_desc(w) != Q4GSW_OK || M < 1 || M > kMaxM || !act_dtype_ok(act_dtype)) return Q4GSW_ROUTE_NONE;
    q4gsw_status st;
    int32_t r = Q4GSW_ROUTE_NONE;
    if (op == Q4GSW_OP_FWD) r = pick_fwd(w, M, act_dtype, false, Q4GSW_ROUTE_NONE, &st);
    else if (op == Q4GSW_OP_BWD_INPUT) r = pick_bwd(w, M, act_dtype, Q4GSW_ROUTE_NONE, &st);
    else if (op == Q4GSW_OP_QKV) r = pick_fwd(w, M, act_dtype, true, Q4GSW_ROUTE_NONE, &st);
    else if (op == Q4GSW_OP_DQ8CA) return dq8ca_supported(view_of(w)) ? Q4GSW_ROUTE_DQ8CA : Q4GSW_ROUTE_NONE;
    else return Q4GSW_ROUTE_NONE;
    return st == Q4GSW_OK ? r : Q4GSW_ROUTE_NONE;
}

q4gsw_status q4gsw_embedding(const q4gsw_weight* w, const int64_t* ids, int64_t T, float* out, void* stream) {
    q4gsw_status st = check_desc(w);
    if (st != Q4GSW_OK) return st;
    if (!ids || !out) return Q4GSW_E_NULL;
    if (T < 1 || T > kMaxM || embedding_blocks(T, w->K) > 0x7FFFFFFFull) return Q4GSW_E_SHAPE;
    const Range orng = range_of(out, (uint64_t)T * w->K * 4);
    if (overlap(orng, range_of(ids, (uint64_t)T * 8)) || overlap(orng, range_of(w->data, w->bytes)))
        return Q4GSW_E_ALIAS;
    return hip_status(launch_embedding(view_of(w), ids, T, out, static_cast<hipStream_t>(stream)));
}

q4gsw_status q4gsw_plan(int32_t op, const q4gsw_weight* w, const q4gsw_weight* wk, const q4gsw_weight* wv,
                        int64_t M, int32_t act_dtype, const q4gsw_options* opts, q4gsw_plan_info* info) {
    if (!info) return Q4GSW_E_NULL;
    *info = q4gsw_plan_info{Q4GSW_ROUTE_NONE, 0, 1};
    q4gsw_status st = op == Q4GSW_OP_QKV ? check_qkv_descs(w, wk, wv) : check_desc(w);
    if (st != Q4GSW_OK) return st;
    Opts o;
    if ((st = read_opts(opts, &o)) != Q4GSW_OK) return st;
    if (M < 1 || M > kMaxM || !act_dtype_ok(act_dtype)) return Q4GSW_OK;
    int32_t r = Q4GSW_ROUTE_NONE;
    q4gsw_status rs = Q4GSW_OK;
    if (op == Q4GSW_OP_FWD) r = pick_fwd(w, M, act_dtype, false, o.route, &rs);
    else if (op == Q4GSW_OP_BWD_INPUT) r = pick_bwd(w, M, act_dtype, o.route, &rs);
    else if (op == Q4GSW_OP_QKV) r = pick_fwd(w, M, act_dtype, true, o.route, &rs);
    else if (op == Q4GSW_OP_DQ8CA) r = dq8ca_supported(view_of(w)) ? Q4GSW_ROUTE_DQ8CA : Q4GSW_ROUTE_NONE;
    if (rs != Q4GSW_OK) r = Q4GSW_ROUTE_NONE;
    info->route = r;
    if (r == Q4GSW_ROUTE_NONE) return Q4GSW_OK;
    const WView v = view_of(w);
    if (r == Q4GSW_ROUTE_GEMV) {
        info->splits = gemv_fwd_splits(v, M);
    } else if (r == Q4GSW_ROUTE_BWD_GEMV) {
        info->splits = gemv_bwd_splits(v, M);
    } else if (r == Q4GSW_ROUTE_DQ8CA) {
        info->tile_rows = 128;
        info->splits = plan_dq8ca(v, M, o.splits).splits;
    } else if (r == Q4GSW_ROUTE_BWD_FOLD || r == Q4GSW_ROUTE_BWD_SPLIT || r == Q4GSW_ROUTE_BWD_BSPLIT) {
        info->tile_rows = 128;
        info->splits = plan_gemm_bwd(v, act_dtype, fold_ok(w), M, o.splits).splits;
    } else if (r == Q4GSW_ROUTE_GEMM_FOLD || r == Q4GSW_ROUTE_GEMM_GROUP || r == Q4GSW_ROUTE_GEMM_SPLIT ||
               r == Q4GSW_ROUTE_QKV_FUSED) {
        FwdSeg segs[3] = {FwdSeg{v, nullptr}, FwdSeg{}, FwdSeg{}};
        int nseg = 1;
        if (r == Q4GSW_ROUTE_QKV_FUSED) {
            segs[1] = FwdSeg{view_of(wk), nullptr};
            segs[2] = FwdSeg{view_of(wv), nullptr};
            nseg = 3;
        }
        const FwdPlan p = plan_gemm_fwd(segs, nseg, act_dtype, fold_ok(w), M, o.rows, o.splits);
        info->tile_rows = 32 * p.mi;
        info->splits = p.splits;
    }
    return Q4GSW_OK;
}

const char* q4gsw_route_name(int32_t route) {
    switch (route) {
        case Q4GSW_ROUTE_NONE: return "none";
        case Q4GSW_ROUTE_GENERIC: return "generic";
        case Q4GSW_ROUTE_GEMV: return "gemv";
        case Q4GSW_ROUTE_GEMM_FOLD: return "gemm_fold";
        case Q4GSW_ROUTE_GEMM_GROUP: return "gemm_group";
        case Q4GSW_ROUTE_GEMM_SPLIT: return "gemm_split";
        case Q4GSW_ROUTE_BWD_GEMV: return "bwd_gemv";
        case Q4GSW_ROUTE_BWD_FOLD: return "bwd_fold";
        case Q4GSW_ROUTE_BWD_SPLIT: return "bwd_split";
        case Q4GSW_ROUTE_QKV_FUSED: return "qkv_fused";
        case Q4GSW_ROUTE_BWD_BSPLIT: return "bwd_bsplit";
        case Q4GSW_ROUTE_DQ8CA: return "dq8ca";
        default: return "unknown";
    }
}

const char* q4gsw_status_str(int32_t status) {
    switch (status) {
        case Q4GSW_OK: return "ok";
        case Q4GSW_E_NULL: return "null pointer";
        case Q4GSW_E_SHAPE: return "size out of range";
        case Q4GSW_E_DTYPE: return "unsupported dtype";
        case Q4GSW_E_GROUP: return "group_size must be >= 1 and divide K";
        case Q4GSW_E_ALIAS: return "output overlaps another buffer";
        case Q4GSW_E_CODE_RANGE: return "code above 15";
        case Q4GSW_E_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
        case Q4GSW_E_DESC: return "invalid or mismatched weight descriptor";
        case Q4GSW_E_HIP: return "HIP runtime error";
        case Q4GSW_E_BUFFER: return "packed buffer too small";
        case Q4GSW_E_ROUTE: return "requested route cannot serve this call";
        case Q4GSW_E_SCRATCH: return "call needs more than the allocation-free entry point's 32 MiB scratch";
        default: return "unknown status";
    }
}

uint32_t q4gsw_layout_version(void) { return Q4GSW_LAYOUT_VERSION; }

const char* q4gsw_build_info(void) { return "q4gsw gfx950 layout-v2 built " __DATE__ " " __TIME__; }

}  // extern "C"
