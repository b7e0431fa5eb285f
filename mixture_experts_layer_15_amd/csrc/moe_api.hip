// moe_api.hip -- the C ABI (include/moe.h): argument validation, workspace
// carving and launch sequencing.  Host code only; every entry point checks
// its arguments before enqueuing anything and never synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <mutex>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

moe_status hip_fail(hipError_t e, const char* where) {
    return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// Exact ceil(cap_num * k * T / (cap_den * E)), saturating; T when cap_den == 0.
int64_t capacity_raw(const moe_config* c) {
    if (c->cap_den == 0) return c->T;
    const __int128 num = (__int128)c->cap_num * c->k * c->T;
    const __int128 den = (__int128)c->cap_den * c->E;
    const __int128 q = (num + den - 1) / den;
    return q > (__int128)INT64_MAX ? INT64_MAX : (int64_t)q;
}

// Capacity as the kernels use it: a limit of T or more never drops anything.
int64_t capacity_eff(const moe_config* c) {
    const int64_t C = capacity_raw(c);
    return C < c->T ? C : c->T;
}

int64_t max_rows(const moe_config* c) {
    const int64_t ce = capacity_eff(c) * c->E;
    if (c->layout == MOE_LAYOUT_PADDED) return ce;
    const int64_t tk = c->T * c->k;
    return tk < ce ? tk : ce;
}

// Entries of token_of_row: every assignment slot and every row.
int64_t tor_len(const moe_config* c) {
    const int64_t tk = c->T * c->k, r = max_rows(c);
    return tk > r ? tk : r;
}

size_t esize(const moe_config* c) { return c->dtype == MOE_BF16 ? 2 : 4; }

// Dynamic expert count per token (route_threshold > 0).
bool dyn_route(const moe_config* c) { return c->route_threshold > 0.f; }

moe::TopkParams topk_params(const moe_config* c) {
    moe::TopkParams tp;
    tp.k = c->k;
    tp.tau = c->temperature;
    tp.renorm = c->renormalize;
    tp.k_min = dyn_route(c) ? c->k_min : c->k;
    tp.theta = dyn_route(c) ? c->route_threshold : 0.f;
    return tp;
}

// The dispatch's plan; with a dynamic expert count the kernels take the
// capacity from the realised assignments, capacity_eff() is its upper bound.
moe::DispatchPlan dispatch_plan(const moe_config* c) {
    return moe::plan_dispatch(c->T, c->E, c->k, capacity_eff(c), c->drop_policy, c->layout,
                              dyn_route(c), c->cap_num, c->cap_den);
}

moe_status check_cfg(const moe_config* c) {
    if (c == nullptr) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
    if (c->T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %lld < 0", (long long)c->T);
    if (c->E < 1 || c->E > 256) return fail(MOE_ERR_INVALID_ARG, "E = %d outside [1, 256]", c->E);
    if (c->k < 1 || c->k > c->E || c->k > 8)
        return fail(MOE_ERR_INVALID_ARG, "k = %d outside [1, min(E, 8)]", c->k);
    if (c->d < 64 || c->d > 16384 || c->d % 64 != 0)
        return fail(MOE_ERR_INVALID_ARG, "d = %d: need a multiple of 64 in [64, 16384]", c->d);
    if (c->d_ff < 64 || c->d_ff > 65536 || c->d_ff % 64 != 0)
        return fail(MOE_ERR_INVALID_ARG, "d_ff = %d: need a multiple of 64 in [64, 65536]", c->d_ff);
    if (c->T > 0 && c->T * (int64_t)c->k >= (int64_t)1 << 31)
        return fail(MOE_ERR_INVALID_ARG, "T * k = %lld must be < 2^31", (long long)(c->T * c->k));
    if (!(c->temperature > 0.f) || !std::isfinite(c->temperature))
        return fail(MOE_ERR_INVALID_ARG, "temperature must be finite and > 0");
    if (c->cap_den < 0 || (c->cap_den > 0 && c->cap_num < 0))
        return fail(MOE_ERR_INVALID_ARG, "capacity factor %d/%d invalid", c->cap_num, c->cap_den);
    if (c->renormalize != 0 && c->renormalize != 1)
        return fail(MOE_ERR_INVALID_ARG, "renormalize must be 0 or 1");
    if (c->dtype != MOE_F32 && c->dtype != MOE_BF16)
        return fail(MOE_ERR_UNSUPPORTED, "dtype %d not supported", c->dtype);
    if (c->drop_policy != MOE_DROP_TOKEN_ORDER && c->drop_policy != MOE_DROP_CHOICE_ORDER)
        return fail(MOE_ERR_INVALID_ARG, "drop_policy %d is not a moe_drop_policy", c->drop_policy);
    if (c->layout != MOE_LAYOUT_COMPACT && c->layout != MOE_LAYOUT_PADDED)
        return fail(MOE_ERR_INVALID_ARG, "layout %d is not a moe_layout", c->layout);
    if (c->route_threshold != 0.f) {
        if (!(c->route_threshold > 0.f) || !(c->route_threshold <= 1.f))
            return fail(MOE_ERR_INVALID_ARG, "route_threshold must be 0 (fixed k) or in (0, 1]");
        if (c->k_min < 1 || c->k_min > c->k)
            return fail(MOE_ERR_INVALID_ARG, "k_min = %d outside [1, k = %d]", c->k_min, c->k);
        if (c->layout == MOE_LAYOUT_PADDED)
            return fail(MOE_ERR_UNSUPPORTED,
                        "the padded layout needs a fixed capacity: no dynamic expert count");
    } else if (c->k_min != 0) {
        return fail(MOE_ERR_INVALID_ARG, "k_min must be 0 when route_threshold is 0");
    }
    if (c->layout == MOE_LAYOUT_PADDED) {
        if (c->cap_den == 0)
            return fail(MOE_ERR_INVALID_ARG, "the padded layout needs a capacity limit (cap_den > 0)");
        if (capacity_eff(c) * (int64_t)c->E >= ((int64_t)1 << 31))
            return fail(MOE_ERR_INVALID_ARG, "padded layout: E * C = %lld must be < 2^31",
                        (long long)(capacity_eff(c) * (int64_t)c->E));
    }
    return MOE_OK;
}

// A NULL pointer is accepted only for an optional argument or an empty buffer.
moe_status check_ptr(const void* p, const char* name, size_t bytes, bool optional = false) {
    if (p == nullptr) {
        if (optional || bytes == 0) return MOE_OK;
        return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);
    }
    if (((uintptr_t)p & 15u) != 0)
        return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return MOE_OK;
}

// Element counts of a config, as size_t, for pointer checks.
#define SIZES(c)                                                              \
    const size_t T = (size_t)(c)->T, d = (size_t)(c)->d, E = (size_t)(c)->E;  \
    const size_t k = (size_t)(c)->k, F = (size_t)(c)->d_ff, es = esize(c);    \
    const size_t R = (size_t)max_rows(c);                                     \
    (void)T; (void)d; (void)E; (void)k; (void)F; (void)es; (void)R

#define CHECK(expr)                          \
    do {                                     \
        moe_status _s = (expr);              \
        if (_s != MOE_OK) return _s;         \
    } while (0)

// Persistent-grid cap of the grouped GEMMs: twice the CU count.  The fp32
// GEMMs (256-thread workgroups, two resident per CU) launch up to this many;
// the bf16 MFMA GEMMs, whose LDS stages hold one workgroup per CU, launch
// half (one per CU).
int gemm_grid_cap() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    v = 2 * cus;
    v = (v + 7) / 8 * 8;
    cached[dev].store(v, std::memory_order_relaxed);
    return v;
}

struct FwdLayout {
    size_t logits, idx, gate, count, offset, row_of, token_of_row, dsp, x_perm, h, y_perm, part,
        total;
};

// The fused forward's output path for bf16 top-1 layers that keep every token
// (capacity >= T, compact layout): each row is its token's only assignment,
// so the down GEMM's result goes straight to y, bit-identical to writing
// y_perm and combining -- unless the down GEMM runs in two K slices
// (down_split_applies: small experts too few to fill the CUs), whose fp32
// partials a second kernel sums, rounds and gates (the summation order then
// differs from the staged calls' by the split).
bool fwd_direct(const moe_config* c) {
    return c->dtype == MOE_BF16 && c->k == 1 && c->layout == MOE_LAYOUT_COMPACT &&
           capacity_eff(c) >= c->T && !dyn_route(c);
}
bool fwd_down_split(const moe_config* c) {
    return fwd_direct(c) &&
           moe::down_split_applies(max_rows(c), c->E, c->d, c->d_ff, gemm_grid_cap() / 2);
}

// The fused forward's input path for bf16 compact layers: the gate/up GEMM
// gathers its rows of x through token_of_row, so x_perm is never formed (the
// GEMM's 32-bit byte offsets must span x).
bool fwd_gather(const moe_config* c) {
    return c->dtype == MOE_BF16 && c->layout == MOE_LAYOUT_COMPACT &&
           (size_t)c->T * (size_t)c->d * esize(c) < ((size_t)1 << 32);
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

FwdLayout fwd_layout(const moe_config* c) {
    const size_t T = (size_t)c->T, E = (size_t)c->E, k = (size_t)c->k;
    const size_t R = (size_t)max_rows(c);
    const moe::DispatchPlan p = dispatch_plan(c);
    FwdLayout L;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
    L.logits = take(T * E * 4);
    L.idx = take(T * k * 4);
    L.gate = take(T * k * 4);
    L.count = take(E * 4);
    L.offset = take((E + 1) * 4);
    L.row_of = take(T * k * 4);
    L.token_of_row = take((size_t)tor_len(c) * 4);
    L.dsp = take(moe::dispatch_workspace_bytes(p));
    // x_perm only when the gate/up GEMM does not gather x itself, y_perm only
    // when the down GEMM does not write y itself
    L.x_perm = take(fwd_gather(c) ? 0 : R * (size_t)c->d * esize(c));
    L.h = take(R * (size_t)c->d_ff * esize(c));
    L.y_perm = take(fwd_direct(c) ? 0 : R * (size_t)c->d * esize(c));
    L.part = take(fwd_down_split(c) ? 2 * R * (size_t)c->d * 4 : 0);   // fp32 K-slice partials
    L.total = o;
    return L;
}

}  // namespace

extern "C" {

int64_t moe_capacity(const moe_config* cfg) {
    if (check_cfg(cfg) != MOE_OK) return -1;
    return capacity_raw(cfg);
}

int64_t moe_max_rows(const moe_config* cfg) {
    if (check_cfg(cfg) != MOE_OK) return -1;
    return max_rows(cfg);
}

moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes) {
    CHECK(check_cfg(cfg));
    if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = fwd_layout(cfg).total;
    return MOE_OK;
}

moe_status moe_dispatch_workspace_size(const moe_config* cfg, size_t* bytes) {
    CHECK(check_cfg(cfg));
    if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = moe::dispatch_workspace_bytes(
        dispatch_plan(cfg));
    return MOE_OK;
}

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
    }
    return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* bias, float* logits, int32_t* topk_idx, float* topk_gate,
                     void* stream) {
    CHECK(check_cfg(cfg));
    SIZES(cfg);
    CHECK(check_ptr(x, "x", T * d * es));
    CHECK(check_ptr(w_router, "w_router", d * E * es));
    CHECK(check_ptr(bias, "bias", E * 4, true));
    CHECK(check_ptr(logits, "logits", T * E * 4));
    CHECK(check_ptr(topk_idx, "topk_idx", T * k * 4));
    CHECK(check_ptr(topk_gate, "topk_gate", T * k * 4));
    hipError_t e = moe::launch_route(cfg->dtype, x, w_router, bias, logits, topk_idx, topk_gate,
                                     cfg->T, cfg->d, cfg->E, topk_params(cfg),
                                     (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route");
}

moe_status moe_route_from_logits(const moe_config* cfg, const float* logits, int32_t* topk_idx,
                                 float* topk_gate, void* stream) {
    CHECK(check_cfg(cfg));
    SIZES(cfg);
    CHECK(check_ptr(logits, "logits", T * E * 4));
    CHECK(check_ptr(topk_idx, "topk_idx", T * k * 4));
    CHECK(check_ptr(topk_gate, "topk_gate", T * k * 4));
    hipError_t e = moe::launch_route_from_logits(logits, topk_idx, topk_gate, cfg->T, cfg->E,
                                                 topk_params(cfg), (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route_from_logits");
}

moe_status moe_dispatch(const moe_config* cfg, const int32_t* topk_idx, const void* x,
                        void* x_perm, int32_t* expert_count, int32_t* expert_offset,
                        int32_t* row_of, int32_t* token_of_row, void* workspace, size_t ws_bytes,
                        void* stream) {
    CHECK(check_cfg(cfg));
    SIZES(cfg);
    CHECK(check_ptr(topk_idx, "topk_idx", T * k * 4));
    CHECK(check_ptr(x, "x", T * d * es));
    CHECK(check_ptr(x_perm, "x_perm", R * d * es));
    if (expert_count == nullptr || expert_offset == nullptr)
        return fail(MOE_ERR_INVALID_ARG, "expert_count / expert_offset is NULL");
    CHECK(check_ptr(expert_count, "expert_count", E * 4));
    CHECK(check_ptr(expert_offset, "expert_offset", (E + 1) * 4));
    CHECK(check_ptr(row_of, "row_of", T * k * 4));
    CHECK(check_ptr(token_of_row, "token_of_row", (size_t)tor_len(cfg) * 4));
    const moe::DispatchPlan p = dispatch_plan(cfg);
    const size_t need = moe::dispatch_workspace_bytes(p);
    if (workspace == nullptr || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "dispatch workspace: need %zu bytes, got %zu", need, ws_bytes);
    CHECK(check_ptr(workspace, "workspace", 1));
    hipError_t e = moe::launch_dispatch(p, cfg->dtype, topk_idx, x, x_perm, expert_count,
                                        expert_offset, row_of, token_of_row, workspace, cfg->d,
                                        (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_dispatch");
}

}  // extern "C"

namespace {

// moe_dispatch_noalloc's workspace: a static device buffer, one copy per
// device.  Host code never uses the array's name as an address: its device
// address comes from hipGetSymbolAddress, once per device, with that device
// current, and is kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[MOE_DISPATCH_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

moe_status scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "moe_dispatch_noalloc/hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MOE_ERR_UNSUPPORTED, "device %d beyond the %d the static buffer serves", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                            "moe_dispatch_noalloc/hipGetSymbolAddress");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_dispatch_noalloc(const moe_config* cfg, const int32_t* topk_idx, const void* x,
                                void* x_perm, int32_t* expert_count, int32_t* expert_offset,
                                int32_t* row_of, int32_t* token_of_row, void* stream) {
    CHECK(check_cfg(cfg));
    SIZES(cfg);
    CHECK(check_ptr(topk_idx, "topk_idx", T * k * 4));
    CHECK(check_ptr(x, "x", T * d * es));
    CHECK(check_ptr(x_perm, "x_perm", R * d * es));
    if (expert_count == nullptr || expert_offset == nullptr)
        return fail(MOE_ERR_INVALID_ARG, "expert_count / expert_offset is NULL");
    CHECK(check_ptr(expert_count, "expert_count", E * 4));
    CHECK(check_ptr(expert_offset, "expert_offset", (E + 1) * 4));
    CHECK(check_ptr(row_of, "row_of", T * k * 4));
    CHECK(check_ptr(token_of_row, "token_of_row", (size_t)tor_len(cfg) * 4));
    const moe::DispatchPlan p = dispatch_plan(cfg);
    const size_t need = moe::dispatch_workspace_bytes(p);
    if (need > MOE_DISPATCH_SCRATCH_BYTES)
        return fail(MOE_ERR_INVALID_ARG,
                    "dispatch tables need %zu bytes, more than the %u of the static buffer", need,
                    (unsigned)MOE_DISPATCH_SCRATCH_BYTES);
    void* ws = nullptr;
    CHECK(scratch_for_current_device(&ws));
    hipError_t e = moe::launch_dispatch(p, cfg->dtype, topk_idx, x, x_perm, expert_count,
                                        expert_offset, row_of, token_of_row, ws, cfg->d,
                                        (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_dispatch_noalloc");
}

moe_status moe_expert_ffn(const moe_config* cfg, const void* x_perm, const int32_t* expert_offset,
                          const void* w_gate, const void* w_up, const void* w_down, void* h,
                          void* y_perm, void* stream) {
    CHECK(check_cfg(cfg));
    SIZES(cfg);
    if (expert_offset == nullptr) return fail(MOE_ERR_INVALID_ARG, "expert_offset is NULL");
    CHECK(check_ptr(expert_offset, "expert_offset", (E + 1) * 4));
    CHECK(check_ptr(x_perm, "x_perm", R * d * es));
    CHECK(check_ptr(w_gate, "w_gate", E * d * F * es));
    CHECK(check_ptr(w_up, "w_up", E * d * F * es));
    CHECK(check_ptr(w_down, "w_down", E * d * F * es));
    CHECK(check_ptr(h, "h", R * F * es));
    CHECK(check_ptr(y_perm, "y_perm", R * d * es));
    hipError_t e = moe::launch_expert_ffn(cfg->dtype, x_perm, expert_offset, w_gate, w_up, w_down,
                                          h, y_perm, cfg->E, cfg->d, cfg->d_ff, max_rows(cfg),
                                          gemm_grid_cap(), (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_expert_ffn");
}

moe_status moe_expert_gate_up(const moe_config* cfg, const void* x_perm,
                              const int32_t* expert_offset, const void* w_gate, const void* w_up,
                              void* h, void* stream) {
    CHECK(check_cfg(cfg));
    SIZES(cfg);
    if (expert_offset == nullptr) return fail(MOE_ERR_INVALID_ARG, "expert_offset is NULL");
    CHECK(check_ptr(expert_offset, "expert_offset", (E + 1) * 4));
    CHECK(check_ptr(x_perm, "x_perm", R * d * es));
    CHECK(check_ptr(w_gate, "w_gate", E * d * F * es));
    CHECK(check_ptr(w_up, "w_up", E * d * F * es));
    CHECK(check_ptr(h, "h", R * F * es));
    hipError_t e = moe::launch_gate_up(cfg->dtype, x_perm, expert_offset, w_gate, w_up, h, cfg->E,
                                       cfg->d, cfg->d_ff, max_rows(cfg), gemm_grid_cap(),
                                       (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_expert_gate_up");
}

moe_status moe_expert_down(const moe_config* cfg, const void* h, const int32_t* expert_offset,
                           const void* w_down, void* y_perm, void* stream) {
    CHECK(check_cfg(cfg));
    SIZES(cfg);
    if (expert_offset == nullptr) return fail(MOE_ERR_INVALID_ARG, "expert_offset is NULL");
    CHECK(check_ptr(expert_offset, "expert_offset", (E + 1) * 4));
    CHECK(check_ptr(h, "h", R * F * es));
    CHECK(check_ptr(w_down, "w_down", E * d * F * es));
    CHECK(check_ptr(y_perm, "y_perm", R * d * es));
    hipError_t e = moe::launch_down(cfg->dtype, h, expert_offset, w_down, y_perm, cfg->E, cfg->d,
                                    cfg->d_ff, max_rows(cfg), gemm_grid_cap(), (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_expert_down");
}

moe_status moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* row_of,
                       const float* topk_gate, void* y, void* stream) {
    CHECK(check_cfg(cfg));
    SIZES(cfg);
    CHECK(check_ptr(y_perm, "y_perm", R * d * es));
    CHECK(check_ptr(row_of, "row_of", T * k * 4));
    CHECK(check_ptr(topk_gate, "topk_gate", T * k * 4));
    CHECK(check_ptr(y, "y", T * d * es));
    hipError_t e = moe::launch_combine(cfg->dtype, y_perm, row_of, topk_gate, y, cfg->T, cfg->d,
                                       cfg->k, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_combine");
}

}  // extern "C"

namespace {

moe_status check_mlp(const moe_config* cfg, const moe_mlp_router* rt) {
    CHECK(check_cfg(cfg));
    if (rt == nullptr) return fail(MOE_ERR_INVALID_ARG, "router is NULL");
    if (rt->r < 64 || rt->r > 1024 || rt->r % 64 != 0)
        return fail(MOE_ERR_INVALID_ARG, "router r = %d: need a multiple of 64 in [64, 1024]", rt->r);
    if (rt->m < 64 || rt->m > 16384 || rt->m % 64 != 0)
        return fail(MOE_ERR_INVALID_ARG, "router m = %d: need a multiple of 64 in [64, 16384]", rt->m);
    if (!std::isfinite(rt->gamma)) return fail(MOE_ERR_INVALID_ARG, "router gamma must be finite");
    if (!(rt->eps >= 0.f) || !std::isfinite(rt->eps))
        return fail(MOE_ERR_INVALID_ARG, "router eps must be finite and >= 0");
    if (cfg->dtype != MOE_BF16)
        return fail(MOE_ERR_UNSUPPORTED, "the MLP router runs on bf16 layers only");
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_mlp_router_workspace_size(const moe_config* cfg, const moe_mlp_router* router,
                                         size_t* bytes) {
    CHECK(check_mlp(cfg, router));
    if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = moe::mlp_router_workspace_bytes(cfg->T, router->r, router->m, cfg->E);
    return MOE_OK;
}

moe_status moe_route_mlp(const moe_config* cfg, const moe_mlp_router* rt, const void* x,
                         const void* prev, float* logits, int32_t* topk_idx, float* topk_gate,
                         void* workspace, size_t ws_bytes, void* stream) {
    CHECK(check_mlp(cfg, rt));
    SIZES(cfg);
    const size_t r = (size_t)rt->r, m = (size_t)rt->m;
    CHECK(check_ptr(x, "x", T * d * es));
    CHECK(check_ptr(prev, "prev", T * r * es, true));
    CHECK(check_ptr(rt->w_down, "w_down", d * r * es));
    CHECK(check_ptr(rt->b_down, "b_down", r * 4, true));
    CHECK(check_ptr(rt->w1, "w1", r * m * es));
    CHECK(check_ptr(rt->b1, "b1", m * 4, true));
    CHECK(check_ptr(rt->w2, "w2", m * m * es));
    CHECK(check_ptr(rt->b2, "b2", m * 4, true));
    CHECK(check_ptr(rt->w3, "w3", m * E * es));
    CHECK(check_ptr(rt->b3, "b3", E * 4, true));
    CHECK(check_ptr(rt->pid_bias, "pid_bias", E * 4, true));
    CHECK(check_ptr(logits, "logits", T * E * 4));
    CHECK(check_ptr(topk_idx, "topk_idx", T * k * 4));
    CHECK(check_ptr(topk_gate, "topk_gate", T * k * 4));
    const size_t need = moe::mlp_router_workspace_bytes(cfg->T, rt->r, rt->m, cfg->E);
    if (T > 0 && (workspace == nullptr || ws_bytes < need))
        return fail(MOE_ERR_WORKSPACE, "MLP router workspace: need %zu bytes, got %zu", need, ws_bytes);
    CHECK(check_ptr(workspace, "workspace", T > 0 ? need : 0));
    hipError_t e = moe::launch_route_mlp(
        (const uint16_t*)x, (const uint16_t*)prev, rt->gamma, rt->eps,
        (const uint16_t*)rt->w_down, rt->b_down, (const uint16_t*)rt->w1, rt->b1,
        (const uint16_t*)rt->w2, rt->b2, (const uint16_t*)rt->w3, rt->b3, rt->pid_bias, logits,
        topk_idx, topk_gate, cfg->T, cfg->d, rt->r, rt->m, cfg->E, topk_params(cfg), workspace,
        gemm_grid_cap() / 2, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route_mlp");
}

moe_status moe_load_stats(const moe_config* cfg, const int32_t* expert_count, double* stats,
                          void* stream) {
    CHECK(check_cfg(cfg));
    SIZES(cfg);
    if (expert_count == nullptr) return fail(MOE_ERR_INVALID_ARG, "expert_count is NULL");
    CHECK(check_ptr(expert_count, "expert_count", E * 4));
    if (stats == nullptr) return fail(MOE_ERR_INVALID_ARG, "stats is NULL");
    CHECK(check_ptr(stats, "stats", 8 * sizeof(double)));
    hipError_t e = moe::launch_load_stats(expert_count, cfg->E, capacity_eff(cfg), stats,
                                          (hipStream_t)stream, dyn_route(cfg), cfg->cap_num,
                                          cfg->cap_den, cfg->T);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_load_stats");
}

moe_status moe_pid_update(const moe_config* cfg, const moe_pid_gains* gains,
                          const int32_t* expert_count, double* state, float* pid_bias,
                          void* stream) {
    CHECK(check_cfg(cfg));
    const size_t E = (size_t)cfg->E;
    if (gains == nullptr) return fail(MOE_ERR_INVALID_ARG, "gains is NULL");
    const double g[4] = {gains->kp, gains->ki, gains->kd, gains->scale};
    for (double v : g)
        if (!std::isfinite(v)) return fail(MOE_ERR_INVALID_ARG, "PID gains and scale must be finite");
    if (expert_count == nullptr) return fail(MOE_ERR_INVALID_ARG, "expert_count is NULL");
    CHECK(check_ptr(expert_count, "expert_count", E * 4));
    if (state == nullptr) return fail(MOE_ERR_INVALID_ARG, "state is NULL");
    CHECK(check_ptr(state, "state", 2 * E * sizeof(double)));
    if (pid_bias == nullptr) return fail(MOE_ERR_INVALID_ARG, "pid_bias is NULL");
    CHECK(check_ptr(pid_bias, "pid_bias", E * 4));
    hipError_t e = moe::launch_pid_update(expert_count, cfg->E, gains->kp, gains->ki, gains->kd,
                                          gains->scale, state, pid_bias, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_pid_update");
}

moe_status moe_forward(const moe_config* cfg, const void* x, const void* w_router,
                       const float* bias, const void* w_gate, const void* w_up,
                       const void* w_down, void* y, void* workspace, size_t ws_bytes,
                       void* stream) {
    CHECK(check_cfg(cfg));
    SIZES(cfg);
    CHECK(check_ptr(x, "x", T * d * es));
    CHECK(check_ptr(w_router, "w_router", d * E * es));
    CHECK(check_ptr(bias, "bias", E * 4, true));
    CHECK(check_ptr(w_gate, "w_gate", E * d * F * es));
    CHECK(check_ptr(w_up, "w_up", E * d * F * es));
    CHECK(check_ptr(w_down, "w_down", E * d * F * es));
    CHECK(check_ptr(y, "y", T * d * es));
    const FwdLayout L = fwd_layout(cfg);
    if (workspace == nullptr || ws_bytes < L.total)
        return fail(MOE_ERR_WORKSPACE, "forward workspace: need %zu bytes, got %zu", L.total, ws_bytes);
    CHECK(check_ptr(workspace, "workspace", 1));
    char* w = (char*)workspace;
    float* logits = (float*)(w + L.logits);
    int32_t* idx = (int32_t*)(w + L.idx);
    float* gate = (float*)(w + L.gate);
    int32_t* count = (int32_t*)(w + L.count);
    int32_t* offset = (int32_t*)(w + L.offset);
    int32_t* row_of = (int32_t*)(w + L.row_of);
    int32_t* tor = (int32_t*)(w + L.token_of_row);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = moe::launch_route(cfg->dtype, x, w_router, bias, logits, idx, gate, cfg->T,
                                     cfg->d, cfg->E, topk_params(cfg), s);
    if (e != hipSuccess) return hip_fail(e, "moe_forward/route");
    const bool gather = fwd_gather(cfg);   // no x_perm: see fwd_gather
    const moe::DispatchPlan p = dispatch_plan(cfg);
    e = moe::launch_dispatch(p, cfg->dtype, idx, x, w + L.x_perm, count, offset, row_of, tor,
                             w + L.dsp, cfg->d, s, !gather);
    if (e != hipSuccess) return hip_fail(e, "moe_forward/dispatch");
    e = moe::launch_gate_up(cfg->dtype, gather ? x : (const void*)(w + L.x_perm), offset, w_gate,
                            w_up, w + L.h, cfg->E, cfg->d, cfg->d_ff, max_rows(cfg),
                            gemm_grid_cap(), s, gather ? tor : nullptr);
    if (e != hipSuccess) return hip_fail(e, "moe_forward/gate_up");
    // output path: see fwd_direct / fwd_down_split
    const bool direct = fwd_direct(cfg);
    if (fwd_down_split(cfg)) {
        const long long pst = max_rows(cfg) * cfg->d;
        float* P = (float*)(w + L.part);
        e = moe::launch_mfma_down_split((const uint16_t*)(w + L.h), offset,
                                        (const uint16_t*)w_down, P, pst, cfg->E, cfg->d,
                                        cfg->d_ff, max_rows(cfg), gemm_grid_cap() / 2, s);
        if (e != hipSuccess) return hip_fail(e, "moe_forward/down");
        e = moe::launch_combine_split(P, pst, row_of, gate, y, cfg->T, cfg->d, s);
        if (e != hipSuccess) return hip_fail(e, "moe_forward/combine");
        return MOE_OK;
    }
    e = moe::launch_down(cfg->dtype, w + L.h, offset, w_down, w + L.y_perm, cfg->E, cfg->d,
                         cfg->d_ff, max_rows(cfg), gemm_grid_cap(), s, direct ? gate : nullptr,
                         direct ? tor : nullptr, direct ? y : nullptr);
    if (e != hipSuccess) return hip_fail(e, "moe_forward/down");
    if (direct) return MOE_OK;
    e = moe::launch_combine(cfg->dtype, w + L.y_perm, row_of, gate, y, cfg->T, cfg->d, cfg->k, s);
    if (e != hipSuccess) return hip_fail(e, "moe_forward/combine");
    return MOE_OK;
}

}  // extern "C"

namespace {

// bf16 backward: the forward's maps, x and dy in expert-grouped row order,
// the recomputed pre-activations and the gradients of every product.
struct BwdLayout {
    size_t logits, idx, gate, count, offset, row_of, token_of_row, dsp, x_perm, dy_perm, G, U,
        gH, rgate, dot, dXp, dgrow, dl, dwr, total;
    int dx_parts;   // parts of dx_perm (K slices; each sums the gate and up products)
};

BwdLayout bwd_layout(const moe_config* c) {
    const size_t T = (size_t)c->T, E = (size_t)c->E, k = (size_t)c->k, d = (size_t)c->d;
    const size_t F = (size_t)c->d_ff, R = (size_t)max_rows(c);
    const moe::DispatchPlan p = dispatch_plan(c);
    BwdLayout L;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
    L.logits = take(T * E * 4);
    L.idx = take(T * k * 4);
    L.gate = take(T * k * 4);
    L.count = take(E * 4);
    L.offset = take((E + 1) * 4);
    L.row_of = take(T * k * 4);
    L.token_of_row = take((size_t)tor_len(c) * 4);   // the padded layout: E * C rows
    L.dsp = take(moe::dispatch_workspace_bytes(p));
    const size_t es = (size_t)esize(c);
    L.x_perm = take(R * d * es);
    L.dy_perm = take(R * d * es);
    L.G = take(R * F * es);
    L.U = take(R * F * es);
    L.gH = take(R * F * es);
    L.rgate = take(R * 4);
    L.dot = take(R * (F / 64) * 4);
    L.dx_parts = c->dtype == MOE_BF16
                     ? moe::bw_nt_ksplit((long long)R, c->E, c->d, c->d_ff, 1, gemm_grid_cap())
                     : 1;
    L.dXp = take((size_t)L.dx_parts * R * d * 4);
    L.dgrow = take(R * 4);
    L.dl = take(T * E * 4);
    L.dwr = take(moe::dwr_workspace_bytes(c->T, c->d, c->E));
    L.total = o;
    return L;
}

moe_status check_bwd(const moe_config* cfg) {
    CHECK(check_cfg(cfg));
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_backward_workspace_size(const moe_config* cfg, size_t* bytes) {
    CHECK(check_bwd(cfg));
    if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = bwd_layout(cfg).total;
    return MOE_OK;
}

moe_status moe_backward(const moe_config* cfg, const void* x, const void* w_router,
                        const float* bias, const void* w_gate, const void* w_up,
                        const void* w_down, const void* dy, void* dx, float* dw_router,
                        float* dbias, float* dw_gate, float* dw_up, float* dw_down, float* dgate,
                        void* workspace, size_t ws_bytes, void* stream) {
    CHECK(check_bwd(cfg));
    SIZES(cfg);
    CHECK(check_ptr(x, "x", T * d * es));
    CHECK(check_ptr(w_router, "w_router", d * E * es));
    CHECK(check_ptr(bias, "bias", E * 4, true));
    CHECK(check_ptr(w_gate, "w_gate", E * d * F * es));
    CHECK(check_ptr(w_up, "w_up", E * d * F * es));
    CHECK(check_ptr(w_down, "w_down", E * d * F * es));
    CHECK(check_ptr(dy, "dy", T * d * es));
    CHECK(check_ptr(dx, "dx", T * d * es));
    CHECK(check_ptr(dw_router, "dw_router", d * E * 4));
    CHECK(check_ptr(dbias, "dbias", E * 4, true));
    CHECK(check_ptr(dw_gate, "dw_gate", E * d * F * 4));
    CHECK(check_ptr(dw_up, "dw_up", E * d * F * 4));
    CHECK(check_ptr(dw_down, "dw_down", E * d * F * 4));
    CHECK(check_ptr(dgate, "dgate", T * k * 4, true));
    const BwdLayout L = bwd_layout(cfg);
    if (workspace == nullptr || ws_bytes < L.total)
        return fail(MOE_ERR_WORKSPACE, "backward workspace: need %zu bytes, got %zu", L.total, ws_bytes);
    CHECK(check_ptr(workspace, "workspace", 1));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
#define BWD(call, where)                                   \
    do {                                                   \
        e = (call);                                        \
        if (e != hipSuccess) return hip_fail(e, where);    \
    } while (0)
    if (T == 0) {   // no tokens: every weight gradient is zero
        BWD(moe::launch_zero_f32(dw_router, (long long)(d * E), s), "moe_backward/zero");
        BWD(moe::launch_zero_f32(dbias, (long long)E, s), "moe_backward/zero");
        BWD(moe::launch_zero_f32(dw_gate, (long long)(E * d * F), s), "moe_backward/zero");
        BWD(moe::launch_zero_f32(dw_up, (long long)(E * d * F), s), "moe_backward/zero");
        BWD(moe::launch_zero_f32(dw_down, (long long)(E * d * F), s), "moe_backward/zero");
        return MOE_OK;
    }
    char* w = (char*)workspace;
    float* logits = (float*)(w + L.logits);
    int32_t* idx = (int32_t*)(w + L.idx);
    float* gate = (float*)(w + L.gate);
    int32_t* count = (int32_t*)(w + L.count);
    int32_t* offset = (int32_t*)(w + L.offset);
    int32_t* row_of = (int32_t*)(w + L.row_of);
    int32_t* tor = (int32_t*)(w + L.token_of_row);
    void* G = w + L.G;
    void* U = w + L.U;
    void* gH = w + L.gH;
    float* rgate = (float*)(w + L.rgate);
    float* dot = (float*)(w + L.dot);
    float* dXp = (float*)(w + L.dXp);
    float* dgrow = (float*)(w + L.dgrow);
    float* dl = (float*)(w + L.dl);
    const bool bf = cfg->dtype == MOE_BF16;
    const int Ei = cfg->E, di = cfg->d, Fi = cfg->d_ff, ki = cfg->k;
    const long long Rl = max_rows(cfg);
    const int cus = gemm_grid_cap();

    // forward recompute: routing, dispatch maps and x_perm, g = x W_gate, u = x W_up
    BWD(moe::launch_route(cfg->dtype, x, w_router, bias, logits, idx, gate, cfg->T, di, Ei,
                          topk_params(cfg), s), "moe_backward/route");
    const moe::DispatchPlan p = dispatch_plan(cfg);
    void* x_perm = w + L.x_perm;
    void* dy_perm = w + L.dy_perm;
    BWD(moe::launch_dispatch(p, cfg->dtype, idx, x, x_perm, count, offset, row_of, tor,
                             w + L.dsp, di, s, true), "moe_backward/dispatch");
    BWD(moe::launch_scatter_rows(dy, row_of, dy_perm, cfg->T, (int)(di * es), ki, s),
        "moe_backward/scatter_dy");
    if (cfg->layout == MOE_LAYOUT_PADDED)   // empty rows of dy in expert order are zero, as x's
        BWD(moe::launch_zero_empty_rows(count, p.C, Ei, tor, dy_perm, (int)(di * es), s),
            "moe_backward/pad_dy");
    if (bf)
        BWD(moe::launch_mfma_gate_up_pre((const uint16_t*)x_perm, nullptr, offset,
                                         (const uint16_t*)w_gate, (const uint16_t*)w_up,
                                         (uint16_t*)G, (uint16_t*)U, Ei, di, Fi, Rl, cus, s),
            "moe_backward/gate_up");
    else
        BWD(moe::launch_gate_up_pre_f32((const float*)x_perm, offset, (const float*)w_gate,
                                        (const float*)w_up, (float*)G, (float*)U, Ei, di, Fi, Rl,
                                        cus, s), "moe_backward/gate_up");
    // dh_raw = dy W_down^T per kept row with the GeGLU backward in its
    // epilogue (G, U -> dg, du in place, gate h, partial dgate sums), then
    // dgate per row
    BWD(moe::launch_row_gate(offset, tor, row_of, gate, Ei, ki, Rl, rgate, s),
        "moe_backward/row_gate");
    if (bf)
        BWD(moe::launch_bw_nt_geglu((const uint16_t*)dy_perm, (const uint16_t*)w_down,
                                    (uint16_t*)G, (uint16_t*)U, (uint16_t*)gH, rgate, dot, offset,
                                    Ei, Fi, di, Rl, cus, s), "moe_backward/dh_geglu");
    else
        BWD(moe::launch_bw_nt_geglu_f32((const float*)dy_perm, (const float*)w_down, (float*)G,
                                        (float*)U, (float*)gH, rgate, dot, offset, Ei, Fi, di, Rl,
                                        cus, s), "moe_backward/dh_geglu");
    BWD(moe::launch_dgate_sum(dot, Fi / 64, offset, Ei, Rl, dgrow, s), "moe_backward/dgate");
    // G, U now hold dg, du
    // dx_perm in parts, one per K slice, each dg W_gate^T + du W_up^T over that
    // slice in one accumulator; summed by launch_dx
    const long long part = Rl * (long long)di;
    if (bf) {
        BWD(moe::launch_bw_nt((const uint16_t*)G, (const uint16_t*)w_gate, (const uint16_t*)U,
                              (const uint16_t*)w_up, dXp, part, L.dx_parts, offset, Ei, di, Fi, Rl,
                              cus, s), "moe_backward/dx_perm");
        BWD(moe::launch_bw_tn((const uint16_t*)x_perm, (const uint16_t*)G, dw_gate, offset, Ei,
                              di, Fi, cus, s), "moe_backward/dw_gate");
        BWD(moe::launch_bw_tn((const uint16_t*)x_perm, (const uint16_t*)U, dw_up, offset, Ei, di,
                              Fi, cus, s), "moe_backward/dw_up");
        BWD(moe::launch_bw_tn((const uint16_t*)gH, (const uint16_t*)dy_perm, dw_down, offset, Ei,
                              Fi, di, cus, s), "moe_backward/dw_down");
    } else {
        BWD(moe::launch_bw_nt_f32((const float*)G, (const float*)w_gate, (const float*)U,
                                  (const float*)w_up, dXp, offset, Ei, di, Fi, Rl, cus, s),
            "moe_backward/dx_perm");
        BWD(moe::launch_bw_tn_f32((const float*)x_perm, (const float*)G, dw_gate, offset, Ei, di,
                                  Fi, cus, s), "moe_backward/dw_gate");
        BWD(moe::launch_bw_tn_f32((const float*)x_perm, (const float*)U, dw_up, offset, Ei, di,
                                  Fi, cus, s), "moe_backward/dw_up");
        BWD(moe::launch_bw_tn_f32((const float*)gH, (const float*)dy_perm, dw_down, offset, Ei,
                                  Fi, di, cus, s), "moe_backward/dw_down");
    }
    // router: dlogit, then dx and the router's weight and bias gradients
    BWD(moe::launch_router_bwd(logits, idx, gate, row_of, dgrow, cfg->T, Ei, ki, cfg->temperature,
                               cfg->renormalize, dl, dgate, s), "moe_backward/router");
    if (bf)
        BWD(moe::launch_dx(dl, (const uint16_t*)w_router, dXp, L.dx_parts, part, row_of,
                           (uint16_t*)dx, cfg->T, di, Ei, ki, s), "moe_backward/dx");
    else
        BWD(moe::launch_dx_f32(dl, (const float*)w_router, dXp, row_of, (float*)dx, cfg->T, di,
                               Ei, ki, s), "moe_backward/dx");
    BWD(moe::launch_dwr(cfg->dtype, x, dl, dw_router, dbias, cfg->T, di, Ei, w + L.dwr, s),
        "moe_backward/dwr");
#undef BWD
    return MOE_OK;
}

}  // extern "C"
