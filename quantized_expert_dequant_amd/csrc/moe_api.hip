// moe_api.hip - the extern "C" boundary of libmoe.so (declared in include/moe.h):
// argument validation, workspace carving and launch sequencing.  No entry point
// allocates memory or synchronizes the host.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/moe.h"
#include "grouped.h"
#include "launch.h"

using namespace moe;

namespace {

thread_local char g_err[512] = "";
thread_local Timing g_timing[KID_COUNT];

int fail(int code, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok()
{
    g_err[0] = '\0';
    return MOE_OK;
}

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }
bool misaligned4(const void* p) { return ((uintptr_t)p & 3u) != 0; }

#define CHECK_PTR(p)                                                                \
    do {                                                                            \
        if (!(p)) return fail(MOE_EINVAL, "%s: %s is NULL", fn, #p);                \
        if (misaligned(p)) return fail(MOE_EINVAL, "%s: %s is not 16-byte aligned", fn, #p); \
    } while (0)

#define CHECK_PTR4(p)                                                               \
    do {                                                                            \
        if (!(p)) return fail(MOE_EINVAL, "%s: %s is NULL", fn, #p);                \
        if (misaligned4(p)) return fail(MOE_EINVAL, "%s: %s is not 4-byte aligned", fn, #p); \
    } while (0)

#define CHECK_OPT_PTR4(p)                                                           \
    do {                                                                            \
        if ((p) && misaligned4(p)) return fail(MOE_EINVAL, "%s: %s is not 4-byte aligned", fn, #p); \
    } while (0)

#define CHECK_OPT_PTR(p)                                                            \
    do {                                                                            \
        if ((p) && misaligned(p)) return fail(MOE_EINVAL, "%s: %s is not 16-byte aligned", fn, #p); \
    } while (0)

int check_shape(const char* fn, int bits, int H, int I, int group)
{
    if (bits != 2 && bits != 4) return fail(MOE_EUNSUPPORTED, "%s: bits=%d (must be 2 or 4)", fn, bits);
    if (group != 64) return fail(MOE_EUNSUPPORTED, "%s: group=%d (must be 64)", fn, group);
    if (H <= 0 || I <= 0 || H % 64 || I % 64)
        return fail(MOE_EINVAL, "%s: H=%d and I=%d must be positive multiples of 64", fn, H, I);
    if (H > 65536 || I > 8192) return fail(MOE_EUNSUPPORTED, "%s: H=%d > 65536 or I=%d > 8192", fn, H, I);
    return MOE_OK;
}

int check_routing(const char* fn, int B, int E, int K)
{
    if (B < 1) return fail(MOE_EINVAL, "%s: B=%d (must be >= 1)", fn, B);
    if (B > MOE_MAX_B) return fail(MOE_EUNSUPPORTED, "%s: B=%d > %d", fn, B, MOE_MAX_B);
    if (E < 1) return fail(MOE_EINVAL, "%s: E=%d (must be >= 1)", fn, E);
    if (E > MOE_MAX_E) return fail(MOE_EUNSUPPORTED, "%s: E=%d > %d", fn, E, MOE_MAX_E);
    if (K < 1) return fail(MOE_EINVAL, "%s: K=%d (must be >= 1)", fn, K);
    if (K > MOE_MAX_K) return fail(MOE_EUNSUPPORTED, "%s: K=%d > %d", fn, K, MOE_MAX_K);
    if (K > E) return fail(MOE_EINVAL, "%s: K=%d > E=%d", fn, K, E);
    return MOE_OK;
}

int check_desc(const char* fn, const moe_layer_desc* d, int B)
{
    if (!d) return fail(MOE_EINVAL, "%s: desc is NULL", fn);
    int rc = check_shape(fn, d->bits, d->H, d->I, d->group);
    if (rc) return rc;
    rc = check_routing(fn, B, d->E, d->K);
    if (rc) return rc;
    if (!d->experts) return fail(MOE_EINVAL, "%s: desc->experts is NULL", fn);
    if (misaligned(d->experts)) return fail(MOE_EINVAL, "%s: desc->experts is not 16-byte aligned", fn);
    return MOE_OK;
}

size_t up256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace sections (each 256-byte aligned): the logits, the routing (when
// the caller does not want it back), the token's dequant operand and h; for a
// batch that takes the grouped path, its sections follow.
struct Work {
    double* logits;
    int32_t* idx;
    float* w;
    uint4* xq;
    float4* xst;
    void* hq;
    bool grouped;
    GroupedWork gw;
    size_t bytes;
};

Work carve(void* ws, int bits, int B, int H, int I, int E, int K)
{
    Work W;
    char* p = (char*)ws;
    size_t off = 0;
    auto take = [&](size_t n) {
        char* q = p ? p + off : nullptr;
        off += up256(n);
        return q;
    };
    const size_t Gh = H / 64, Gi = I / 64, S = (size_t)B * (K + 1);
    W.logits = (double*)take((size_t)B * E * 8);
    W.idx = (int32_t*)take((size_t)B * K * 4);
    W.w = (float*)take((size_t)B * K * 4);
    W.xq = (uint4*)take((size_t)B * Gh * 128);
    W.xst = (float4*)take((size_t)B * Gh * 16);
    W.hq = take(S * Gi * 256);  // h in fp32
    const Layout L = make_layout(bits, H, I);
    W.grouped = grouped_supported(L, B, K);
    W.gw = GroupedWork{};
    if (W.grouped) {
        const size_t n = grouped_workspace_bytes(L, B, K, E);
        if (p) W.gw = carve_grouped(p + off, L, B, K, E);
        off += up256(n);
    }
    W.bytes = off;
    return W;
}

int hip_status(const char* fn)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", fn, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err; }

int moe_set_timing_events(int kernel, void* start_event, void* stop_event)
{
    const char* fn = "moe_set_timing_events";
    if (kernel < MOE_KERNEL_ROUTER || kernel > MOE_KERNEL_DOWN) return fail(MOE_EINVAL, "%s: kernel=%d", fn, kernel);
    if ((start_event == nullptr) != (stop_event == nullptr))
        return fail(MOE_EINVAL, "%s: set both events or neither", fn);
    g_timing[kernel].start = (hipEvent_t)start_event;
    g_timing[kernel].stop = (hipEvent_t)stop_event;
    return ok();
}

size_t moe_expert_record_bytes(int bits, int H, int I, int group)
{
    if (check_shape("moe_expert_record_bytes", bits, H, I, group)) return 0;
    return (size_t)make_layout(bits, H, I).record;
}

size_t moe_workspace_bytes(const moe_layer_desc* desc, int B)
{
    if (!desc || check_shape("moe_workspace_bytes", desc->bits, desc->H, desc->I, desc->group) ||
        check_routing("moe_workspace_bytes", B, desc->E, desc->K))
        return 0;
    return carve(nullptr, desc->bits, B, desc->H, desc->I, desc->E, desc->K).bytes;
}

size_t moe_route_workspace_bytes(int B, int E, int K)
{
    if (check_routing("moe_route_workspace_bytes", B, E, K)) return 0;
    return up256((size_t)B * E * 8);
}

size_t moe_stack_extra_bytes(int B, int H)
{
    if (B < 1 || B > MOE_MAX_B || H <= 0) return 0;
    return 2 * up256((size_t)B * H * 4);
}

int moe_pack_experts(int bits, int H, int I, int group, int n_experts, const uint8_t* gate_codes,
                     const uint8_t* up_codes, const uint8_t* down_codes, const uint16_t* scales_bf16,
                     const uint16_t* biases_bf16, void* slab_out, int first_expert, void* stream)
{
    const char* fn = "moe_pack_experts";
    int rc = check_shape(fn, bits, H, I, group);
    if (rc) return rc;
    if (n_experts < 1 || n_experts > 65535 || first_expert < 0)
        return fail(MOE_EINVAL, "%s: n_experts=%d first_expert=%d", fn, n_experts, first_expert);
    CHECK_PTR(gate_codes);
    CHECK_PTR(up_codes);
    CHECK_PTR(down_codes);
    CHECK_PTR(scales_bf16);
    CHECK_PTR(biases_bf16);
    CHECK_PTR(slab_out);
    const Layout L = make_layout(bits, H, I);
    launch_pack(L, n_experts, gate_codes, up_codes, down_codes, scales_bf16, biases_bf16, slab_out, first_expert,
                (hipStream_t)stream);
    return hip_status(fn);
}

int moe_dequant_expert(int bits, int H, int I, int group, const void* record, float* W_out, void* stream)
{
    const char* fn = "moe_dequant_expert";
    int rc = check_shape(fn, bits, H, I, group);
    if (rc) return rc;
    CHECK_PTR(record);
    CHECK_PTR(W_out);
    launch_dequant(make_layout(bits, H, I), record, W_out, (hipStream_t)stream);
    return hip_status(fn);
}

int moe_route_topk(const float* x, int B, const float* w_router, const float* logit_bias, int H, int E, int K,
                   int renormalize, int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes, void* stream)
{
    const char* fn = "moe_route_topk";
    int rc = check_routing(fn, B, E, K);
    if (rc) return rc;
    if (H <= 0 || H % 64) return fail(MOE_EINVAL, "%s: H=%d must be a positive multiple of 64", fn, H);
    CHECK_PTR(x);
    CHECK_PTR(w_router);
    CHECK_OPT_PTR4(logit_bias);
    CHECK_PTR4(idx_out);
    CHECK_PTR4(w_out);
    CHECK_PTR(ws);
    const size_t need = moe_route_workspace_bytes(B, E, K);
    if (ws_bytes < need) return fail(MOE_EINVAL, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
    hipStream_t s = (hipStream_t)stream;
    launch_router(4, x, B, w_router, logit_bias, H, E, (double*)ws, nullptr, nullptr, s, g_timing[KID_ROUTER]);
    launch_topk((const double*)ws, B, E, K, renormalize ? 1 : 0, idx_out, w_out, s);
    return hip_status(fn);
}

static int expert_ffn(const char* fn, int bits, const moe_layer_desc* desc, const float* x, int B,
                      const int32_t* idx, const float* w, float* y_out, void* ws, size_t ws_bytes, void* stream)
{
    int rc = check_desc(fn, desc, B);
    if (rc) return rc;
    if (desc->bits != bits) return fail(MOE_EINVAL, "%s: desc->bits=%d, this entry point needs %d", fn, desc->bits, bits);
    CHECK_PTR(x);
    CHECK_PTR4(idx);
    CHECK_PTR4(w);
    CHECK_PTR(y_out);
    CHECK_PTR(ws);
    const Work W = carve(ws, desc->bits, B, desc->H, desc->I, desc->E, desc->K);
    if (ws_bytes < W.bytes) return fail(MOE_EINVAL, "%s: workspace %zu < %zu bytes", fn, ws_bytes, W.bytes);
    hipStream_t s = (hipStream_t)stream;
    const Layout L = make_layout(desc->bits, desc->H, desc->I);
    if (W.grouped) {
        launch_group(idx, B, desc->K, desc->E, gemv_tokens(L), W.gw.g, s);
        launch_ffn_grouped(L, desc->experts, W.gw, x, w, desc->shared_weight, B, desc->K, desc->E, W.xq, W.xst, false,
                           y_out, s, g_timing[KID_GATEUP], g_timing[KID_DOWN]);
        return hip_status(fn);
    }
    launch_prep(desc->bits, x, B, desc->H, W.xq, W.xst, s);
    launch_ffn(L, desc->experts, W.xq, W.xst, nullptr, 0, const_cast<int32_t*>(idx), const_cast<float*>(w), B,
               desc->K, desc->E, desc->shared_weight, W.hq, y_out, s, g_timing[KID_GATEUP], g_timing[KID_DOWN]);
    return hip_status(fn);
}

int moe_expert_ffn_q4(const moe_layer_desc* desc, const float* x, int B, const int32_t* idx, const float* w,
                      float* y_out, void* ws, size_t ws_bytes, void* stream)
{
    return expert_ffn("moe_expert_ffn_q4", 4, desc, x, B, idx, w, y_out, ws, ws_bytes, stream);
}

int moe_expert_ffn_q2(const moe_layer_desc* desc, const float* x, int B, const int32_t* idx, const float* w,
                      float* y_out, void* ws, size_t ws_bytes, void* stream)
{
    return expert_ffn("moe_expert_ffn_q2", 2, desc, x, B, idx, w, y_out, ws, ws_bytes, stream);
}

// norm_eps >= 0 (per-token path only): x is the previous layer's output, renormalized
// by the router kernel on the fly
static int layer_impl(const char* fn, const moe_layer_desc* d, const float* x, int B, float* y_out,
                      int32_t* idx_out, float* w_out, const Work& W, hipStream_t s, float norm_eps = -1.f)
{
    int32_t* idx = idx_out ? idx_out : W.idx;
    float* w = w_out ? w_out : W.w;
    const Layout L = make_layout(d->bits, d->H, d->I);
    if (W.grouped) {
        const TokenPrep P{x, d->H, W.gw.xh, W.gw.xsum, W.gw.xscale, gemv_tokens(L) > 1 ? W.xq : nullptr, W.xst};
        launch_route_batched(x, B, d->w_router, d->logit_bias, d->H, d->E, d->K, d->renormalize ? 1 : 0,
                             W.gw.partial, idx, w, P, s, g_timing[KID_ROUTER]);
        launch_group(idx, B, d->K, d->E, gemv_tokens(L), W.gw.g, s);
        launch_ffn_grouped(L, d->experts, W.gw, x, w, d->shared_weight, B, d->K, d->E, W.xq, W.xst, true, y_out, s,
                           g_timing[KID_GATEUP], g_timing[KID_DOWN]);
        return hip_status(fn);
    }
    launch_router(d->bits, x, B, d->w_router, d->logit_bias, d->H, d->E, W.logits, W.xq, W.xst, s,
                  g_timing[KID_ROUTER], norm_eps);
    launch_ffn(L, d->experts, W.xq, W.xst, W.logits, d->renormalize ? 1 : 0, idx, w, B, d->K, d->E,
               d->shared_weight, W.hq, y_out, s, g_timing[KID_GATEUP], g_timing[KID_DOWN]);
    return hip_status(fn);
}

int moe_layer_decode(const moe_layer_desc* desc, const float* x, int B, float* y_out, int32_t* idx_out,
                     float* w_out, void* ws, size_t ws_bytes, void* stream)
{
    const char* fn = "moe_layer_decode";
    int rc = check_desc(fn, desc, B);
    if (rc) return rc;
    CHECK_PTR(desc->w_router);
    CHECK_OPT_PTR4(desc->logit_bias);
    CHECK_PTR(x);
    CHECK_PTR(y_out);
    CHECK_OPT_PTR4(idx_out);
    CHECK_OPT_PTR4(w_out);
    CHECK_PTR(ws);
    const Work W = carve(ws, desc->bits, B, desc->H, desc->I, desc->E, desc->K);
    if (ws_bytes < W.bytes) return fail(MOE_EINVAL, "%s: workspace %zu < %zu bytes", fn, ws_bytes, W.bytes);
    return layer_impl(fn, desc, x, B, y_out, idx_out, w_out, W, (hipStream_t)stream);
}

int moe_group_tokens(const int32_t* idx, int B, int K, int E, int32_t* offsets_out, int32_t* tokens_out,
                     int32_t* slots_out, void* stream)
{
    const char* fn = "moe_group_tokens";
    int rc = check_routing(fn, B, E, K);
    if (rc) return rc;
    CHECK_PTR4(idx);
    CHECK_PTR4(offsets_out);
    CHECK_PTR4(tokens_out);
    CHECK_PTR4(slots_out);
    GroupOut O{};
    O.offsets = offsets_out;
    O.tokens = tokens_out;
    O.slots = slots_out;
    launch_group(idx, B, K, E, 1, O, (hipStream_t)stream);
    return hip_status(fn);
}

int moe_rmsnorm(const float* y, int B, int H, float eps, float* x_out, void* stream)
{
    const char* fn = "moe_rmsnorm";
    if (B < 1 || B > MOE_MAX_B || H <= 0) return fail(MOE_EINVAL, "%s: B=%d H=%d", fn, B, H);
    if (!(eps >= 0.f)) return fail(MOE_EINVAL, "%s: eps must be >= 0", fn);
    CHECK_PTR(y);
    CHECK_PTR(x_out);
    launch_rmsnorm(y, B, H, eps, x_out, (hipStream_t)stream);
    return hip_status(fn);
}

int moe_stack_decode(const moe_layer_desc* layers, int n_layers, const float* x, int B, float eps, float* y_out,
                     int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes, void* stream)
{
    const char* fn = "moe_stack_decode";
    if (!layers || n_layers < 1) return fail(MOE_EINVAL, "%s: no layers", fn);
    if (!(eps >= 0.f)) return fail(MOE_EINVAL, "%s: eps must be >= 0", fn);
    for (int l = 0; l < n_layers; ++l) {
        int rc = check_desc(fn, &layers[l], B);
        if (rc) return rc;
        const moe_layer_desc& a = layers[l];
        const moe_layer_desc& z = layers[0];
        if (a.H != z.H || a.I != z.I || a.K != z.K || a.bits != z.bits || a.E != z.E)
            return fail(MOE_EINVAL, "%s: layer %d differs in shape from layer 0", fn, l);
        CHECK_PTR(a.w_router);
        CHECK_OPT_PTR4(a.logit_bias);
    }
    CHECK_PTR(x);
    CHECK_PTR(y_out);
    CHECK_OPT_PTR4(idx_out);
    CHECK_OPT_PTR4(w_out);
    CHECK_PTR(ws);
    const moe_layer_desc& d0 = layers[0];
    const Work W = carve(ws, d0.bits, B, d0.H, d0.I, d0.E, d0.K);
    const size_t vec = up256((size_t)B * d0.H * 4);
    const size_t need = W.bytes + 2 * vec;
    if (ws_bytes < need) return fail(MOE_EINVAL, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
    float* ybuf = (float*)((char*)ws + W.bytes);
    float* xbuf = (float*)((char*)ws + W.bytes + vec);
    hipStream_t s = (hipStream_t)stream;
    // Per-token path: each layer's router renormalizes the previous layer's output
    // itself (no separate pass), and the two buffers alternate so a layer never
    // writes the y it reads; the grouped path renormalizes ybuf into xbuf.
    const float* xl = x;
    float norm = -1.f;
    for (int l = 0; l < n_layers; ++l) {
        const bool last = (l == n_layers - 1);
        float* yl = last ? y_out : ((W.grouped || !(l & 1)) ? ybuf : xbuf);
        int32_t* il = idx_out ? idx_out + (size_t)l * B * d0.K : nullptr;
        float* wl = w_out ? w_out + (size_t)l * B * d0.K : nullptr;
        int rc = layer_impl(fn, &layers[l], xl, B, yl, il, wl, W, s, norm);
        if (rc) return rc;
        if (!last) {
            if (W.grouped) {
                launch_rmsnorm(ybuf, B, d0.H, eps, xbuf, s);
                xl = xbuf;
            } else {
                xl = yl;
                norm = eps;
            }
        }
    }
    return hip_status(fn);
}

}  // extern "C"
