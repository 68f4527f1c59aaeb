// moe_api.hip - the extern "C" boundary of libmoe.so (declared in include/moe.h):
// argument validation, workspace carving and launch sequencing.  No entry point
// allocates memory or synchronizes the host.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/moe.h"
#include "cache.h"
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
    if (bits != 2 && bits != 3 && bits != 4) return fail(MOE_EUNSUPPORTED, "%s: bits=%d (must be 2, 3 or 4)", fn, bits);
    if (group != 64 && group != 128 && group != 256)
        return fail(MOE_EUNSUPPORTED, "%s: group=%d (must be 64, 128 or 256)", fn, group);
    if (H <= 0 || I <= 0 || H % group || I % group)
        return fail(MOE_EINVAL, "%s: H=%d and I=%d must be positive multiples of the group (%d)", fn, H, I, group);
    if (H > 65536 || I > 8192) return fail(MOE_EUNSUPPORTED, "%s: H=%d > 65536 or I=%d > 8192", fn, H, I);
    // 3-bit down rows hold their high bits as half chunks, two units to a 16-byte chunk
    if (bits == 3 && I % 128) return fail(MOE_EINVAL, "%s: 3-bit codes need I=%d to be a multiple of 128", fn, I);
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

// allow_grouped = false: the per-token path's workspace only
Work carve(void* ws, int bits, int B, int H, int I, int E, int K, bool allow_grouped = true)
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
    const Layout L = make_layout(bits, H, I, 64);  // the workspace does not depend on the weight group
    W.grouped = allow_grouped && grouped_supported(L, B, K);
    W.gw = GroupedWork{};
    if (W.grouped) {
        const size_t n = grouped_workspace_bytes(L, B, K, E);
        if (p) W.gw = carve_grouped(p + off, L, B, K, E);
        off += up256(n);
    }
    W.bytes = off;
    return W;
}

// The backing store as a device address: pinned host memory is translated, device
// memory is used as it is.
const void* backing_device_ptr(const void* p)
{
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (a.type == hipMemoryTypeHost) {
        void* d = nullptr;
        if (hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        return d;
    }
    return p;
}

int hip_status(const char* fn)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", fn, hipGetErrorString(e));
    return ok();
}

// Workspace of moe_layer_decode_noalloc: one array per GPU, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not device
// memory: its device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;

// Device address of `scratch` on the current device, looked up on the first call
// per device (with that device current) under a lock; nullptr if the lookup fails.
void* scratch_ptr(const char* fn, int& rc)
{
    static std::mutex mu;
    static void* ptrs[NOALLOC_MAX_DEVICES];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) {
        rc = fail(MOE_EHIP, "%s: no current HIP device (or device id >= %d)", fn, NOALLOC_MAX_DEVICES);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            rc = fail(MOE_EHIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", fn, dev,
                      hipGetErrorString(e));
            return nullptr;
        }
        ptrs[dev] = p;
    }
    rc = MOE_OK;
    return ptrs[dev];
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
    return (size_t)make_layout(bits, H, I, group).record;
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
    const Layout L = make_layout(bits, H, I, group);
    launch_pack(L, n_experts, gate_codes, up_codes, down_codes, scales_bf16, biases_bf16, slab_out, first_expert,
                (hipStream_t)stream);
    return hip_status(fn);
}

int moe_requant_4to2(int H, int I, int group, int n_experts, const uint8_t* gate4, const uint8_t* up4,
                     const uint8_t* down4, const uint16_t* scales4, const uint16_t* biases4, uint8_t* gate2,
                     uint8_t* up2, uint8_t* down2, uint16_t* scales2, uint16_t* biases2, void* stream)
{
    const char* fn = "moe_requant_4to2";
    int rc = check_shape(fn, 4, H, I, group);
    if (rc) return rc;
    if (n_experts < 1 || n_experts > 65535) return fail(MOE_EINVAL, "%s: n_experts=%d", fn, n_experts);
    CHECK_PTR(gate4);
    CHECK_PTR(up4);
    CHECK_PTR(down4);
    CHECK_PTR(scales4);
    CHECK_PTR(biases4);
    CHECK_PTR(gate2);
    CHECK_PTR(up2);
    CHECK_PTR(down2);
    CHECK_PTR4(scales2);
    CHECK_PTR4(biases2);
    launch_requant_4to2(H, I, group, n_experts, gate4, up4, down4, scales4, biases4, gate2, up2, down2, scales2, biases2,
                        (hipStream_t)stream);
    return hip_status(fn);
}

int moe_expert_ranges(int bits, int H, int I, int group, const void* slab, int n_experts, int32_t* flags_out,
                      void* stream)
{
    const char* fn = "moe_expert_ranges";
    int rc = check_shape(fn, bits, H, I, group);
    if (rc) return rc;
    if (n_experts < 1 || n_experts > (1 << 24)) return fail(MOE_EINVAL, "%s: n_experts=%d", fn, n_experts);
    CHECK_PTR(slab);
    CHECK_PTR4(flags_out);
    const void* src = backing_device_ptr(slab);
    if (!src) return fail(MOE_EINVAL, "%s: slab is neither device memory nor pinned host memory", fn);
    const void* dst = backing_device_ptr(flags_out);
    if (!dst) return fail(MOE_EINVAL, "%s: flags_out is neither device memory nor pinned host memory", fn);
    launch_expert_ranges(make_layout(bits, H, I, group), src, n_experts, (int32_t*)dst, (hipStream_t)stream);
    return hip_status(fn);
}

int moe_gdn_step(int n_heads, int dk, int dv, float* state, const float* q, const float* k, const float* v,
                 const float* alpha, const float* beta, float* o_out, void* stream)
{
    const char* fn = "moe_gdn_step";
    if (n_heads < 1 || n_heads > 4096) return fail(MOE_EINVAL, "%s: n_heads=%d", fn, n_heads);
    if (dk != 64 && dk != 128 && dk != 256) return fail(MOE_EUNSUPPORTED, "%s: dk=%d (must be 64, 128 or 256)", fn, dk);
    if (dv < 1 || dv > 4096) return fail(MOE_EINVAL, "%s: dv=%d", fn, dv);
    CHECK_PTR4(state);
    CHECK_PTR4(q);
    CHECK_PTR4(k);
    CHECK_PTR4(v);
    CHECK_PTR4(alpha);
    CHECK_PTR4(beta);
    CHECK_PTR4(o_out);
    launch_gdn_step(n_heads, dk, dv, state, q, k, v, alpha, beta, o_out, (hipStream_t)stream);
    return hip_status(fn);
}

static int check_attn(const char* fn, int n_q, int n_kv, int d, int T)
{
    if (n_kv < 1 || n_q < n_kv || n_q % n_kv) return fail(MOE_EINVAL, "%s: n_q=%d must be a multiple of n_kv=%d", fn, n_q, n_kv);
    if (n_q / n_kv > attn_max_per())
        return fail(MOE_EUNSUPPORTED, "%s: %d query heads per KV head (at most %d)", fn, n_q / n_kv, attn_max_per());
    if (n_kv > 65535 || n_q > 65536) return fail(MOE_EUNSUPPORTED, "%s: n_q=%d n_kv=%d", fn, n_q, n_kv);
    if (d != 64 && d != 128 && d != 256) return fail(MOE_EUNSUPPORTED, "%s: d=%d (must be 64, 128 or 256)", fn, d);
    if (T < 1 || T > (1 << 22)) return fail(MOE_EINVAL, "%s: T=%d", fn, T);
    return MOE_OK;
}

size_t moe_attn_workspace_bytes(int n_q, int n_kv, int d, int T)
{
    if (check_attn("moe_attn_workspace_bytes", n_q, n_kv, d, T)) return 0;
    return attn_workspace_bytes(n_q, n_kv, d, T);
}

int moe_attn_decode(int n_q, int n_kv, int d, int T, const float* q, const uint16_t* K, const uint16_t* V,
                    float* o_out, void* ws, size_t ws_bytes, void* stream)
{
    const char* fn = "moe_attn_decode";
    int rc = check_attn(fn, n_q, n_kv, d, T);
    if (rc) return rc;
    CHECK_PTR(q);
    CHECK_PTR(K);
    CHECK_PTR(V);
    CHECK_PTR4(o_out);
    CHECK_PTR(ws);
    const size_t need = attn_workspace_bytes(n_q, n_kv, d, T);
    if (ws_bytes < need) return fail(MOE_EINVAL, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
    launch_attn_decode(n_q, n_kv, d, T, q, K, V, (float*)ws, o_out, (hipStream_t)stream);
    return hip_status(fn);
}

int moe_dequant_expert(int bits, int H, int I, int group, const void* record, float* W_out, void* stream)
{
    const char* fn = "moe_dequant_expert";
    int rc = check_shape(fn, bits, H, I, group);
    if (rc) return rc;
    CHECK_PTR(record);
    CHECK_PTR(W_out);
    launch_dequant(make_layout(bits, H, I, group), record, W_out, (hipStream_t)stream);
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

// The batched (grouped) path of a call: the shapes allow it (the workspace always has
// room for it then) and, when range flags are given, the grouping has GEMV groups to
// move the flagged experts to.  It has them for 4-bit layers with rows of at most 64
// groups (gemv_tokens > 1); a 2-bit or wider layer given flags takes the per-token path.
static bool flags_groupable(const Layout& L, const int32_t* flags) { return !flags || gemv_tokens(L) > 1; }
static bool use_grouped(const Work& W, const moe_layer_desc& d)
{
    return W.grouped && flags_groupable(make_layout(d.bits, d.H, d.I, d.group), d.expert_flags);
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
    const Layout L = make_layout(desc->bits, desc->H, desc->I, desc->group);
    if (use_grouped(W, *desc)) {
        launch_group(idx, B, desc->K, desc->E, gemv_tokens(L), desc->expert_flags, W.gw.g, s);
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

int moe_expert_ffn_q3(const moe_layer_desc* desc, const float* x, int B, const int32_t* idx, const float* w,
                      float* y_out, void* ws, size_t ws_bytes, void* stream)
{
    return expert_ffn("moe_expert_ffn_q3", 3, desc, x, B, idx, w, y_out, ws, ws_bytes, stream);
}

// norm_eps >= 0 (per-token path only): x is the previous layer's output, renormalized
// by the router kernel on the fly; grouped: the call takes the batched path (use_grouped)
static int layer_impl(const char* fn, const moe_layer_desc* d, const float* x, int B, float* y_out,
                      int32_t* idx_out, float* w_out, const Work& W, bool grouped, hipStream_t s,
                      float norm_eps = -1.f)
{
    int32_t* idx = idx_out ? idx_out : W.idx;
    float* w = w_out ? w_out : W.w;
    const Layout L = make_layout(d->bits, d->H, d->I, d->group);
    if (grouped) {
        const TokenPrep P{x, d->H, W.gw.xh, W.gw.xsum, W.gw.xscale, gemv_tokens(L) > 1 ? W.xq : nullptr, W.xst};
        launch_route_batched(x, B, d->w_router, d->logit_bias, d->H, d->E, d->K, d->renormalize ? 1 : 0,
                             W.gw.partial, idx, w, P, s, g_timing[KID_ROUTER]);
        launch_group(idx, B, d->K, d->E, gemv_tokens(L), d->expert_flags, W.gw.g, s);
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
    return layer_impl(fn, desc, x, B, y_out, idx_out, w_out, W, use_grouped(W, *desc),
                      (hipStream_t)stream);
}

int moe_grouped_launch_info(const moe_layer_desc* desc, int B, int32_t* info_out)
{
    const char* fn = "moe_grouped_launch_info";
    int rc = check_desc(fn, desc, B);
    if (rc) return rc;
    if (!info_out) return fail(MOE_EINVAL, "%s: info_out is NULL", fn);
    const Layout L = make_layout(desc->bits, desc->H, desc->I, desc->group);
    const bool grouped = grouped_supported(L, B, desc->K) && flags_groupable(L, desc->expert_flags);
    const GroupedBlocks nb = grouped_blocks();
    info_out[0] = grouped ? 1 : 0;
    info_out[1] = desc->bits == 2 ? nb.gateup2 : (desc->bits == 3 ? nb.gateup3 : nb.gateup);
    info_out[2] = grouped_tiles(L, 0);
    info_out[3] = grouped_gateup_chunks();
    info_out[4] = desc->bits == 2 ? nb.down2 : (desc->bits == 3 ? nb.down3 : nb.down);
    info_out[5] = grouped_tiles(L, 1);
    info_out[6] = gemv_tokens(L);
    info_out[7] = grouped_group_tokens();
    return ok();
}

int moe_layer_decode_noalloc(const moe_layer_desc* desc, const float* x, int B, float* y_out, int32_t* idx_out,
                             float* w_out, void* stream)
{
    const char* fn = "moe_layer_decode_noalloc";
    int rc = check_desc(fn, desc, B);
    if (rc) return rc;
    CHECK_PTR(desc->w_router);
    CHECK_OPT_PTR4(desc->logit_bias);
    CHECK_PTR(x);
    CHECK_PTR(y_out);
    CHECK_OPT_PTR4(idx_out);
    CHECK_OPT_PTR4(w_out);
    // the batched path when its workspace fits the scratch, else the per-token kernels
    bool allow_grouped = true;
    Work need = carve(nullptr, desc->bits, B, desc->H, desc->I, desc->E, desc->K);
    if (need.bytes > (size_t)MOE_NOALLOC_SCRATCH_BYTES) {
        allow_grouped = false;
        need = carve(nullptr, desc->bits, B, desc->H, desc->I, desc->E, desc->K, false);
    }
    if (need.bytes > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MOE_EUNSUPPORTED, "%s: B=%d needs %zu bytes of scratch, more than the %d this entry point holds "
                    "per GPU (use moe_layer_decode with a workspace)", fn, B, need.bytes, MOE_NOALLOC_SCRATCH_BYTES);
    void* ws = scratch_ptr(fn, rc);
    if (!ws) return rc;
    const Work W = carve(ws, desc->bits, B, desc->H, desc->I, desc->E, desc->K, allow_grouped);
    return layer_impl(fn, desc, x, B, y_out, idx_out, w_out, W, use_grouped(W, *desc),
                      (hipStream_t)stream);
}

size_t moe_cache_state_bytes(int E, int slots)
{
    if (E < 1 || E > MOE_MAX_E || slots < 1 || slots > MOE_MAX_CACHE_SLOTS) return 0;
    return cache_state_bytes(E, slots);
}

// Workspace of a cached decode: the layer's workspace carved for max(E, slots)
// experts (the router works on E ids, the expert FFNs on slot ids), then the slot
// ids of the selection and the copy plan.
static size_t cached_extra_bytes(int B, int K, int E, int slots)
{
    return up256((size_t)B * K * 4) + up256(4 * (1 + 2 * (size_t)std::min(E, B * K))) + up256(4 * ((size_t)slots + 1));
}

size_t moe_cache_workspace_bytes(const moe_layer_desc* desc, int slots, int B)
{
    if (!desc || check_shape("moe_cache_workspace_bytes", desc->bits, desc->H, desc->I, desc->group) ||
        check_routing("moe_cache_workspace_bytes", B, desc->E, desc->K) || slots < 1 || slots > MOE_MAX_CACHE_SLOTS)
        return 0;
    const int Eb = std::max(desc->E, slots);
    return carve(nullptr, desc->bits, B, desc->H, desc->I, Eb, desc->K).bytes +
           cached_extra_bytes(B, desc->K, desc->E, slots);
}

static int check_cache(const char* fn, const moe_layer_desc* d, const moe_expert_cache* c)
{
    if (!c) return fail(MOE_EINVAL, "%s: cache is NULL", fn);
    if (c->slots < 1 || c->slots > MOE_MAX_CACHE_SLOTS)
        return fail(MOE_EINVAL, "%s: cache->slots=%d (must be in [1, %d])", fn, c->slots, MOE_MAX_CACHE_SLOTS);
    if (!c->slab || misaligned(c->slab)) return fail(MOE_EINVAL, "%s: cache->slab is NULL or not 16-byte aligned", fn);
    if (!c->state || misaligned(c->state))
        return fail(MOE_EINVAL, "%s: cache->state is NULL or not 16-byte aligned", fn);
    return MOE_OK;
}

int moe_cache_init(const moe_layer_desc* desc, const moe_expert_cache* cache, void* stream)
{
    const char* fn = "moe_cache_init";
    int rc = check_desc(fn, desc, 1);
    if (rc) return rc;
    rc = check_cache(fn, desc, cache);
    if (rc) return rc;
    const void* src = backing_device_ptr(desc->experts);
    if (!src) return fail(MOE_EINVAL, "%s: desc->experts is neither device memory nor pinned host memory", fn);
    const Layout L = make_layout(desc->bits, desc->H, desc->I, desc->group);
    hipStream_t s = (hipStream_t)stream;
    launch_cache_reset(cache->state, desc->E, cache->slots, s);
    // the shared expert (record E of the store) has a slot of its own, after the routed ones
    const hipError_t e = hipMemcpyAsync((char*)cache->slab + (size_t)cache->slots * L.record,
                                        (const char*)desc->experts + (size_t)desc->E * L.record, L.record,
                                        hipMemcpyDefault, s);
    if (e != hipSuccess) return fail(MOE_EHIP, "%s: copy of the shared expert: %s", fn, hipGetErrorString(e));
    return hip_status(fn);
}

int moe_layer_decode_cached(const moe_layer_desc* desc, const moe_expert_cache* cache, const float* x, int B,
                            float* y_out, int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes, void* stream)
{
    const char* fn = "moe_layer_decode_cached";
    int rc = check_desc(fn, desc, B);
    if (rc) return rc;
    rc = check_cache(fn, desc, cache);
    if (rc) return rc;
    CHECK_PTR(desc->w_router);
    CHECK_OPT_PTR4(desc->logit_bias);
    CHECK_PTR(x);
    CHECK_PTR(y_out);
    CHECK_OPT_PTR4(idx_out);
    CHECK_OPT_PTR4(w_out);
    CHECK_PTR(ws);
    const int E = desc->E, K = desc->K, S = cache->slots;
    if (S < std::min(E, B * K))
        return fail(MOE_EINVAL, "%s: %d slots cannot hold the up to %d distinct experts of %d tokens x K=%d", fn, S,
                    std::min(E, B * K), B, K);
    const void* src = backing_device_ptr(desc->experts);
    if (!src) return fail(MOE_EINVAL, "%s: desc->experts is neither device memory nor pinned host memory", fn);
    const int Eb = std::max(E, S);
    const Work W = carve(ws, desc->bits, B, desc->H, desc->I, Eb, K);
    const size_t need = W.bytes + cached_extra_bytes(B, K, E, S);
    if (ws_bytes < need) return fail(MOE_EINVAL, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
    int32_t* idx_slot = (int32_t*)((char*)ws + W.bytes);
    int32_t* plan = (int32_t*)((char*)ws + W.bytes + up256((size_t)B * K * 4));
    int32_t* slot_flags = desc->expert_flags ? (int32_t*)((char*)plan + up256(4 * (1 + 2 * (size_t)std::min(E, B * K))))
                                             : nullptr;
    int32_t* idx = idx_out ? idx_out : W.idx;
    float* w = w_out ? w_out : W.w;
    const Layout L = make_layout(desc->bits, desc->H, desc->I, desc->group);
    hipStream_t s = (hipStream_t)stream;
    const int renorm = desc->renormalize ? 1 : 0;
    const bool grouped = use_grouped(W, *desc);
    // 1. route on the E expert ids
    if (grouped) {
        const TokenPrep P{x, desc->H, W.gw.xh, W.gw.xsum, W.gw.xscale, gemv_tokens(L) > 1 ? W.xq : nullptr, W.xst};
        launch_route_batched(x, B, desc->w_router, desc->logit_bias, desc->H, E, K, renorm, W.gw.partial, idx, w, P,
                             s, g_timing[KID_ROUTER]);
    } else {
        launch_router(desc->bits, x, B, desc->w_router, desc->logit_bias, desc->H, E, W.logits, W.xq, W.xst, s,
                      g_timing[KID_ROUTER]);
        if (B > CP_ROUTE_MAX_B) launch_topk(W.logits, B, E, K, renorm, idx, w, s);
    }
    // 2. map the selection onto slots (small per-token batches select there too) and
    //    bring in the missing records
    const bool plan_routes = !grouped && B <= CP_ROUTE_MAX_B;
    launch_cache_plan(idx, B * K, E, S, cache->state, idx_slot, plan, L.record, desc->expert_flags, slot_flags,
                      plan_routes ? W.logits : nullptr, K, renorm, w, s);
    // the single-token kernels fill the missed records inside their gate/up launch;
    // otherwise a copy launch brings them in first
    const int cap = std::min(E, B * K);
    const bool fill = !grouped && ffn_fills_cache(L, K, S, cap);
    if (!fill) launch_cache_copy(plan, cap, src, cache->slab, L.record, s);
    // 3. the expert FFNs on the cache, by slot id (the shared expert at slot S)
    if (grouped) {
        launch_group(idx_slot, B, K, S, gemv_tokens(L), slot_flags, W.gw.g, s);
        launch_ffn_grouped(L, cache->slab, W.gw, x, w, desc->shared_weight, B, K, S, W.xq, W.xst, true, y_out, s,
                           g_timing[KID_GATEUP], g_timing[KID_DOWN]);
    } else {
        launch_ffn(L, cache->slab, W.xq, W.xst, nullptr, 0, idx_slot, w, B, K, S, desc->shared_weight, W.hq, y_out,
                   s, g_timing[KID_GATEUP], g_timing[KID_DOWN], fill ? plan : nullptr, src, cap);
    }
    return hip_status(fn);
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
    launch_group(idx, B, K, E, 1, nullptr, O, (hipStream_t)stream);
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
        // the workspace depends on H, I, E, K and B only, so the code width and the group
        // size may differ between layers
        if (a.H != z.H || a.I != z.I || a.K != z.K || a.E != z.E)
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
    bool grouped = W.grouped;  // one path for the whole stack
    for (int l = 0; l < n_layers; ++l) grouped = grouped && use_grouped(W, layers[l]);
    for (int l = 0; l < n_layers; ++l) {
        const bool last = (l == n_layers - 1);
        float* yl = last ? y_out : ((grouped || !(l & 1)) ? ybuf : xbuf);
        int32_t* il = idx_out ? idx_out + (size_t)l * B * d0.K : nullptr;
        float* wl = w_out ? w_out + (size_t)l * B * d0.K : nullptr;
        int rc = layer_impl(fn, &layers[l], xl, B, yl, il, wl, W, grouped, s, norm);
        if (rc) return rc;
        if (!last) {
            if (grouped) {
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
