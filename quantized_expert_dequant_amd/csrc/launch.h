// launch.h - host-side launchers of the gfx950 kernels (kernels.hip, grouped.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace moe {

// Optional start/stop events recorded around one kernel launch (hipExtLaunchKernelGGL).
struct Timing {
    hipEvent_t start = nullptr, stop = nullptr;
};

enum KernelId { KID_ROUTER = 1, KID_GATEUP = 2, KID_DOWN = 3, KID_COUNT = 4 };

void launch_pack(const Layout& L, int n, const uint8_t* gate, const uint8_t* up, const uint8_t* down,
                 const uint16_t* scales, const uint16_t* biases, void* slab, int first, hipStream_t s);
void launch_dequant(const Layout& L, const void* rec, float* W, hipStream_t s);
void launch_prep(int bits, const float* v, int n_vec, int len, uint4* q, float4* st, hipStream_t s);
// norm_eps >= 0: x is the previous layer's output, renormalized on the fly (as launch_rmsnorm)
void launch_router(int bits, const float* x, int B, const float* W, const float* bias, int H, int E, double* logits,
                   uint4* xq, float4* xst, hipStream_t s, Timing t = Timing(), float norm_eps = -1.f);
void launch_topk(const double* logits, int B, int E, int K, int renorm, int32_t* idx, float* w, hipStream_t s);
void launch_ffn(const Layout& L, const void* slab, const uint4* xq, const float4* xst, const double* logits,
                int renorm, int32_t* idx, float* w, int B, int K, int E, float shared_w, void* hq, float* y,
                hipStream_t s, Timing t_gateup = Timing(), Timing t_down = Timing(),
                const int32_t* fill_plan = nullptr, const void* fill_src = nullptr, int fill_cap = 0);
// fill_plan (a cache plan of at most fill_cap entries) fills the missed records inside the
// gate/up launch, from the store at fill_src; only where ffn_fills_cache says so
bool ffn_fills_cache(const Layout& L, int K, int E, int cap);
void launch_rmsnorm(const float* y, int B, int H, float eps, float* x, hipStream_t s);
// the attention half of a decode step (attention.hip)
void launch_gdn_step(int n_heads, int dk, int dv, float* S, const float* q, const float* k, const float* v,
                     const float* alpha, const float* beta, float* o, hipStream_t s);
size_t attn_workspace_bytes(int n_q, int n_kv, int d, int T);
int attn_max_per();
void launch_attn_decode(int n_q, int n_kv, int d, int T, const float* q, const uint16_t* K, const uint16_t* V,
                        float* part, float* o, hipStream_t s);
// canonical 4-bit experts -> canonical 2-bit experts (requant.hip)
void launch_requant_4to2(int H, int I, int group, int n, const uint8_t* gate4, const uint8_t* up4,
                         const uint8_t* down4, const uint16_t* s4, const uint16_t* b4, uint8_t* gate2, uint8_t* up2,
                         uint8_t* down2, uint16_t* s2, uint16_t* b2, hipStream_t s);

}  // namespace moe
