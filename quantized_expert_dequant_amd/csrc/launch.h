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
void launch_router(const float* x, int B, const float* W, const float* bias, int H, int E, int K, int renorm,
                   double* logits, unsigned* counter, int32_t* idx, float* w, hipStream_t s,
                   Timing t = Timing());
void launch_gateup(const Layout& L, const void* slab, const uint4* xq, const float4* xst, const int32_t* idx,
                   int B, int K, int E, float* h, hipStream_t s, Timing t = Timing());
void launch_down(const Layout& L, const void* slab, const uint4* hq, const float4* hst, const int32_t* idx,
                 const float* w, int B, int K, int E, float shared_w, float* y, hipStream_t s,
                 Timing t = Timing());
void launch_rmsnorm(const float* y, int B, int H, float eps, float* x, hipStream_t s);

}  // namespace moe
