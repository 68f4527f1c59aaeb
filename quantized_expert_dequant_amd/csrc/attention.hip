// attention.hip - the attention half of a decode step on gfx950: one step of the
// gated delta rule (GatedDeltaNet linear attention) and grouped-query decode
// attention over a bf16 KV cache.
//
// Pages (titles as published):
//   [LLMAPIS] llmapis.com, "Flash-MoE：把 397B MoE 真正跑进消费级笔记本，意味着
//             '大模型本地化'开始从演示走向系统工程"
//   [MFFB]    f.mffb.com.cn, Flash-MoE article ("HN上281票 ... 8200行纯C代码 ...")
//
// The pages name the model's attention layers, 45 GatedDeltaNet (linear attention)
// and 15 full-attention layers, and say the linear attention ran on the CPU with
// BLAS ([LLMAPIS] section 深度分析; [MFFB] section 有效的优化); they give no
// formulas.  Readings:
//   gated delta rule, per head h with state S_h (dv x dk, fp32, row-major):
//     S_h <- alpha_h S_h (I - beta_h k_h k_h^T) + beta_h v_h k_h^T,  o_h = S_h q_h
//     (the rule as published by Yang, Kautz and Hatamizadeh, 2024)
//   decode attention: query head h reads KV head h / (n_q / n_kv) over T cached
//     positions, o_h = sum_t softmax_t(q_h . K[t] / sqrt(d)) V[t], K and V bf16.
// Both are bandwidth-bound at one token: the gated delta step reads and writes
// the state once (8 dk dv bytes per head), attention reads the cache once
// (4 d T bytes per KV head).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "launch.h"

namespace moe {

// ----------------------------------------------------------------------------
// Gated delta rule.  One wave owns GD_ROWS consecutive rows of one head's state;
// lane l holds columns l + 64 j (j < NC = dk / 64) of each row.  It loads its rows,
// reduces u = S k per row, writes S' = alpha (S - beta u k^T) + beta v k^T in place
// and reduces o = S' q from the registers: the state is read once and written once.
// ----------------------------------------------------------------------------
constexpr int GD_ROWS = 4;
constexpr int GD_WAVES = 4;

template <int NC>
__global__ __launch_bounds__(64 * GD_WAVES) void k_gdn_step(int n_heads, int dv, float* __restrict__ S,
                                                            const float* __restrict__ q, const float* __restrict__ k,
                                                            const float* __restrict__ v,
                                                            const float* __restrict__ alpha,
                                                            const float* __restrict__ beta, float* __restrict__ o)
{
    constexpr int DK = 64 * NC;
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * GD_WAVES + (threadIdx.x >> 6);
    const int wpr = (dv + GD_ROWS - 1) / GD_ROWS;  // waves per head
    const int h = w / wpr, r0 = (w - h * wpr) * GD_ROWS;
    if (h >= n_heads) return;
    float kk[NC], qq[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        kk[j] = k[(long long)h * DK + lane + 64 * j];
        qq[j] = q[(long long)h * DK + lane + 64 * j];
    }
    const float a = alpha[h], b = beta[h];
    float* Sh = S + (long long)h * dv * DK;
    float s[GD_ROWS][NC];
#pragma unroll
    for (int i = 0; i < GD_ROWS; ++i) {
        const int r = min(r0 + i, dv - 1);
#pragma unroll
        for (int j = 0; j < NC; ++j) s[i][j] = Sh[(long long)r * DK + lane + 64 * j];
    }
#pragma unroll
    for (int i = 0; i < GD_ROWS; ++i) {
        const int r = r0 + i;
        float u = 0.f;
#pragma unroll
        for (int j = 0; j < NC; ++j) u = fmaf(s[i][j], kk[j], u);
        u = wave_sum(u);
        const float vr = v[(long long)h * dv + min(r, dv - 1)];
        const float bu = b * u, bv = b * vr;
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const float m = fmaf(-bu, kk[j], s[i][j]);   // S - beta (S k) k^T
            const float n = fmaf(a, m, bv * kk[j]);       // alpha (...) + beta v k^T
            s[i][j] = n;
            acc = fmaf(n, qq[j], acc);
        }
        acc = wave_sum(acc);
        if (r < dv) {
#pragma unroll
            for (int j = 0; j < NC; ++j) Sh[(long long)r * DK + lane + 64 * j] = s[i][j];
            if (lane == 0) o[(long long)h * dv + r] = acc;
        }
    }
}

void launch_gdn_step(int n_heads, int dk, int dv, float* S, const float* q, const float* k, const float* v,
                     const float* alpha, const float* beta, float* o, hipStream_t s)
{
    const long long waves = (long long)n_heads * ((dv + GD_ROWS - 1) / GD_ROWS);
    const dim3 grid((unsigned)((waves + GD_WAVES - 1) / GD_WAVES));
    switch (dk) {
    case 64: hipLaunchKernelGGL(k_gdn_step<1>, grid, dim3(64 * GD_WAVES), 0, s, n_heads, dv, S, q, k, v, alpha, beta, o); break;
    case 128: hipLaunchKernelGGL(k_gdn_step<2>, grid, dim3(64 * GD_WAVES), 0, s, n_heads, dv, S, q, k, v, alpha, beta, o); break;
    default: hipLaunchKernelGGL(k_gdn_step<4>, grid, dim3(64 * GD_WAVES), 0, s, n_heads, dv, S, q, k, v, alpha, beta, o); break;
    }
}

// ----------------------------------------------------------------------------
// Decode attention, split over the cached positions (64 per slice).  One wave per
// (KV head g, slice): lane t first scores position t of the slice against every
// query head of the group (the K row is read once for all of them), the wave
// takes each head's slice maximum and exp-weights, then lane c accumulates
// columns c + 64 j of sum_t p[h][t] V[t] for every head from the V rows (read once,
// coalesced).  Each (head, slice) leaves (max, sum of weights, weighted V); the
// combine kernel merges the slices in slice order.
// ----------------------------------------------------------------------------
constexpr int AT_SLICE = 64;
constexpr int AT_MAX_PER = 16;  // query heads per KV head

__device__ inline float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <int NC>
__global__ __launch_bounds__(64) void k_attn_partial(int n_q, int n_kv, int T, const float* __restrict__ q,
                                                     const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                                     float* __restrict__ part)
{
    constexpr int D = 64 * NC;
    __shared__ float qs[AT_MAX_PER][D];
    __shared__ float ps[AT_MAX_PER][AT_SLICE];
    const int g = blockIdx.y, sl = blockIdx.x, lane = threadIdx.x;
    const int per = n_q / n_kv, nsl = gridDim.x;
    const int t0 = sl * AT_SLICE;
    for (int i = lane; i < per * D; i += 64) qs[i / D][i % D] = q[(long long)(g * per + i / D) * D + i % D];
    __syncthreads();
    // scores: lane = position
    const int t = min(t0 + lane, T - 1);
    const bool tv = t0 + lane < T;
    const uint16_t* Kt = K + ((long long)g * T + t) * D;
    float sc[AT_MAX_PER];
#pragma unroll
    for (int h = 0; h < AT_MAX_PER; ++h) sc[h] = 0.f;
#pragma unroll
    for (int c0 = 0; c0 < D; c0 += 8) {
        const uint4 raw = *reinterpret_cast<const uint4*>(Kt + c0);
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float k0 = bf16_lo(w4[e]), k1 = bf16_hi(w4[e]);
#pragma unroll
            for (int h = 0; h < AT_MAX_PER; ++h) {
                if (h < per) sc[h] = fmaf(k1, qs[h][c0 + 2 * e + 1], fmaf(k0, qs[h][c0 + 2 * e], sc[h]));
            }
        }
    }
    const float scale = rsqrtf((float)D);
    float mh[AT_MAX_PER], lh[AT_MAX_PER];
#pragma unroll
    for (int h = 0; h < AT_MAX_PER; ++h) {
        if (h >= per) continue;
        const float s = tv ? sc[h] * scale : -INFINITY;
        const float m = wave_max(s);
        const float p = tv ? __expf(s - m) : 0.f;
        lh[h] = wave_sum(p);
        mh[h] = m;
        ps[h][lane] = p;
    }
    __syncthreads();
    // weighted values: lane = column
    float acc[AT_MAX_PER][NC];
#pragma unroll
    for (int h = 0; h < AT_MAX_PER; ++h)
#pragma unroll
        for (int j = 0; j < NC; ++j) acc[h][j] = 0.f;
    const int nt = min(AT_SLICE, T - t0);
    for (int i = 0; i < nt; ++i) {
        const uint16_t* Vt = V + ((long long)g * T + t0 + i) * D;
        float vv[NC];
#pragma unroll
        for (int j = 0; j < NC; ++j) vv[j] = bf16f(Vt[lane + 64 * j]);
#pragma unroll
        for (int h = 0; h < AT_MAX_PER; ++h) {
            if (h >= per) continue;
            const float p = ps[h][i];
#pragma unroll
            for (int j = 0; j < NC; ++j) acc[h][j] = fmaf(p, vv[j], acc[h][j]);
        }
    }
    // part[(head, slice)] = (max, sum, acc[D])
#pragma unroll
    for (int h = 0; h < AT_MAX_PER; ++h) {
        if (h >= per) continue;
        float* pp = part + ((long long)(g * per + h) * nsl + sl) * (D + 2);
        if (lane == 0) {
            pp[0] = mh[h];
            pp[1] = lh[h];
        }
#pragma unroll
        for (int j = 0; j < NC; ++j) pp[2 + lane + 64 * j] = acc[h][j];
    }
}

template <int NC>
__global__ __launch_bounds__(64) void k_attn_combine(int nsl, const float* __restrict__ part, float* __restrict__ o)
{
    constexpr int D = 64 * NC;
    const int h = blockIdx.x, lane = threadIdx.x;
    const float* ph = part + (long long)h * nsl * (D + 2);
    float M = -INFINITY;
    for (int s = 0; s < nsl; ++s) M = fmaxf(M, ph[(long long)s * (D + 2)]);
    float L = 0.f, acc[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) acc[j] = 0.f;
    for (int s = 0; s < nsl; ++s) {
        const float* p = ph + (long long)s * (D + 2);
        const float f = __expf(p[0] - M);
        L = fmaf(p[1], f, L);
#pragma unroll
        for (int j = 0; j < NC; ++j) acc[j] = fmaf(p[2 + lane + 64 * j], f, acc[j]);
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int j = 0; j < NC; ++j) o[(long long)h * D + lane + 64 * j] = acc[j] * inv;
}

size_t attn_workspace_bytes(int n_q, int d, int T)
{
    const long long nsl = (T + AT_SLICE - 1) / AT_SLICE;
    return (size_t)n_q * nsl * (d + 2) * 4;
}

int attn_max_per() { return AT_MAX_PER; }

void launch_attn_decode(int n_q, int n_kv, int d, int T, const float* q, const uint16_t* K, const uint16_t* V,
                        float* part, float* o, hipStream_t s)
{
    const int nsl = (T + AT_SLICE - 1) / AT_SLICE;
    const dim3 grid(nsl, n_kv);
    switch (d) {
    case 64:
        hipLaunchKernelGGL(k_attn_partial<1>, grid, dim3(64), 0, s, n_q, n_kv, T, q, K, V, part);
        hipLaunchKernelGGL(k_attn_combine<1>, dim3(n_q), dim3(64), 0, s, nsl, part, o);
        break;
    case 128:
        hipLaunchKernelGGL(k_attn_partial<2>, grid, dim3(64), 0, s, n_q, n_kv, T, q, K, V, part);
        hipLaunchKernelGGL(k_attn_combine<2>, dim3(n_q), dim3(64), 0, s, nsl, part, o);
        break;
    default:
        hipLaunchKernelGGL(k_attn_partial<4>, grid, dim3(64), 0, s, n_q, n_kv, T, q, K, V, part);
        hipLaunchKernelGGL(k_attn_combine<4>, dim3(n_q), dim3(64), 0, s, nsl, part, o);
        break;
    }
}

}  // namespace moe
