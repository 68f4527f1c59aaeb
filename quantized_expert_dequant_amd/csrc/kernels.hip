// kernels.hip - gfx950 kernels of the quantized MoE decode layer.
//
// Pages (titles as published):
//   [LLMAPIS] llmapis.com, "Flash-MoE：把 397B MoE 真正跑进消费级笔记本，意味着
//             '大模型本地化'开始从演示走向系统工程"
//   [CLAUDAY] clauday.com, "Flash-MoE: Running a 397B Parameter Model on a MacBook
//             with Pure C and Metal"
//
// Per-token path ([LLMAPIS] section 深度分析: route, read, dequantize, compute,
// combine):
//   k_router  logits (fp32 products accumulated in fp64); also preps the token:
//             integer digit planes (4- and 2-bit) or fp16 pairs (3-bit) + per-group
//             stats, the operand of the folded dequant
//             (scale*x and bias*x per group, the FMA rearrangement described in
//             [LLMAPIS] section 深度分析, applied per 64-column unit)
//   k_gateup  softmax / top-K per wave, then the fused gate/up dequant-GEMV +
//             SiLU*mul over the K routed + shared experts
//   k_down    down dequant-GEMV + router-weighted combine in one pass (no atomics)
//   k_prep    the token prep alone, for callers that bring their own routing
//   k_topk    softmax / top-K alone, for the router entry point
#include <hip/hip_ext.h>

#include "common.h"
#include "topk.h"
#include "launch.h"

namespace moe {

__device__ inline uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
// the 8 bytes of a 3-bit unit's high bits, in .x and .y
__device__ inline uint4 ld8(const uint8_t* p)
{
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    return make_uint4(v.x, v.y, 0u, 0u);
}

// sum_t acc_t / t of one row unit (64 columns) against the token operand xp:
// 4-bit c0, c1 = the unit's two chunks; 3-bit c0 = its low-bit chunk, c1.xy its
// high bits; 2-bit c0 = its chunk
template <int BITS>
__device__ inline float group_dot(const Masks& M, uint4 c0, uint4 c1, const uint4* xp)
{
    if constexpr (BITS == 4) return group_dot_q4(M, c0, c1, xp);
    else if constexpr (BITS == 3) return group_dot_q3(M, c0, make_uint2(c1.x, c1.y), xp);
    else return group_dot_q2(M, c0, xp);
}

// ----------------------------------------------------------------------------
// pack: canonical -> packed record
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pack(Layout L, const uint8_t* __restrict__ gate,
                                              const uint8_t* __restrict__ up,
                                              const uint8_t* __restrict__ down,
                                              const uint16_t* __restrict__ scales,
                                              const uint16_t* __restrict__ biases,
                                              uint8_t* __restrict__ slab, int first)
{
    const int j = blockIdx.y;  // expert within the batch
    const long long cb = (long long)L.I * L.hb;  // canonical code bytes of one gate/up matrix
    const long long ng = 2LL * L.I * L.Sh + (long long)L.H * L.Si;  // groups (scales) of one expert
    const int cpg = L.bits / 2;  // 16-byte chunks per 64-column unit
    const long long n_gu_chunks = 2LL * L.I * (L.hb / 16);
    const long long n_gu_sb = (long long)L.I * L.Sh;
    const long long n_d_chunks = (long long)L.H * (L.ib / 16);
    const long long n_d_sb = (long long)L.H * L.Si;
    const long long total = n_gu_chunks + n_gu_sb + n_d_chunks + n_d_sb;
    uint8_t* rec = slab + (long long)(first + j) * L.record;
    const uint16_t* sc = scales + j * ng;
    const uint16_t* bi = biases + j * ng;
    for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (long long)gridDim.x * blockDim.x) {
        if (t < n_gu_chunks) {
            const long long per_row = L.hb / 16;  // chunks per matrix row
            const long long r = t / (2 * per_row);
            const long long rem = t - r * 2 * per_row;
            const int m = (int)(rem / per_row);  // 0 gate, 1 up
            const int pos = (int)(rem - m * per_row);
            const int half = pos / L.Gh, g = pos - half * L.Gh;
            const uint8_t* src = (m == 0 ? gate : up) + j * cb + r * L.hb + (long long)(g * cpg + half) * 16;
            *reinterpret_cast<uint4*>(rec + r * 2 * L.hb + m * L.hb + (long long)pos * 16) =
                *reinterpret_cast<const uint4*>(src);
        } else if (t < n_gu_chunks + n_gu_sb) {
            const long long i = t - n_gu_chunks;  // r * Sh + group
            const long long nu = (long long)L.I * L.Sh;
            ushort4 v = make_ushort4(sc[i], bi[i], sc[nu + i], bi[nu + i]);
            *reinterpret_cast<ushort4*>(rec + L.off_gu_sb + i * 8) = v;
        } else if (t < n_gu_chunks + n_gu_sb + n_d_chunks) {
            const long long c = t - n_gu_chunks - n_gu_sb;
            const long long per_row = L.ib / 16;
            const long long r = c / per_row;
            const int pos = (int)(c - r * per_row);
            const int half = pos / L.Gi, g = pos - half * L.Gi;
            const uint8_t* src = down + j * ((long long)L.H * L.ib) + r * L.ib + (long long)(g * cpg + half) * 16;
            *reinterpret_cast<uint4*>(rec + L.off_d_codes + d_chunk_off(L, (int)r, pos)) =
                *reinterpret_cast<const uint4*>(src);
        } else {
            const long long i = t - n_gu_chunks - n_gu_sb - n_d_chunks;  // r * Si + group
            const long long o = 2LL * L.I * L.Sh;
            ushort2 v = make_ushort2(sc[o + i], bi[o + i]);
            *reinterpret_cast<ushort2*>(rec + L.off_d_sb + i * 4) = v;
        }
    }
}

// 3-bit: the 24 canonical bytes of one 64-column unit (a little-endian bit string,
// code c at bits 3c..3c+2) -> the unit's low-bit chunk (2-bit chunk order: code c at
// bits 2(c % 16) of dword c / 16) and its two high-bit dwords (the order group_dot_q3
// reads: dword d's code pairs (c, c + 8), c % 16 = i < 8, at bits (2i + 2, 2i + 18)
// for i < 4 and (2i - 5, 2i + 11) for i >= 4; odd d rotated left by 8 beside d - 1).
__device__ inline void pack_unit3(const uint8_t* __restrict__ src, uint4& lo, uint2& hi)
{
    uint32_t lw[4] = {0u, 0u, 0u, 0u}, S[4] = {0u, 0u, 0u, 0u};
    for (int c = 0; c < 64; ++c) {
        const int bit = 3 * c, by = bit >> 3;
        const uint32_t win = (uint32_t)src[by] | (by + 1 < 24 ? (uint32_t)src[by + 1] << 8 : 0u);
        const uint32_t q = (win >> (bit & 7)) & 7u;
        const int d = c >> 4, r = c & 15, i = r & 7, half = r >> 3;
        lw[d] |= (q & 3u) << (2 * r);
        const int pos = (i < 4 ? 2 * i + 2 : 2 * (i - 4) + 3) + 16 * half;
        S[d] |= (q >> 2) << pos;
    }
    lo = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    hi = make_uint2(S[0] | ((S[1] << 8) | (S[1] >> 24)), S[2] | ((S[3] << 8) | (S[3] >> 24)));
}

// byte offsets in a record of unit g's low-bit chunk and high-bit dwords: gate/up row r
// of matrix m (0 gate, 1 up) is [G_h low chunks | G_h x 8 bytes of high bits]; a down
// row is G_i low chunks then the high bits as chunks G_i + g / 2, through the panel order
__host__ __device__ inline long long q3_gu_lo(const Layout& L, int r, int m, int g)
{
    return (long long)r * 2 * L.hb + m * L.hb + 16LL * g;
}
__host__ __device__ inline long long q3_gu_hi(const Layout& L, int r, int m, int g)
{
    return (long long)r * 2 * L.hb + m * L.hb + 16LL * L.Gh + 8LL * g;
}
__host__ __device__ inline long long q3_d_lo(const Layout& L, int r, int g) { return L.off_d_codes + d_chunk_off(L, r, g); }
__host__ __device__ inline long long q3_d_hi(const Layout& L, int r, int g)
{
    return L.off_d_codes + d_chunk_off(L, r, L.Gi + (g >> 1)) + 8 * (g & 1);
}

__global__ __launch_bounds__(256) void k_pack3(Layout L, const uint8_t* __restrict__ gate,
                                               const uint8_t* __restrict__ up, const uint8_t* __restrict__ down,
                                               const uint16_t* __restrict__ scales,
                                               const uint16_t* __restrict__ biases, uint8_t* __restrict__ slab,
                                               int first)
{
    const int j = blockIdx.y;
    const long long cb = (long long)L.I * L.hb;
    const long long ng = 2LL * L.I * L.Sh + (long long)L.H * L.Si;
    const long long n_gu_units = 2LL * L.I * L.Gh, n_gu_sb = (long long)L.I * L.Sh;
    const long long n_d_units = (long long)L.H * L.Gi, n_d_sb = (long long)L.H * L.Si;
    const long long total = n_gu_units + n_gu_sb + n_d_units + n_d_sb;
    uint8_t* rec = slab + (long long)(first + j) * L.record;
    const uint16_t* sc = scales + j * ng;
    const uint16_t* bi = biases + j * ng;
    for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (long long)gridDim.x * blockDim.x) {
        uint4 lo;
        uint2 hi;
        if (t < n_gu_units) {
            const int r = (int)(t / (2 * L.Gh)), rem = (int)(t - (long long)r * 2 * L.Gh);
            const int m = rem / L.Gh, g = rem - m * L.Gh;
            pack_unit3((m == 0 ? gate : up) + j * cb + (long long)r * L.hb + 24LL * g, lo, hi);
            *reinterpret_cast<uint4*>(rec + q3_gu_lo(L, r, m, g)) = lo;
            *reinterpret_cast<uint2*>(rec + q3_gu_hi(L, r, m, g)) = hi;
        } else if (t < n_gu_units + n_gu_sb) {
            const long long i = t - n_gu_units;  // r * Sh + group
            const long long nu = (long long)L.I * L.Sh;
            *reinterpret_cast<ushort4*>(rec + L.off_gu_sb + i * 8) = make_ushort4(sc[i], bi[i], sc[nu + i], bi[nu + i]);
        } else if (t < n_gu_units + n_gu_sb + n_d_units) {
            const long long u = t - n_gu_units - n_gu_sb;
            const int r = (int)(u / L.Gi), g = (int)(u - (long long)r * L.Gi);
            pack_unit3(down + j * ((long long)L.H * L.ib) + (long long)r * L.ib + 24LL * g, lo, hi);
            *reinterpret_cast<uint4*>(rec + q3_d_lo(L, r, g)) = lo;
            *reinterpret_cast<uint2*>(rec + q3_d_hi(L, r, g)) = hi;
        } else {
            const long long i = t - n_gu_units - n_gu_sb - n_d_units;  // r * Si + group
            const long long o = 2LL * L.I * L.Sh;
            *reinterpret_cast<ushort2*>(rec + L.off_d_sb + i * 4) = make_ushort2(sc[o + i], bi[o + i]);
        }
    }
}

void launch_pack(const Layout& L, int n, const uint8_t* gate, const uint8_t* up, const uint8_t* down,
                 const uint16_t* scales, const uint16_t* biases, void* slab, int first, hipStream_t s)
{
    if (L.bits == 3) {
        const long long total = 2LL * L.I * L.Gh + (long long)L.I * L.Sh + (long long)L.H * L.Gi + (long long)L.H * L.Si;
        long long blocks = (total + 255) / 256;
        if (blocks > 4096) blocks = 4096;
        hipLaunchKernelGGL(k_pack3, dim3((unsigned)blocks, n), dim3(256), 0, s, L, gate, up, down, scales, biases,
                           (uint8_t*)slab, first);
        return;
    }
    const long long total = 2LL * L.I * (L.hb / 16) + (long long)L.I * L.Sh + (long long)L.H * (L.ib / 16) +
                            (long long)L.H * L.Si;
    long long blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_pack, dim3((unsigned)blocks, n), dim3(256), 0, s, L, gate, up, down, scales, biases,
                       (uint8_t*)slab, first);
}

// ----------------------------------------------------------------------------
// dequant of one packed record (layout check)
// ----------------------------------------------------------------------------
// chunk position of column c of a row with G groups, and c's place in the chunk
__device__ inline int packed_pos(int bits, int G, int c, int& k)
{
    const int g = c >> 6, cc = c & 63;
    const int per_chunk = 128 / bits;  // codes per 16-byte chunk
    const int half = cc / per_chunk;
    k = cc - half * per_chunk;
    return half * G + g;
}
__device__ inline int chunk_code(const uint8_t* chunk, int bits, int k)
{
    if (bits == 4) return (chunk[k >> 1] >> ((k & 1) * 4)) & 15;
    return (chunk[k >> 2] >> ((k & 3) * 2)) & 3;
}

// 3-bit code cc (0..63) of a unit from its low-bit chunk and high-bit dwords
__device__ inline int q3_code(const uint8_t* lo, const uint8_t* hi, int cc)
{
    const int d = cc >> 4, r = cc & 15, i = r & 7, half = r >> 3;
    const uint32_t lw = reinterpret_cast<const uint32_t*>(lo)[d];
    uint32_t S = reinterpret_cast<const uint32_t*>(hi)[d >> 1];
    if (d & 1) S = (S >> 8) | (S << 24);
    const int pos = (i < 4 ? 2 * i + 2 : 2 * (i - 4) + 3) + 16 * half;
    return (int)(((lw >> (2 * r)) & 3u) | (((S >> pos) & 1u) << 2));
}

__global__ __launch_bounds__(256) void k_dequant(Layout L, const uint8_t* __restrict__ rec,
                                                 float* __restrict__ W)
{
    const long long n_gu = (long long)L.I * L.H;
    const long long total = 3 * n_gu;
    for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (long long)gridDim.x * blockDim.x) {
        float s, b;
        int q;
        if (t < 2 * n_gu) {
            const int m = (int)(t / n_gu);
            const long long i = t - m * n_gu;
            const int r = (int)(i / L.H), c = (int)(i - (long long)r * L.H);
            if (L.bits == 3) {
                q = q3_code(rec + q3_gu_lo(L, r, m, c >> 6), rec + q3_gu_hi(L, r, m, c >> 6), c & 63);
            } else {
                const uint8_t* row = rec + (long long)r * 2 * L.hb + m * L.hb;
                int k;
                const int P = packed_pos(L.bits, L.Gh, c, k);
                q = chunk_code(row + (long long)P * 16, L.bits, k);
            }
            const uint16_t* sb = reinterpret_cast<const uint16_t*>(rec + L.off_gu_sb + ((long long)r * L.Sh + (c >> (6 + L.gs))) * 8);
            s = __uint_as_float((uint32_t)sb[2 * m] << 16);
            b = __uint_as_float((uint32_t)sb[2 * m + 1] << 16);
        } else {
            const long long i = t - 2 * n_gu;
            const int r = (int)(i / L.I), c = (int)(i - (long long)r * L.I);
            if (L.bits == 3) {
                q = q3_code(rec + q3_d_lo(L, r, c >> 6), rec + q3_d_hi(L, r, c >> 6), c & 63);
            } else {
                int k;
                const int P = packed_pos(L.bits, L.Gi, c, k);
                q = chunk_code(rec + L.off_d_codes + d_chunk_off(L, r, P), L.bits, k);
            }
            const uint16_t* sb = reinterpret_cast<const uint16_t*>(rec + L.off_d_sb + ((long long)r * L.Si + (c >> (6 + L.gs))) * 4);
            s = __uint_as_float((uint32_t)sb[0] << 16);
            b = __uint_as_float((uint32_t)sb[1] << 16);
        }
        W[t] = fmaf(s, (float)q, b);
    }
}

void launch_dequant(const Layout& L, const void* rec, float* W, hipStream_t s)
{
    const long long total = 3LL * L.I * L.H;
    long long blocks = (total + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(k_dequant, dim3((unsigned)blocks), dim3(256), 0, s, L, (const uint8_t*)rec, W);
}

// ----------------------------------------------------------------------------
// prep of the token activations: fp32 [B][H] -> the operand of the code width
// (integer digit planes or fp16 pairs, common.h) + per-group stats.
// One wave per (token, group); shared by the standalone prep kernel and the
// router kernel, which preps the token while it computes the logits.
// ----------------------------------------------------------------------------

// 1 / sqrt(mean(y^2) + eps) of a row of n4 float4, by one wave: lane l sums the
// squares of float4 l, l+64, ... in fp64 in that order, then the wave adds the
// lanes.  The standalone RMS renorm and the router that renormalizes its input
// on the fly both use this, so they produce bit-identical activations.
__device__ inline float row_inv_rms(const float4* __restrict__ y4, int n4, float eps, int lane)
{
    double ss = 0.0;
    for (int c = lane; c < n4; c += 64) {
        const float4 v = y4[c];
        ss = fma((double)v.x, (double)v.x, ss);
        ss = fma((double)v.y, (double)v.y, ss);
        ss = fma((double)v.z, (double)v.z, ss);
        ss = fma((double)v.w, (double)v.w, ss);
    }
    ss = wave_sum(ss);
    return (float)(1.0 / sqrt(ss / (4.0 * n4) + (double)eps));
}

template <int BITS>
__global__ __launch_bounds__(256) void k_prep(const float* __restrict__ v, int n_vec, int G, uint4* __restrict__ q,
                                              float4* __restrict__ st)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int i = blockIdx.x * 4 + wave; i < n_vec * G; i += gridDim.x * 4) {
        const int vec = i / G, g = i - vec * G;
        prep_group<BITS>(v, G, vec, g, lane, q, st);
    }
}

void launch_prep(int bits, const float* v, int n_vec, int len, uint4* q, float4* st, hipStream_t s)
{
    const int G = len / 64;
    int blocks = (n_vec * G + 3) / 4;
    if (blocks > 1024) blocks = 1024;
    if (bits == 4)
        hipLaunchKernelGGL(k_prep<4>, dim3(blocks), dim3(256), 0, s, v, n_vec, G, q, st);
    else if (bits == 3)
        hipLaunchKernelGGL(k_prep<3>, dim3(blocks), dim3(256), 0, s, v, n_vec, G, q, st);
    else
        hipLaunchKernelGGL(k_prep<2>, dim3(blocks), dim3(256), 0, s, v, n_vec, G, q, st);
}

// ----------------------------------------------------------------------------
// routing: logits (fp32 products accumulated in fp64), then softmax / top-K
// ----------------------------------------------------------------------------

// logits[b][e] = W_r[e] . x[b] (+ bias[e]); one wave per expert.  The token's
// dequant operand (digit planes or fp16 pairs, + stats) is prepared by the same launch.
__device__ inline double dot4d(float4 w, float4 x, double acc)
{
    acc = fma((double)w.x, (double)x.x, acc);
    acc = fma((double)w.y, (double)x.y, acc);
    acc = fma((double)w.z, (double)x.z, acc);
    return fma((double)w.w, (double)x.w, acc);
}

// router: waves (experts or prep groups) per block.  A token as given: one, so the
// 512 logit waves of a layer land on every CU instead of on half of them (measured
// at H=4096, E=512: step 18.05 -> 17.47 us; two per block 17.6-17.9).  A token
// renormalized on the fly (stacked layers): four (60-layer step 1088 us, against
// 1126 with one and 1130 with two).
constexpr int RT_WAVES = 1;
constexpr int RT_NORM_WAVES = 4;

template <int BITS>
// Blocks [0, rblocks) compute the logits (one wave per expert); blocks from
// rblocks on prepare the token operand at the same time (one wave per group).
__global__ __launch_bounds__(256) void k_router(const float* __restrict__ x, int B, int prepB,
                                                const float* __restrict__ W, const float* __restrict__ bias, int H,
                                                int E, double* __restrict__ logits, uint4* __restrict__ xq,
                                                float4* __restrict__ xst, float norm_eps, int rblocks)
{
    // norm_eps >= 0: x is the previous layer's output y; the token is renormalized
    // on the fly, x = y / sqrt(mean(y^2) + eps), exactly as k_rmsnorm would
    const bool norm = norm_eps >= 0.f;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rw = (int)(blockDim.x >> 6);  // waves per block
    const int e = blockIdx.x * rw + wave;
    const int n4 = H >> 2;
    const float4* x4 = reinterpret_cast<const float4*>(x);
    if ((int)blockIdx.x >= rblocks) {
        const int Gh = H / 64, nw = ((int)gridDim.x - rblocks) * rw;
        for (int i = ((int)blockIdx.x - rblocks) * rw + wave; i < prepB * Gh; i += nw) {
            const int vec = i / Gh, g = i - vec * Gh;
            const float inv = norm ? row_inv_rms(x4 + (long long)vec * n4, n4, norm_eps, lane) : 1.f;
            prep_group<BITS>(x, Gh, vec, g, lane, xq, xst, inv);
        }
        return;
    }
    if (e < E) {
        const float4* W4 = reinterpret_cast<const float4*>(W) + (long long)e * n4;
        const double bb = bias ? (double)bias[e] : 0.0;
        if (n4 <= 1024) {
            // token 0's activations (cache-resident) first, then the router row (HBM)
            // clamped indices: every load is unconditional (no branch, no serialising wait);
            // columns past H are zeroed after the loads
            float4 xv[16], wv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) xv[i] = x4[min(lane + 64 * i, n4 - 1)];
#pragma unroll
            for (int i = 0; i < 16; ++i) wv[i] = W4[min(lane + 64 * i, n4 - 1)];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (lane + 64 * i >= n4) wv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int b = 0; b < B; ++b) {
                if (b > 0) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) xv[i] = x4[(long long)b * n4 + min(lane + 64 * i, n4 - 1)];
                }
                if (norm) {  // the sum of squares in row_inv_rms's order, from the registers
                    double ss = 0.0;
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (lane + 64 * i < n4) {
                            ss = fma((double)xv[i].x, (double)xv[i].x, ss);
                            ss = fma((double)xv[i].y, (double)xv[i].y, ss);
                            ss = fma((double)xv[i].z, (double)xv[i].z, ss);
                            ss = fma((double)xv[i].w, (double)xv[i].w, ss);
                        }
                    ss = wave_sum(ss);
                    const float inv = (float)(1.0 / sqrt(ss / (4.0 * n4) + (double)norm_eps));
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        xv[i] = make_float4(xv[i].x * inv, xv[i].y * inv, xv[i].z * inv, xv[i].w * inv);
                }
                double acc = 0.0;
#pragma unroll
                for (int i = 0; i < 16; ++i) acc = dot4d(wv[i], xv[i], acc);
                acc = wave_sum(acc);
                if (lane == 0) logits[(long long)b * E + e] = acc + bb;
            }
        } else {
            for (int b = 0; b < B; ++b) {
                const float inv = norm ? row_inv_rms(x4 + (long long)b * n4, n4, norm_eps, lane) : 1.f;
                double acc = 0.0;
                for (int c = lane; c < n4; c += 64) {
                    const float4 v = x4[(long long)b * n4 + c];
                    acc = dot4d(W4[c], norm ? make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv) : v, acc);
                }
                acc = wave_sum(acc);
                if (lane == 0) logits[(long long)b * E + e] = acc + bb;
            }
        }
    }
}

void launch_router(int bits, const float* x, int B, const float* W, const float* bias, int H, int E, double* logits,
                   uint4* xq, float4* xst, hipStream_t s, Timing t, float norm_eps)
{
    const int rw = norm_eps >= 0.f ? RT_NORM_WAVES : RT_WAVES;
    const int rblocks = (E + rw - 1) / rw;
    const int prepB = xq ? B : 0;
    int prep_blocks = (prepB * (H / 64) + rw - 1) / rw;
    if (prep_blocks > 1024) prep_blocks = 1024;
    const int blocks = rblocks + prep_blocks;
    if (bits == 2)
        hipExtLaunchKernelGGL(k_router<2>, dim3(blocks), dim3(64 * rw), 0, s, t.start, t.stop, 0, x, B, prepB, W, bias,
                              H, E, logits, xq, xst, norm_eps, rblocks);
    else if (bits == 3)
        hipExtLaunchKernelGGL(k_router<3>, dim3(blocks), dim3(64 * rw), 0, s, t.start, t.stop, 0, x, B, prepB, W, bias,
                              H, E, logits, xq, xst, norm_eps, rblocks);
    else
        hipExtLaunchKernelGGL(k_router<4>, dim3(blocks), dim3(64 * rw), 0, s, t.start, t.stop, 0, x, B, prepB, W, bias,
                              H, E, logits, xq, xst, norm_eps, rblocks);
}

// one wave per token: logits -> idx, w
__global__ __launch_bounds__(256) void k_topk(const double* __restrict__ logits, int B, int E, int K, int renorm,
                                              int32_t* __restrict__ idx, float* __restrict__ w)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int b = blockIdx.x * 4 + wave;
    if (b >= B) return;
    int id;
    float wt;
    double lv[16];
    topk_load<16>(logits + (long long)b * E, E, lane, lv);
    topk_select<32, 16>(lv, E, K, renorm, lane, id, wt);
    if (lane < K) {
        idx[(long long)b * K + lane] = id;
        w[(long long)b * K + lane] = wt;
    }
}

void launch_topk(const double* logits, int B, int E, int K, int renorm, int32_t* idx, float* w, hipStream_t s)
{
    hipLaunchKernelGGL(k_topk, dim3((B + 3) / 4), dim3(256), 0, s, logits, B, E, K, renorm, idx, w);
}

// ----------------------------------------------------------------------------
// gate/up: fused dequant-GEMV of the gate and up rows + SwiGLU, for every
// active expert of one token.  A wave owns RPW rows (RPP rows per pass when a
// row has fewer than 64 groups) of all K+1 experts.  It first issues the
// shared expert's loads (no routing needed), then selects the token's experts
// from the logits while those loads are in flight (or takes the caller's
// routing), then issues the routed experts' loads.  h = silu(g) * u is written
// in fp32 in the order of the pair layout the down GEMV reads.
// ----------------------------------------------------------------------------
constexpr int GU_RPW = 1;   // row passes per wave
constexpr int GU_SC = 5;    // expert slots held in registers per round
constexpr int DN_RPW = 1;   // row passes per wave, down
constexpr int DN_SC = 5;    // expert slots staged per LDS round, down

struct FfnArgs {
    const uint8_t* slab;
    Layout L;
    const uint4* xq;
    const float4* xst;
    const double* logits;  // route from logits (nullptr: use idx / w)
    int renorm;
    int32_t* idx;          // [B][K]: read, or written by block 0 when routing from logits
    float* w;
    int K, E;
    float shared_w;
    float* hq;             // h in fp32, pair-layout order: [B*(K+1)][8][Gi][8]
    float* y;
    int sc;                // down: slots per LDS round
    // tiered residency, filled inside the gate/up launch (k_gateup_fill): the cache
    // plan (count, then (expert, slot) pairs of this call's misses), the store of
    // records in host memory, and the extra blocks that copy the records' scale/bias
    // and down part
    const int32_t* fill_plan;
    const uint8_t* fill_src;
    int fill_cap;     // most entries the plan holds (<= 64)
    int fill_blocks;
};

template <int BITS>
struct SlotRegs {
    uint4 g0, g1, u0, u1;
    uint2 sb;
};

template <int BITS>
__global__ __launch_bounds__(256) void k_gateup(FfnArgs A)
{
    const Layout& L = A.L;
    const int b = blockIdx.y, K = A.K, KS = K + 1;
    const int G = L.Gh, LPR = lanes_per_row(G), RPP = 64 / LPR;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane / LPR, gl = lane & (LPR - 1);
    const int row0 = (blockIdx.x * 4 + wave) * GU_RPW * RPP + sub;
    const Masks M = load_masks();
    float* hq_tok = A.hq + (long long)b * KS * L.Gi * 64;

    // routing inputs first: they are cache-resident and gate every routed load
    double lv[16];
    int my_id = 0;
    float my_w = 0.f;
    if (A.logits)
        topk_load<16>(A.logits + (long long)b * A.E, A.E, lane, lv);
    else if (lane < K)
        my_id = A.idx[(long long)b * K + lane];
    bool routed = false;

    auto issue = [&](SlotRegs<BITS> (&R)[GU_RPW], int e, int g, bool gv) {
        const uint8_t* rec = A.slab + (long long)e * L.record;
#pragma unroll
        for (int p = 0; p < GU_RPW; ++p) {
            const int r = row0 + p * RPP;
            if (gv && r < L.I) {
                const uint8_t* base = rec + (long long)r * 2 * L.hb;
                R[p].g0 = ld16(base + g * 16);
                R[p].u0 = ld16(base + L.hb + g * 16);
                if (BITS == 4) {
                    R[p].g1 = ld16(base + (G + g) * 16);
                    R[p].u1 = ld16(base + L.hb + (G + g) * 16);
                } else if (BITS == 3) {
                    R[p].g1 = ld8(base + 16 * G + 8 * g);
                    R[p].u1 = ld8(base + L.hb + 16 * G + 8 * g);
                }
                R[p].sb = *reinterpret_cast<const uint2*>(rec + L.off_gu_sb + ((long long)r * L.Sh + (g >> L.gs)) * 8);
            }
        }
    };

    // slot order: the shared expert first (pos 0), then routed expert k at pos k + 1
    for (int r0 = 0; r0 < KS; r0 += GU_SC) {
        const int nr = min(GU_SC, KS - r0);
        float gacc[GU_SC][GU_RPW], uacc[GU_SC][GU_RPW];
        int eid[GU_SC];
#pragma unroll
        for (int i = 0; i < GU_SC; ++i)
#pragma unroll
            for (int p = 0; p < GU_RPW; ++p) gacc[i][p] = uacc[i][p] = 0.f;
        for (int g0 = 0; g0 < G; g0 += LPR) {
            const int g = g0 + gl;
            const bool gv = g < G;
            uint4 xp[8];
            float4 st = make_float4(0.f, 0.f, 0.f, 0.f);
            if (gv) {
#pragma unroll
                for (int j = 0; j < 8; ++j) xp[j] = A.xq[((long long)b * 8 + j) * G + g];
                st = A.xst[(long long)b * G + g];
            }
            SlotRegs<BITS> R[GU_SC][GU_RPW];
            int i0 = 0;
            if (r0 == 0) {
                eid[0] = A.E;  // the shared expert needs no routing: its loads go out first
                issue(R[0], A.E, g, gv);
                i0 = 1;
                if (!routed) {
                    if (A.logits) {
                        topk_select<32, 16>(lv, A.E, K, A.renorm, lane, my_id, my_w);
                        if (blockIdx.x == 0 && wave == 0 && lane < K) {
                            A.idx[(long long)b * K + lane] = my_id;
                            A.w[(long long)b * K + lane] = my_w;
                        }
                    }
                    routed = true;
                }
            }
#pragma unroll
            for (int i = 0; i < GU_SC; ++i) {
                if (i < i0 || i >= nr) continue;
                int e = __builtin_amdgcn_readlane(my_id, r0 + i - 1);
                if (e < 0 || e >= A.E) e = -2;  // invalid id: its h becomes NaN
                eid[i] = e;
                if (e >= 0) issue(R[i], e, g, gv);
            }
#pragma unroll
            for (int i = 0; i < GU_SC; ++i)
#pragma unroll
                for (int p = 0; p < GU_RPW; ++p) {
                    const int r = row0 + p * RPP;
                    if (i < nr && eid[i] >= 0 && gv && r < L.I) {
                        const float dg = group_dot<BITS>(M, R[i][p].g0, R[i][p].g1, xp);
                        const float du = group_dot<BITS>(M, R[i][p].u0, R[i][p].u1, xp);
                        const uint2 sb = R[i][p].sb;
                        gacc[i][p] = fmaf(bf16_lo(sb.x) * st.z, dg - st.x, fmaf(bf16_hi(sb.x), st.y, gacc[i][p]));
                        uacc[i][p] = fmaf(bf16_lo(sb.y) * st.z, du - st.x, fmaf(bf16_hi(sb.y), st.y, uacc[i][p]));
                    }
                }
        }
#pragma unroll
        for (int i = 0; i < GU_SC; ++i) {
            if (i >= nr) continue;
            const int pos = r0 + i;
            const int k = pos == 0 ? K : pos - 1;
            float* hq = hq_tok + (long long)k * L.Gi * 64;
#pragma unroll
            for (int p = 0; p < GU_RPW; ++p) {
                const float gg = lane_group_sum(gacc[i][p], LPR);
                const float uu = lane_group_sum(uacc[i][p], LPR);
                const int r = row0 + p * RPP;
                if (gl == 0 && r < L.I) {
                    const float h = eid[i] < 0 ? __builtin_nanf("") : gg / (1.f + __expf(-gg)) * uu;
                    // input column r of the down GEMV, in the pair layout
                    const int grp = r >> 6, cc = r & 63;
                    int pp, hi;
                    if (BITS == 4) {
                        pp = 4 * (cc >> 3) + (cc & 3);
                        hi = (cc >> 2) & 1;
                    } else {
                        pp = 8 * (cc >> 4) + (cc & 7);
                        hi = (cc >> 3) & 1;
                    }
                    hq[((long long)(pp >> 2) * L.Gi + grp) * 8 + (pp & 3) * 2 + hi] = h;
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------
// h staging of the down kernels.  An item is one quarter of a (slot s, group g)
// pair: the pair-layout uint4 j = 2*part and 2*part + 1 of that group, 16 fp32
// values of h.  The group's four items scale it by a power of two taken from
// the group's largest |h|, store it in the operand format of the code width
// (4- and 2-bit: digit planes; 3-bit: fp16 pairs) and derive the group's stats
// (C, S, scale) in one pass: a group whose h is tiny keeps its relative precision.
// pairs: uint4 (s, j, g) at pair_base + s * pair_slot + j * G + g
// stats: uint4 (s, g) at stat_base + s * stat_slot + g
// ----------------------------------------------------------------------------
struct HItem {
    float4 v[4];
};

__device__ inline void h_item_load(const float4* htok, int G, int it, int n_items, HItem& H)
{
    const int itc = it < n_items ? it : 0;
    const int sg = itc >> 2, part = itc & 3;
    const int sl = sg / G, g = sg - sl * G;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int u = (sl * 8 + 2 * part + jj) * G + g;
        H.v[2 * jj] = htok[2 * u];
        H.v[2 * jj + 1] = htok[2 * u + 1];
    }
}

// every lane of a 4-lane group must call this (the group reductions are DPP)
template <int BITS>
__device__ inline void h_item_stage(const HItem& H, int G, int it, int n_items, uint4* lds, int pair_slot,
                                    int stat_base, int stat_slot)
{
    const bool ok = it < n_items;
    const int itc = ok ? it : 0;
    const int sg = itc >> 2, part = itc & 3;
    const int sl = sg / G, g = sg - sl * G;
    float m = fmaxf(absmax8(H.v[0], H.v[1]), absmax8(H.v[2], H.v[3]));
    m = group_reduce(m, OpMax(), 4);
    if constexpr (BITS == 4 || BITS == 2) {
        const int e = q4_exponent(m);
        const float inv = exp2i_f(-e);
        // the item's 16 values in natural column order per output uint4: 4-bit, the
        // pair-layout uint4 j hold columns 0 4 1 5 2 6 3 7 of their 8; 2-bit, the two
        // hold columns 0 8 1 9 2 10 3 11 and 4 12 5 13 6 14 7 15 of the item's 16, and
        // the outputs are the even and the odd columns
        const float4 v0 = H.v[0], v1 = H.v[1], v2 = H.v[2], v3 = H.v[3];
        float c[2][8];
        if constexpr (BITS == 4) {
            const float a[2][8] = {{v0.x, v0.z, v1.x, v1.z, v0.y, v0.w, v1.y, v1.w},
                                   {v2.x, v2.z, v3.x, v3.z, v2.y, v2.w, v3.y, v3.w}};
#pragma unroll
            for (int i = 0; i < 16; ++i) c[i >> 3][i & 7] = a[i >> 3][i & 7];
        } else {
            const float a[2][8] = {{v0.x, v1.x, v2.x, v3.x, v0.y, v1.y, v2.y, v3.y},
                                   {v0.z, v1.z, v2.z, v3.z, v0.w, v1.w, v2.w, v3.w}};
#pragma unroll
            for (int i = 0; i < 16; ++i) c[i >> 3][i & 7] = a[i >> 3][i & 7];
        }
        float sx = 0.f;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            uint32_t W[8], su = 0u;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                W[i] = q4_bits(c[jj][i], inv);
                su += W[i];
            }
            sx += (float)(int)(su - 8u * (Q4_HIGH + 0x8888u));  // sum of the 8 X, mod 2^32 exact
            if (ok) lds[sl * pair_slot + (2 * part + jj) * G + g] = digit_planes(W);
        }
        float sum = ((v0.x + v0.y) + (v0.z + v0.w)) + ((v1.x + v1.y) + (v1.z + v1.w)) +
                    (((v2.x + v2.y) + (v2.z + v2.w)) + ((v3.x + v3.y) + (v3.z + v3.w)));
        sx = group_reduce(sx, OpAdd(), 4);
        sum = group_reduce(sum, OpAdd(), 4);
        if (ok && part == 0) {
            const float sc = (m <= 3.4e38f) ? exp2i_f(e) : __builtin_nanf("");
            lds[stat_base + sl * stat_slot + g] =
                __builtin_bit_cast(uint4, make_float4(q_int_C<BITS>(sx, sum, inv), sum, sc, 0.f));
        }
        return;
    }
    const int e = h_exponent(m);
    const float inv = exp2i_f(-e);
    float off = 0.f, sum = 0.f;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * part + jj;
        const uint4 u = h_pairs(H.v[2 * jj], H.v[2 * jj + 1], inv);
        if (ok) lds[sl * pair_slot + j * G + g] = u;
        const uint32_t pr[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int el = 0; el < 4; ++el) {
            const h2 hh = __builtin_bit_cast(h2, pr[el]);
            const float ps = (float)hh.x + (float)hh.y;
            off = fmaf(pair_class_inv(BITS, 4 * j + el), ps, off);
            sum += ps;
        }
    }
    off = group_reduce(off, OpAdd(), 4);
    sum = group_reduce(sum, OpAdd(), 4);
    if (ok && part == 0) {
        const float sc = exp2i_f(e);
        lds[stat_base + sl * stat_slot + g] = __builtin_bit_cast(uint4, make_float4(1024.f * off, sc * sum, sc, 0.f));
    }
}

// ----------------------------------------------------------------------------
// down: dequant-GEMV of the down rows + router-weighted combine, one pass.  A
// block owns output rows of one token for every active expert.  It fetches
// the token's h (fp32, cache-resident) first, then issues its weight loads,
// scales each expert's h by a power of two from its largest |h|, stages it in
// LDS in the operand format of the code width and derives each group's stats there while the weights
// stream in, and writes y = sum_k w_k Wd_k h_k + shared_weight * Wd_s h_s.
// ----------------------------------------------------------------------------
constexpr int DN_HREG = 4;  // pair-layout uint4 of h staged per thread per round

template <int BITS>
__global__ __launch_bounds__(256) void k_down(FfnArgs A)
{
    extern __shared__ uint4 lds[];  // [sc][9][Gi]: 8 uint4 of h pairs, then the group stats
    const Layout& L = A.L;
    const int b = blockIdx.y, K = A.K, KS = K + 1;
    const int G = L.Gi, LPR = lanes_per_row(G), RPP = 64 / LPR;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane / LPR, gl = lane & (LPR - 1);
    const int row0 = (blockIdx.x * 4 + wave) * DN_RPW * RPP + sub;
    const Masks M = load_masks();
    const float4* hq4 = reinterpret_cast<const float4*>(A.hq) + (long long)b * KS * 8 * G * 2;
    float acc[DN_RPW];
#pragma unroll
    for (int p = 0; p < DN_RPW; ++p) acc[p] = 0.f;

    for (int s0 = 0; s0 < KS; s0 += A.sc) {
        const int ns = min(A.sc, KS - s0);
        const int n_items = ns * G * 4;  // <= 512: two items per thread
        // the round's h (cache-resident) first; clamped indices keep every load in bounds
        static_assert(DN_HREG == 4, "a round stages at most 1024 pair-layout uint4 of h");
        const float4* hsrc = hq4 + (long long)s0 * 8 * G * 2;
        HItem hi0, hi1;
        h_item_load(hsrc, G, threadIdx.x, n_items, hi0);
        h_item_load(hsrc, G, threadIdx.x + 256, n_items, hi1);
        const uint8_t* rec[DN_SC];
        float wt[DN_SC];
#pragma unroll
        for (int s = 0; s < DN_SC; ++s) {
            rec[s] = nullptr;
            wt[s] = 0.f;
            if (s < ns) {
                const int k = s0 + s;
                const int e = (k < K) ? A.idx[b * K + k] : A.E;
                const bool bad = (k < K) && (e < 0 || e >= A.E);
                wt[s] = bad ? __builtin_nanf("") : ((k < K) ? A.w[b * K + k] : A.shared_w);
                rec[s] = bad ? nullptr : A.slab + (long long)e * L.record;
            }
        }
        uint4 c0[DN_SC][DN_RPW], c1[DN_SC][DN_RPW];
        uint32_t sbv[DN_SC][DN_RPW];
        auto issue = [&](int g, bool gv) {
#pragma unroll
            for (int s = 0; s < DN_SC; ++s)
#pragma unroll
                for (int p = 0; p < DN_RPW; ++p) {
                    const int r = row0 + p * RPP;
                    if (rec[s] && gv && r < L.H) {
                        const uint8_t* base = rec[s] + L.off_d_codes;
                        c0[s][p] = ld16(base + d_chunk_off(L, r, g));
                        if (BITS == 4) c1[s][p] = ld16(base + d_chunk_off(L, r, G + g));
                        if (BITS == 3) c1[s][p] = ld8(base + d_chunk_off(L, r, G + (g >> 1)) + 8 * (g & 1));
                        sbv[s][p] = *reinterpret_cast<const uint32_t*>(rec[s] + L.off_d_sb +
                                                                       ((long long)r * L.Si + (g >> L.gs)) * 4);
                    }
                }
        };
        auto compute = [&](int g, bool gv) {
#pragma unroll
            for (int s = 0; s < DN_SC; ++s) {
                if (s >= ns || !gv) continue;
                uint4 xp[8];
                const uint4* src = lds + s * 9 * G + g;
#pragma unroll
                for (int j = 0; j < 8; ++j) xp[j] = src[j * G];
                const float4 st = __builtin_bit_cast(float4, src[8 * G]);
#pragma unroll
                for (int p = 0; p < DN_RPW; ++p) {
                    const int r = row0 + p * RPP;
                    if (r < L.H) {
                        if (!rec[s]) {
                            acc[p] += wt[s];  // NaN for an invalid expert id
                            continue;
                        }
                        const float d = group_dot<BITS>(M, c0[s][p], c1[s][p], xp);
                        const float part = fmaf(bf16_lo(sbv[s][p]) * st.z, d - st.x, bf16_hi(sbv[s][p]) * st.y);
                        acc[p] = fmaf(wt[s], part, acc[p]);
                    }
                }
            }
        };
        if (s0 > 0) __syncthreads();  // the previous round's LDS reads are done
        issue(gl, gl < G);
        h_item_stage<BITS>(hi0, G, threadIdx.x, n_items, lds, 9 * G, 8 * G, 9 * G);
        h_item_stage<BITS>(hi1, G, threadIdx.x + 256, n_items, lds, 9 * G, 8 * G, 9 * G);
        __syncthreads();
        compute(gl, gl < G);
        for (int g0 = LPR; g0 < G; g0 += LPR) {
            issue(g0 + gl, g0 + gl < G);
            compute(g0 + gl, g0 + gl < G);
        }
    }
#pragma unroll
    for (int p = 0; p < DN_RPW; ++p) {
        const float v = lane_group_sum(acc[p], LPR);
        const int r = row0 + p * RPP;
        if (gl == 0 && r < L.H) A.y[(long long)b * L.H + r] = v;
    }
}

// ----------------------------------------------------------------------------
// Straight-line fast path for the common shapes (K+1 <= 9 experts per token,
// H <= 4096, I <= 4096): one group pass, one round of slots, every load at a
// clamped in-bounds address and every boundary handled by selects, so the
// compiler can keep the loads of all phases in flight and wait only for what
// each phase needs.
// ----------------------------------------------------------------------------
constexpr int FAST_NL = 8;  // fast path: E <= 512 logits per token, 8 per lane

constexpr int GUF_WAVES = 8;  // fast gate/up: waves per block
constexpr long long FILL_CHUNK = 64 * 1024;  // bytes of a missed record per extra fill block
constexpr int GUF_XQ = (64 * 9 + 64 * GUF_WAVES - 1) / (64 * GUF_WAVES);  // operand uint4 per thread (G <= 64)

// One (row pass, expert slot) per wave, blocks in slot-major order: the shared
// expert's blocks (slot 0) come first and need no routing; a routed block's wave
// 0 selects its expert while the block stages the token's operand.
// Many small waves per SIMD overlap one another's loads and dequant arithmetic.
template <int BITS, int KS, bool ROUTE, bool FILL>
__device__ __forceinline__ void gateup_fast(const FfnArgs& A, uint4* __restrict__ xs, int& s_id, int& s_src)
{
    constexpr int K = KS - 1;
    const Layout& L = A.L;
    const int b = blockIdx.y;
    const int G = L.Gh, LPR = lanes_per_row(G), RPP = 64 / LPR;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane / LPR, gl = lane & (LPR - 1);
    const bool gv = gl < G;
    const int g = gv ? gl : G - 1;
    const int rows_pb = GUF_WAVES * RPP;
    const int bps = (L.I + rows_pb - 1) / rows_pb;  // blocks per slot
    // block groups: the shared expert's first, then the routed experts from the
    // last rank to the first, so that the blocks dispatched last need the fewest
    // selection rounds (a block selects only up to its own rank)
    if (FILL && (int)blockIdx.x >= KS * bps) {
        // extra blocks: copy chunk c of the scale/bias and down part of each missed
        // record (the routed blocks write its gate/up codes), token 0's grid row only
        if (blockIdx.y != 0) return;
        const int c = blockIdx.x - KS * bps;
        const long long part = L.record - L.off_gu_sb;
        const int nch = (int)((part + FILL_CHUNK - 1) / FILL_CHUNK);
        const int i = c / nch, ch = c - i * nch;
        if (i >= A.fill_plan[0]) return;
        const int e = A.fill_plan[1 + 2 * i], sl = A.fill_plan[2 + 2 * i];
        if (sl < 0) return;
        const long long lo = L.off_gu_sb + (long long)ch * FILL_CHUNK;
        const long long hi = lo + FILL_CHUNK < L.record ? lo + FILL_CHUNK : L.record;
        const uint4* from = reinterpret_cast<const uint4*>(A.fill_src + (long long)e * L.record);
        uint4* to = reinterpret_cast<uint4*>(const_cast<uint8_t*>(A.slab) + (long long)sl * L.record);
        for (long long o = lo / 16 + threadIdx.x; o < hi / 16; o += 64 * GUF_WAVES) to[o] = from[o];
        return;
    }
    const int sg = blockIdx.x / bps;
    const int slot = (sg > 0) ? KS - sg : 0;  // 0: shared expert, k + 1: routed expert of rank k
    const int r = ((blockIdx.x - sg * bps) * GUF_WAVES + wave) * RPP + sub;
    const bool rv = r < L.I;
    const int rc = rv ? r : L.I - 1;
    const Masks M = load_masks();

    // 1. cache-resident inputs first (so waiting for them never waits for weights):
    //    a routed block's wave 0 the routing inputs, every thread a share of the operand
    double lv[FAST_NL];
    int my_id = 0;
    int f_n = 0, f_e = 0, f_s = -1;  // FILL: the plan's count and lane l's miss (expert, slot)
    if (slot > 0 && wave == 0) {
        if (ROUTE)
            topk_load<FAST_NL>(A.logits + (long long)b * A.E, A.E, lane, lv);
        else
            my_id = A.idx[(long long)b * K + min(lane, K - 1)];
        if (FILL) {  // at most 64 misses (the launcher's condition), read with the routing
            const int l = min(lane, A.fill_cap - 1);
            f_n = A.fill_plan[0];
            f_e = A.fill_plan[1 + 2 * l];
            f_s = A.fill_plan[2 + 2 * l];
        }
    }
    const int nx = G * 9;  // uint4 of pairs ([8][G]) then stats ([G])
    uint4 xv[GUF_XQ];
#pragma unroll
    for (int q = 0; q < GUF_XQ; ++q) {
        const int t = min((int)threadIdx.x + 64 * GUF_WAVES * q, nx - 1);
        xv[q] = t < 8 * G ? A.xq[(long long)b * 8 * G + t]
                          : __builtin_bit_cast(uint4, A.xst[(long long)b * G + (t - 8 * G)]);
    }
    __builtin_amdgcn_sched_barrier(0);

    SlotRegs<BITS> R;
    auto issue = [&](const uint8_t* rec) {
        const uint8_t* base = rec + (long long)rc * 2 * L.hb;
        R.g0 = ld16(base + g * 16);
        R.u0 = ld16(base + L.hb + g * 16);
        if (BITS == 4) {
            R.g1 = ld16(base + (G + g) * 16);
            R.u1 = ld16(base + L.hb + (G + g) * 16);
        } else if (BITS == 3) {
            R.g1 = ld8(base + 16 * G + 8 * g);
            R.u1 = ld8(base + L.hb + 16 * G + 8 * g);
        }
        R.sb = *reinterpret_cast<const uint2*>(rec + L.off_gu_sb + ((long long)rc * L.Sh + (g >> L.gs)) * 8);
    };
    // 2. the shared expert needs no routing: its loads go out now
    if (slot == 0) issue(A.slab + (long long)A.E * L.record);
    __builtin_amdgcn_sched_barrier(0);
    // 3. stage the token's operand; wave 0 of a routed block selects its expert meanwhile
#pragma unroll
    for (int q = 0; q < GUF_XQ; ++q) {
        const int t = threadIdx.x + 64 * GUF_WAVES * q;
        if (t < nx) xs[t] = xv[q];
    }
    if (slot > 0 && wave == 0) {
        int id;
        if (ROUTE && blockIdx.x != bps) {
            id = __builtin_amdgcn_readfirstlane(topk_nth<K, FAST_NL>(lv, A.E, slot - 1, lane));
        } else {
            if (ROUTE) {  // the first routed block (rank K - 1) selects all K and publishes the routing
                float my_w;
                topk_select<K, FAST_NL>(lv, A.E, K, A.renorm, lane, my_id, my_w);
                if (lane < K) {
                    A.idx[(long long)b * K + lane] = my_id;
                    A.w[(long long)b * K + lane] = my_w;
                }
            }
            id = __builtin_amdgcn_readlane(my_id, slot - 1);
        }
        if (FILL) {  // a slot filled by this call: its record comes from the store, by expert
            const unsigned long long m = __ballot(lane < f_n && f_s == id);
            if (lane == 0) s_src = m ? __builtin_amdgcn_readlane(f_e, __builtin_ctzll(m)) : -1;
        }
        if (lane == 0) s_id = id;
    }
    __syncthreads();
    // 4. a routed block's loads (an invalid id reads expert 0 and yields NaN)
    bool bad = false;
    int src = -1;
    if (slot > 0) {
        const int e = s_id;
        bad = (e < 0 || e >= A.E);
        if (FILL && !bad) src = s_src;
        issue((FILL && src >= 0) ? A.fill_src + (long long)src * L.record : A.slab + (long long)(bad ? 0 : e) * L.record);
    }
    __builtin_amdgcn_sched_barrier(0);
    uint4 xp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xp[j] = xs[j * G + g];
    const float4 st = __builtin_bit_cast(float4, xs[8 * G + g]);
    // 5. dequant-GEMV of the row's gate and up, SwiGLU, h into the pair-layout order
    const float dg = group_dot<BITS>(M, R.g0, R.g1, xp);
    const float du = group_dot<BITS>(M, R.u0, R.u1, xp);
    float ga = fmaf(bf16_lo(R.sb.x) * st.z, dg - st.x, bf16_hi(R.sb.x) * st.y);
    float ua = fmaf(bf16_lo(R.sb.y) * st.z, du - st.x, bf16_hi(R.sb.y) * st.y);
    ga = lane_group_sum(gv ? ga : 0.f, LPR);
    ua = lane_group_sum(gv ? ua : 0.f, LPR);
    if (gl == 0 && rv) {
        const float h = bad ? __builtin_nanf("") : ga / (1.f + __expf(-ga)) * ua;
        const int k = (slot == 0) ? K : slot - 1;
        const int grp = rc >> 6, cc = rc & 63;
        int pp, hi;
        if (BITS == 4) {
            pp = 4 * (cc >> 3) + (cc & 3);
            hi = (cc >> 2) & 1;
        } else {
            pp = 8 * (cc >> 4) + (cc & 7);
            hi = (cc >> 3) & 1;
        }
        A.hq[((long long)b * KS + k) * L.Gi * 64 + ((long long)(pp >> 2) * L.Gi + grp) * 8 + (pp & 3) * 2 + hi] = h;
    }
    if (FILL && src >= 0) {  // the codes this wave read from the store go into the slot
        uint8_t* base = const_cast<uint8_t*>(A.slab) + (long long)s_id * L.record + (long long)rc * 2 * L.hb;
        *reinterpret_cast<uint4*>(base + g * 16) = R.g0;
        *reinterpret_cast<uint4*>(base + L.hb + g * 16) = R.u0;
        if (BITS == 4) {
            *reinterpret_cast<uint4*>(base + (G + g) * 16) = R.g1;
            *reinterpret_cast<uint4*>(base + L.hb + (G + g) * 16) = R.u1;
        } else if (BITS == 3) {
            *reinterpret_cast<uint2*>(base + 16 * G + 8 * g) = make_uint2(R.g1.x, R.g1.y);
            *reinterpret_cast<uint2*>(base + L.hb + 16 * G + 8 * g) = make_uint2(R.u1.x, R.u1.y);
        }
    }
}

template <int BITS, int KS, bool ROUTE>
__global__ __launch_bounds__(64 * GUF_WAVES) void k_gateup_fast(FfnArgs A)
{
    __shared__ uint4 xs[64 * 9];  // the token's operand: 8 uint4 of pairs + stats per group (G <= 64)
    __shared__ int s_id;          // a routed block's expert
    int unused = -1;
    gateup_fast<BITS, KS, ROUTE, false>(A, xs, s_id, unused);
}

// The cached decode's gate/up: routing given as slot ids, and the records this
// call's plan brings in are filled inside the launch.  A routed block whose slot
// was just assigned reads its rows from the store in host memory and writes the
// codes into the slot; extra blocks after the gate/up blocks copy the rest of
// each missed record, so the down launch finds the records whole.
template <int BITS, int KS>
__global__ __launch_bounds__(64 * GUF_WAVES) void k_gateup_fill(FfnArgs A)
{
    __shared__ uint4 xs[64 * 9];
    __shared__ int s_id, s_src;
    gateup_fast<BITS, KS, false, true>(A, xs, s_id, s_src);
}

constexpr int DNF_WAVES = 4;  // fast down: waves per block

template <int BITS, int KS>
__global__ __launch_bounds__(64 * DNF_WAVES) void k_down_fast(FfnArgs A)
{
    constexpr int K = KS - 1;
    extern __shared__ uint4 lds[];  // h pairs [KS][8][Gi], then stats [KS][Gi]
    const Layout& L = A.L;
    const int b = blockIdx.y;
    const int G = L.Gi, LPR = lanes_per_row(G), RPP = 64 / LPR;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane / LPR, gl = lane & (LPR - 1);
    const bool gv = gl < G;
    const int g = gv ? gl : G - 1;
    const int r = (blockIdx.x * DNF_WAVES + wave) * RPP + sub;
    const bool rv = r < L.H;
    const int rc = rv ? r : L.H - 1;
    const Masks M = load_masks();
    const int n = KS * 8 * G;  // pair-layout uint4 of the token's h, <= 1024
    const int n_items = KS * G * 4;  // <= 512
    static_assert(64 * DNF_WAVES * 2 >= 512, "h staging takes two items per thread");
    // Issue order matters: gfx9 counts outstanding vector loads in order, so each
    // wait below covers only what was issued before the data it needs.
    // 1. the routing (cache-resident, one slot per lane): the routed rows wait for it
    const int my_id = A.idx[b * K + min(lane, K - 1)];
    const float my_w = A.w[b * K + min(lane, K - 1)];
    __builtin_amdgcn_sched_barrier(0);
    // 2. the token's h (cache-resident): the staging waits for it
    const float4* hsrc = reinterpret_cast<const float4*>(A.hq) + (long long)b * n * 2;
    HItem hi0, hi1;
    h_item_load(hsrc, G, threadIdx.x, n_items, hi0);
    h_item_load(hsrc, G, threadIdx.x + 64 * DNF_WAVES, n_items, hi1);
    __builtin_amdgcn_sched_barrier(0);
    // 3. the shared expert's rows need no routing: they go out before the routing returns
    uint4 c0[KS], c1[KS];
    uint32_t sbv[KS];
    const long long o0 = L.off_d_codes + d_chunk_off(L, rc, g);
    const long long o1 = BITS == 3 ? L.off_d_codes + d_chunk_off(L, rc, G + (g >> 1)) + 8 * (g & 1)
                                   : L.off_d_codes + d_chunk_off(L, rc, G + g);
    auto issue = [&](int k, int e) {
        const uint8_t* rec = A.slab + (long long)e * L.record;
        c0[k] = ld16(rec + o0);
        if (BITS == 4) c1[k] = ld16(rec + o1);
        if (BITS == 3) c1[k] = ld8(rec + o1);
        sbv[k] = *reinterpret_cast<const uint32_t*>(rec + L.off_d_sb + ((long long)rc * L.Si + (g >> L.gs)) * 4);
    };
    issue(K, A.E);
    float wt[KS];
    wt[K] = A.shared_w;
    __builtin_amdgcn_sched_barrier(0);
    // 4. the routed rows
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int e = __builtin_amdgcn_readlane(my_id, k);
        const bool bad = (e < 0 || e >= A.E);
        wt[k] = bad ? __builtin_nanf("") : __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), k));
        issue(k, bad ? 0 : e);
    }
    __builtin_amdgcn_sched_barrier(0);
    // 3. scale h per group, stage it in the operand format and derive each group's stats
    //    while the weights stream in
    uint4* lst = lds + n;
    h_item_stage<BITS>(hi0, G, threadIdx.x, n_items, lds, 8 * G, n, G);
    h_item_stage<BITS>(hi1, G, threadIdx.x + 64 * DNF_WAVES, n_items, lds, 8 * G, n, G);
    __syncthreads();
    // 4. dequant-GEMV and combine
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        uint4 xp[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) xp[j] = lds[(k * 8 + j) * G + g];
        const float4 sv = __builtin_bit_cast(float4, lst[k * G + g]);
        const float d = group_dot<BITS>(M, c0[k], c1[k], xp);
        const float part = fmaf(bf16_lo(sbv[k]) * sv.z, d - sv.x, bf16_hi(sbv[k]) * sv.y);
        acc = fmaf(wt[k], part, acc);
    }
    acc = lane_group_sum(gv ? acc : 0.f, LPR);
    if (gl == 0 && rv) A.y[(long long)b * L.H + r] = acc;
}

int down_slots_per_round(const Layout& L)
{
    int sc = (256 * DN_HREG) / (8 * L.Gi);  // h of a round fits the per-thread staging registers
    if (sc > DN_SC) sc = DN_SC;
    return sc;  // >= 1 for I <= 8192
}

template <int BITS, int KS>
void launch_fast_ks(bool route, dim3 fg, dim3 fd, size_t flds, const FfnArgs& A, hipStream_t s, Timing tg, Timing td)
{
    if (A.fill_plan)
        hipExtLaunchKernelGGL((k_gateup_fill<BITS, KS>), dim3(fg.x + A.fill_blocks, fg.y), dim3(64 * GUF_WAVES), 0, s,
                              tg.start, tg.stop, 0, A);
    else if (route)
        hipExtLaunchKernelGGL((k_gateup_fast<BITS, KS, true>), fg, dim3(64 * GUF_WAVES), 0, s, tg.start, tg.stop, 0, A);
    else
        hipExtLaunchKernelGGL((k_gateup_fast<BITS, KS, false>), fg, dim3(64 * GUF_WAVES), 0, s, tg.start, tg.stop, 0,
                              A);
    hipExtLaunchKernelGGL((k_down_fast<BITS, KS>), fd, dim3(64 * DNF_WAVES), flds, s, td.start, td.stop, 0, A);
}

template <int BITS>
void launch_fast(int KS, bool route, dim3 fg, dim3 fd, size_t flds, const FfnArgs& A, hipStream_t s, Timing tg,
                 Timing td)
{
    switch (KS) {
    case 2: launch_fast_ks<BITS, 2>(route, fg, fd, flds, A, s, tg, td); break;
    case 3: launch_fast_ks<BITS, 3>(route, fg, fd, flds, A, s, tg, td); break;
    case 5: launch_fast_ks<BITS, 5>(route, fg, fd, flds, A, s, tg, td); break;
    case 7: launch_fast_ks<BITS, 7>(route, fg, fd, flds, A, s, tg, td); break;
    default: launch_fast_ks<BITS, 9>(route, fg, fd, flds, A, s, tg, td); break;
    }
}

// The single-token kernels apply (the fast path) and a cache plan of at most cap
// entries fits the gate/up launch's fill (one entry per lane of a wave).
static bool fast_path(const Layout& L, int K, int E)
{
    const int KS = K + 1;
    return L.Gh <= 64 && L.Gi <= 64 && KS * 8 * L.Gi <= 1024 && E <= 64 * FAST_NL &&
           (KS == 2 || KS == 3 || KS == 5 || KS == 7 || KS == 9);
}

bool ffn_fills_cache(const Layout& L, int K, int E, int cap) { return fast_path(L, K, E) && cap >= 1 && cap <= 64; }

void launch_ffn(const Layout& L, const void* slab, const uint4* xq, const float4* xst, const double* logits,
                int renorm, int32_t* idx, float* w, int B, int K, int E, float shared_w, void* hq, float* y,
                hipStream_t s, Timing t_gateup, Timing t_down, const int32_t* fill_plan, const void* fill_src,
                int fill_cap)
{
    FfnArgs A;
    A.fill_plan = fill_plan;
    A.fill_src = (const uint8_t*)fill_src;
    A.fill_cap = fill_cap;
    A.fill_blocks = fill_plan ? fill_cap * (int)((L.record - L.off_gu_sb + FILL_CHUNK - 1) / FILL_CHUNK) : 0;
    A.slab = (const uint8_t*)slab;
    A.L = L;
    A.xq = xq;
    A.xst = xst;
    A.logits = logits;
    A.renorm = renorm;
    A.idx = idx;
    A.w = w;
    A.K = K;
    A.E = E;
    A.shared_w = shared_w;
    A.hq = (float*)hq;
    A.y = y;
    A.sc = down_slots_per_round(L);
    const int grows = 4 * GU_RPW * (64 / lanes_per_row(L.Gh));
    const int drows = 4 * DN_RPW * (64 / lanes_per_row(L.Gi));
    const dim3 ggrid((L.I + grows - 1) / grows, B), dgrid((L.H + drows - 1) / drows, B);
    const int KS = K + 1;
    if (fast_path(L, K, E)) {
        const int grows = GUF_WAVES * (64 / lanes_per_row(L.Gh));
        const dim3 fg(KS * ((L.I + grows - 1) / grows), B);
        const int frows = DNF_WAVES * (64 / lanes_per_row(L.Gi));
        const dim3 fd((L.H + frows - 1) / frows, B);
        const size_t flds = (size_t)KS * 9 * L.Gi * 16;
        if (L.bits == 4)
            launch_fast<4>(KS, logits != nullptr, fg, fd, flds, A, s, t_gateup, t_down);
        else if (L.bits == 3)
            launch_fast<3>(KS, logits != nullptr, fg, fd, flds, A, s, t_gateup, t_down);
        else
            launch_fast<2>(KS, logits != nullptr, fg, fd, flds, A, s, t_gateup, t_down);
        return;
    }
    const size_t lds = (size_t)A.sc * 9 * L.Gi * 16;
    if (L.bits == 4) {
        hipExtLaunchKernelGGL(k_gateup<4>, ggrid, dim3(256), 0, s, t_gateup.start, t_gateup.stop, 0, A);
        hipExtLaunchKernelGGL(k_down<4>, dgrid, dim3(256), lds, s, t_down.start, t_down.stop, 0, A);
    } else if (L.bits == 3) {
        hipExtLaunchKernelGGL(k_gateup<3>, ggrid, dim3(256), 0, s, t_gateup.start, t_gateup.stop, 0, A);
        hipExtLaunchKernelGGL(k_down<3>, dgrid, dim3(256), lds, s, t_down.start, t_down.stop, 0, A);
    } else {
        hipExtLaunchKernelGGL(k_gateup<2>, ggrid, dim3(256), 0, s, t_gateup.start, t_gateup.stop, 0, A);
        hipExtLaunchKernelGGL(k_down<2>, dgrid, dim3(256), lds, s, t_down.start, t_down.stop, 0, A);
    }
}

// ----------------------------------------------------------------------------
// RMS renorm between stacked layers
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ y, int H, float eps, float* __restrict__ x)
{
    const int b = blockIdx.x, lane = threadIdx.x & 63;
    const float* yb = y + (long long)b * H;
    const float inv = row_inv_rms(reinterpret_cast<const float4*>(yb), H / 4, eps, lane);  // every wave alike
    for (int c = threadIdx.x; c < H; c += 256) x[(long long)b * H + c] = yb[c] * inv;
}

void launch_rmsnorm(const float* y, int B, int H, float eps, float* x, hipStream_t s)
{
    hipLaunchKernelGGL(k_rmsnorm, dim3(B), dim3(256), 0, s, y, H, eps, x);
}

}  // namespace moe
