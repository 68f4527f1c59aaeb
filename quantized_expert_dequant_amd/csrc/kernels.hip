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
//   k_prep    activation -> fp16 pairs + per-group stats (the operand of the
//             folded dequant: scale*x and bias*x per group, the FMA rearrangement
//             described in [LLMAPIS] section 深度分析, applied per group of 64)
//   k_router  logits (fp32 products accumulated in fp64), softmax, top-K
//   k_gateup  fused gate/up dequant-GEMV + SiLU*mul over the K routed + shared experts
//   k_down    down dequant-GEMV + router-weighted combine in one pass (no atomics)
#include <hip/hip_ext.h>

#include "common.h"
#include "launch.h"

namespace moe {

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
    const long long ng = 2LL * L.I * L.Gh + (long long)L.H * L.Gi;
    const int cpg = L.bits / 2;  // 16-byte chunks per group
    const long long n_gu_chunks = 2LL * L.I * (L.hb / 16);
    const long long n_gu_sb = (long long)L.I * L.Gh;
    const long long n_d_chunks = (long long)L.H * (L.ib / 16);
    const long long n_d_sb = (long long)L.H * L.Gi;
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
            const long long i = t - n_gu_chunks;  // r * Gh + g
            const long long nu = (long long)L.I * L.Gh;
            ushort4 v = make_ushort4(sc[i], bi[i], sc[nu + i], bi[nu + i]);
            *reinterpret_cast<ushort4*>(rec + L.off_gu_sb + i * 8) = v;
        } else if (t < n_gu_chunks + n_gu_sb + n_d_chunks) {
            const long long c = t - n_gu_chunks - n_gu_sb;
            const long long per_row = L.ib / 16;
            const long long r = c / per_row;
            const int pos = (int)(c - r * per_row);
            const int half = pos / L.Gi, g = pos - half * L.Gi;
            const uint8_t* src = down + j * ((long long)L.H * L.ib) + r * L.ib + (long long)(g * cpg + half) * 16;
            *reinterpret_cast<uint4*>(rec + L.off_d_codes + r * L.ib + (long long)pos * 16) =
                *reinterpret_cast<const uint4*>(src);
        } else {
            const long long i = t - n_gu_chunks - n_gu_sb - n_d_chunks;  // r * Gi + g
            const long long o = 2LL * L.I * L.Gh;
            ushort2 v = make_ushort2(sc[o + i], bi[o + i]);
            *reinterpret_cast<ushort2*>(rec + L.off_d_sb + i * 4) = v;
        }
    }
}

void launch_pack(const Layout& L, int n, const uint8_t* gate, const uint8_t* up, const uint8_t* down,
                 const uint16_t* scales, const uint16_t* biases, void* slab, int first, hipStream_t s)
{
    const long long total = 2LL * L.I * (L.hb / 16) + (long long)L.I * L.Gh + (long long)L.H * (L.ib / 16) +
                            (long long)L.H * L.Gi;
    long long blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_pack, dim3((unsigned)blocks, n), dim3(256), 0, s, L, gate, up, down, scales, biases,
                       (uint8_t*)slab, first);
}

// ----------------------------------------------------------------------------
// dequant of one packed record (layout check)
// ----------------------------------------------------------------------------
__device__ inline int packed_code(const uint8_t* row, int bits, int G, int c)
{
    const int g = c >> 6, cc = c & 63;
    const int per_chunk = 128 / bits;  // codes per 16-byte chunk
    const int half = cc / per_chunk, k = cc - half * per_chunk;
    const uint8_t* chunk = row + (long long)(half * G + g) * 16;
    if (bits == 4) return (chunk[k >> 1] >> ((k & 1) * 4)) & 15;
    return (chunk[k >> 2] >> ((k & 3) * 2)) & 3;
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
            const uint8_t* row = rec + (long long)r * 2 * L.hb + m * L.hb;
            q = packed_code(row, L.bits, L.Gh, c);
            const uint16_t* sb = reinterpret_cast<const uint16_t*>(rec + L.off_gu_sb + ((long long)r * L.Gh + (c >> 6)) * 8);
            s = __uint_as_float((uint32_t)sb[2 * m] << 16);
            b = __uint_as_float((uint32_t)sb[2 * m + 1] << 16);
        } else {
            const long long i = t - 2 * n_gu;
            const int r = (int)(i / L.I), c = (int)(i - (long long)r * L.I);
            q = packed_code(rec + L.off_d_codes + (long long)r * L.ib, L.bits, L.Gi, c);
            const uint16_t* sb = reinterpret_cast<const uint16_t*>(rec + L.off_d_sb + ((long long)r * L.Gi + (c >> 6)) * 4);
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
// prep: fp32 vectors [n_vec][len] -> fp16 pairs + stats, one wave per group
// ----------------------------------------------------------------------------
__device__ inline float exp2i(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

template <int BITS>
__global__ __launch_bounds__(256) void k_prep(const float* __restrict__ v, int len, int G,
                                              uint4* __restrict__ q, float4* __restrict__ st)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int g = blockIdx.x * 4 + wave, vec = blockIdx.y;
    if (g >= G) return;
    const float val = v[(long long)vec * len + g * 64 + lane];
    const float amax = wave_max(fabsf(val));
    int e = 0;
    if (amax > 0.f && amax <= 3.4e38f) {
        e = ilogbf(amax) - 14;  // amax * 2^-e in [2^14, 2^15)
        e = e < -110 ? -110 : (e > 113 ? 113 : e);
    }
    const float vs = val * exp2i(-e);  // exact power-of-two scaling
    const _Float16 vh = (_Float16)vs;
    int p, hi;
    if (BITS == 4) {
        const int d = lane >> 3, r = lane & 7;
        p = 4 * d + (r & 3);
        hi = r >> 2;
    } else {
        const int d = lane >> 4, r = lane & 15;
        p = 8 * d + (r & 7);
        hi = r >> 3;
    }
    uint16_t* qb = reinterpret_cast<uint16_t*>(q + (long long)vec * 8 * G);
    qb[((long long)(p >> 2) * G + g) * 8 + (p & 3) * 2 + hi] = __builtin_bit_cast(uint16_t, vh);
    // C = offset the fp16 code patterns add (1024 * sum_t S_t / t) plus the code
    // midpoint times the group's fp16 rounding error, so that the kernels compute
    // sum (q - mid) v_h + mid * sum v: the rounding errors of v then meet only
    // zero-mean code offsets and do not add up coherently across rows.
    constexpr float mid = BITS == 4 ? 7.5f : 1.5f;
    const float off = wave_sum((float)vh * pair_class_inv(BITS, p));
    const float rnd = wave_sum((float)vh - vs);  // exact per lane
    const float C = fmaf(off, 1024.f, mid * rnd);
    const float S = wave_sum(val);
    if (lane == 0) st[(long long)vec * G + g] = make_float4(C, S, exp2i(e), 0.f);
}

void launch_prep(int bits, const float* v, int n_vec, int len, uint4* q, float4* st, hipStream_t s)
{
    const int G = len / 64;
    dim3 grid((G + 3) / 4, n_vec);
    if (bits == 4)
        hipLaunchKernelGGL(k_prep<4>, grid, dim3(256), 0, s, v, len, G, q, st);
    else
        hipLaunchKernelGGL(k_prep<2>, grid, dim3(256), 0, s, v, len, G, q, st);
}

// ----------------------------------------------------------------------------
// router: logits + (last block) softmax / top-K
// ----------------------------------------------------------------------------
__device__ inline bool ranks_before(double va, int ia, double vb, int ib)
{
    return va > vb || (va == vb && ia < ib);
}

// one wave selects the top K of token b's E logits
__device__ void topk_wave(const double* __restrict__ lg, int E, int K, int renorm, int lane,
                          int32_t* __restrict__ idx_out, float* __restrict__ w_out)
{
    const int NL = (E + 63) / 64;  // <= 16
    double lv[16];
    uint32_t taken = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int id = lane + 64 * j;
        if (j < NL && id < E)
            lv[j] = __builtin_nontemporal_load(lg + id);
        else {
            lv[j] = -INFINITY;
            taken |= 1u << j;
        }
    }
    double my_v = -INFINITY;
    int my_id = 0x7FFFFFFF;
    double lmax = -INFINITY;
    for (int k = 0; k < K; ++k) {
        double bv = -INFINITY;
        int bid = 0x7FFFFFFF;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int id = lane + 64 * j;
            if (!(taken & (1u << j)) && ranks_before(lv[j], id, bv, bid)) {
                bv = lv[j];
                bid = id;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const double ov = __shfl_xor(bv, off, 64);
            const int oid = __shfl_xor(bid, off, 64);
            if (ranks_before(ov, oid, bv, bid)) {
                bv = ov;
                bid = oid;
            }
        }
        if (bid != 0x7FFFFFFF && (bid & 63) == lane) taken |= 1u << (bid >> 6);
        if (k == 0) lmax = bv;
        if (lane == k) {
            my_v = bv;
            my_id = bid;
        }
    }
    const double ew = (lane < K) ? exp(my_v - lmax) : 0.0;
    double denom;
    if (renorm) {
        denom = wave_sum(ew);
    } else {
        double part = 0.0;
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (j < NL && lane + 64 * j < E) part += exp(lv[j] - lmax);
        denom = wave_sum(part);
    }
    if (lane < K) {
        idx_out[lane] = my_id;
        w_out[lane] = (float)(ew / denom);
    }
}

__global__ __launch_bounds__(256) void k_router(const float* __restrict__ x, int B, const float* __restrict__ W,
                                                const float* __restrict__ bias, int H, int E, int K, int renorm,
                                                double* __restrict__ logits, unsigned* __restrict__ counter,
                                                int32_t* __restrict__ idx_out, float* __restrict__ w_out)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + wave;
    const int n4 = H >> 2;
    if (e < E) {
        const float4* W4 = reinterpret_cast<const float4*>(W) + (long long)e * n4;
        const double bb = bias ? (double)bias[e] : 0.0;
        if (n4 <= 1024) {
            float4 wv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int c = lane + 64 * i;
                wv[i] = c < n4 ? W4[c] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
            for (int b = 0; b < B; ++b) {
                const float4* x4 = reinterpret_cast<const float4*>(x) + (long long)b * n4;
                double acc = 0.0;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int c = lane + 64 * i;
                    if (c < n4) {
                        const float4 xv = x4[c];
                        acc = fma((double)wv[i].x, (double)xv.x, acc);
                        acc = fma((double)wv[i].y, (double)xv.y, acc);
                        acc = fma((double)wv[i].z, (double)xv.z, acc);
                        acc = fma((double)wv[i].w, (double)xv.w, acc);
                    }
                }
                acc = wave_sum(acc);
                if (lane == 0) logits[(long long)b * E + e] = acc + bb;
            }
        } else {
            for (int b = 0; b < B; ++b) {
                const float4* x4 = reinterpret_cast<const float4*>(x) + (long long)b * n4;
                double acc = 0.0;
                for (int c = lane; c < n4; c += 64) {
                    const float4 wv = W4[c], xv = x4[c];
                    acc = fma((double)wv.x, (double)xv.x, acc);
                    acc = fma((double)wv.y, (double)xv.y, acc);
                    acc = fma((double)wv.z, (double)xv.z, acc);
                    acc = fma((double)wv.w, (double)xv.w, acc);
                }
                acc = wave_sum(acc);
                if (lane == 0) logits[(long long)b * E + e] = acc + bb;
            }
        }
    }
    // the last block to arrive selects the experts of every token
    __shared__ int s_last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) s_last = (atomicAdd(counter, 1u) == gridDim.x - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    for (int b = wave; b < B; b += 4)
        topk_wave(logits + (long long)b * E, E, K, renorm, lane, idx_out + (long long)b * K, w_out + (long long)b * K);
    __syncthreads();
    if (threadIdx.x == 0) *counter = 0u;
}

void launch_router(const float* x, int B, const float* W, const float* bias, int H, int E, int K, int renorm,
                   double* logits, unsigned* counter, int32_t* idx, float* w, hipStream_t s, Timing t)
{
    hipExtLaunchKernelGGL(k_router, dim3((E + 3) / 4), dim3(256), 0, s, t.start, t.stop, 0, x, B, W, bias, H, E, K,
                          renorm, logits, counter, idx, w);
}

// ----------------------------------------------------------------------------
// fused gate/up dequant-GEMV + SwiGLU, per (token, expert slot)
// ----------------------------------------------------------------------------
__device__ inline uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

template <int BITS, int RPW>
__global__ __launch_bounds__(256) void k_gateup(const uint8_t* __restrict__ slab, Layout L,
                                                const uint4* __restrict__ xq, const float4* __restrict__ xst,
                                                const int32_t* __restrict__ idx, int K, int E,
                                                float* __restrict__ h)
{
    const int slot = blockIdx.y, KS = K + 1;
    const int b = slot / KS, k = slot - b * KS;
    const int e = (k < K) ? idx[b * K + k] : E;
    const bool bad = (k < K) && (e < 0 || e >= E);
    const int G = L.Gh, LPR = lanes_per_row(G), RPP = 64 / LPR;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane / LPR, gl = lane & (LPR - 1);
    const int row0 = (blockIdx.x * 4 + wave) * RPW * RPP + sub;
    float* hrow = h + (long long)slot * L.I;
    if (bad) {
#pragma unroll
        for (int p = 0; p < RPW; ++p) {
            const int r = row0 + p * RPP;
            if (gl == 0 && r < L.I) hrow[r] = __builtin_nanf("");
        }
        return;
    }
    const uint8_t* rec = slab + (long long)e * L.record;
    const Masks M = load_masks();
    float gacc[RPW], uacc[RPW];
#pragma unroll
    for (int p = 0; p < RPW; ++p) gacc[p] = uacc[p] = 0.f;

    for (int g0 = 0; g0 < G; g0 += LPR) {
        const int g = g0 + gl;
        const bool gv = g < G;
        uint4 xp[8];
        float4 st = make_float4(0.f, 0.f, 0.f, 0.f);
        if (gv) {
#pragma unroll
            for (int j = 0; j < 8; ++j) xp[j] = xq[((long long)b * 8 + j) * G + g];
            st = xst[(long long)b * G + g];
        }
        uint4 gc0[RPW], gc1[RPW], uc0[RPW], uc1[RPW];
        uint2 sb[RPW];
#pragma unroll
        for (int p = 0; p < RPW; ++p) {
            const int r = row0 + p * RPP;
            if (gv && r < L.I) {
                const uint8_t* base = rec + (long long)r * 2 * L.hb;
                gc0[p] = ld16(base + g * 16);
                uc0[p] = ld16(base + L.hb + g * 16);
                if (BITS == 4) {
                    gc1[p] = ld16(base + (G + g) * 16);
                    uc1[p] = ld16(base + L.hb + (G + g) * 16);
                }
                sb[p] = *reinterpret_cast<const uint2*>(rec + L.off_gu_sb + ((long long)r * G + g) * 8);
            }
        }
#pragma unroll
        for (int p = 0; p < RPW; ++p) {
            const int r = row0 + p * RPP;
            if (gv && r < L.I) {
                float dg, du;
                if (BITS == 4) {
                    dg = group_dot_q4(M, gc0[p], gc1[p], xp);
                    du = group_dot_q4(M, uc0[p], uc1[p], xp);
                } else {
                    dg = group_dot_q2(M, gc0[p], xp);
                    du = group_dot_q2(M, uc0[p], xp);
                }
                gacc[p] = fmaf(bf16_lo(sb[p].x) * st.z, dg - st.x, fmaf(bf16_hi(sb[p].x), st.y, gacc[p]));
                uacc[p] = fmaf(bf16_lo(sb[p].y) * st.z, du - st.x, fmaf(bf16_hi(sb[p].y), st.y, uacc[p]));
            }
        }
    }
#pragma unroll
    for (int p = 0; p < RPW; ++p) {
        const float g = lane_group_sum(gacc[p], LPR);
        const float u = lane_group_sum(uacc[p], LPR);
        const int r = row0 + p * RPP;
        if (gl == 0 && r < L.I) hrow[r] = g / (1.f + __expf(-g)) * u;
    }
}

constexpr int GU_RPW = 2;

int gateup_rows_per_block(const Layout& L) { return 4 * GU_RPW * (64 / lanes_per_row(L.Gh)); }

void launch_gateup(const Layout& L, const void* slab, const uint4* xq, const float4* xst, const int32_t* idx,
                   int B, int K, int E, float* h, hipStream_t s, Timing t)
{
    const int rpb = gateup_rows_per_block(L);
    dim3 grid((L.I + rpb - 1) / rpb, B * (K + 1));
    if (L.bits == 4)
        hipExtLaunchKernelGGL((k_gateup<4, GU_RPW>), grid, dim3(256), 0, s, t.start, t.stop, 0, (const uint8_t*)slab,
                              L, xq, xst, idx, K, E, h);
    else
        hipExtLaunchKernelGGL((k_gateup<2, GU_RPW>), grid, dim3(256), 0, s, t.start, t.stop, 0, (const uint8_t*)slab,
                              L, xq, xst, idx, K, E, h);
}

// ----------------------------------------------------------------------------
// down dequant-GEMV + weighted combine, per token; output rows owned by one wave
// ----------------------------------------------------------------------------
constexpr int DN_SC = 8;  // expert slots staged per LDS round
constexpr int DN_RPW = 1;

template <int BITS, int RPW>
__global__ __launch_bounds__(256) void k_down(const uint8_t* __restrict__ slab, Layout L,
                                              const uint4* __restrict__ hq, const float4* __restrict__ hst,
                                              const int32_t* __restrict__ idx, const float* __restrict__ w, int K,
                                              int E, float shared_w, int sc, float* __restrict__ y)
{
    extern __shared__ uint4 lds[];  // [sc][9][G]: 8 uint4 of pairs, then the stats float4
    const int b = blockIdx.y, KS = K + 1;
    const int G = L.Gi, LPR = lanes_per_row(G), RPP = 64 / LPR;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane / LPR, gl = lane & (LPR - 1);
    const int row0 = (blockIdx.x * 4 + wave) * RPW * RPP + sub;
    const Masks M = load_masks();
    float acc[RPW];
#pragma unroll
    for (int p = 0; p < RPW; ++p) acc[p] = 0.f;

    for (int s0 = 0; s0 < KS; s0 += sc) {
        const int ns = min(sc, KS - s0);
        const uint8_t* rec[DN_SC];
        float wt[DN_SC];
#pragma unroll
        for (int s = 0; s < DN_SC; ++s) {
            rec[s] = nullptr;
            wt[s] = 0.f;
            if (s < ns) {
                const int k = s0 + s;
                const int e = (k < K) ? idx[b * K + k] : E;
                const bool bad = (k < K) && (e < 0 || e >= E);
                wt[s] = bad ? __builtin_nanf("") : ((k < K) ? w[b * K + k] : shared_w);
                rec[s] = bad ? nullptr : slab + (long long)e * L.record;
            }
        }
        if (s0 > 0) __syncthreads();  // previous round's LDS reads are done
        for (int g0 = 0; g0 < G; g0 += LPR) {
            const int g = g0 + gl;
            const bool gv = g < G;
            uint4 c0[DN_SC][RPW], c1[DN_SC][RPW];
            uint32_t sbv[DN_SC][RPW];
#pragma unroll
            for (int s = 0; s < DN_SC; ++s)
#pragma unroll
                for (int p = 0; p < RPW; ++p) {
                    const int r = row0 + p * RPP;
                    if (rec[s] && gv && r < L.H) {
                        const uint8_t* base = rec[s] + L.off_d_codes + (long long)r * L.ib;
                        c0[s][p] = ld16(base + g * 16);
                        if (BITS == 4) c1[s][p] = ld16(base + (G + g) * 16);
                        sbv[s][p] = *reinterpret_cast<const uint32_t*>(rec[s] + L.off_d_sb + ((long long)r * G + g) * 4);
                    }
                }
            if (g0 == 0) {
                // stage this round's activation operands
                const int n = ns * 9 * G;
                for (int t = threadIdx.x; t < n; t += 256) {
                    const int s = t / (9 * G), rem = t - s * 9 * G, j = rem / G, gg = rem - j * G;
                    const long long slot = (long long)b * KS + s0 + s;
                    lds[t] = (j < 8) ? hq[(slot * 8 + j) * G + gg]
                                     : __builtin_bit_cast(uint4, hst[slot * G + gg]);
                }
                __syncthreads();
            }
#pragma unroll
            for (int s = 0; s < DN_SC; ++s) {
                if (s >= ns) break;
                if (!gv) continue;
                uint4 xp[8];
                const uint4* src = lds + (long long)s * 9 * G + g;
#pragma unroll
                for (int j = 0; j < 8; ++j) xp[j] = src[j * G];
                const float4 st = __builtin_bit_cast(float4, src[8 * G]);
#pragma unroll
                for (int p = 0; p < RPW; ++p) {
                    const int r = row0 + p * RPP;
                    if (r < L.H) {
                        if (!rec[s]) {
                            acc[p] += wt[s];  // NaN for an invalid expert id
                            continue;
                        }
                        const float d = (BITS == 4) ? group_dot_q4(M, c0[s][p], c1[s][p], xp)
                                                    : group_dot_q2(M, c0[s][p], xp);
                        const float part = fmaf(bf16_lo(sbv[s][p]) * st.z, d - st.x, bf16_hi(sbv[s][p]) * st.y);
                        acc[p] = fmaf(wt[s], part, acc[p]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int p = 0; p < RPW; ++p) {
        const float v = lane_group_sum(acc[p], LPR);
        const int r = row0 + p * RPP;
        if (gl == 0 && r < L.H) y[(long long)b * L.H + r] = v;
    }
}

int down_slots_per_round(const Layout& L)
{
    const int per_slot = 9 * L.Gi * 16;
    int sc = (64 * 1024) / per_slot;
    if (sc > DN_SC) sc = DN_SC;
    return sc;  // >= 1 for I <= 16384
}

void launch_down(const Layout& L, const void* slab, const uint4* hq, const float4* hst, const int32_t* idx,
                 const float* w, int B, int K, int E, float shared_w, float* y, hipStream_t s, Timing t)
{
    const int rpb = 4 * DN_RPW * (64 / lanes_per_row(L.Gi));
    const int sc = down_slots_per_round(L);
    const size_t lds = (size_t)sc * 9 * L.Gi * 16;
    dim3 grid((L.H + rpb - 1) / rpb, B);
    if (L.bits == 4)
        hipExtLaunchKernelGGL((k_down<4, DN_RPW>), grid, dim3(256), lds, s, t.start, t.stop, 0, (const uint8_t*)slab,
                              L, hq, hst, idx, w, K, E, shared_w, sc, y);
    else
        hipExtLaunchKernelGGL((k_down<2, DN_RPW>), grid, dim3(256), lds, s, t.start, t.stop, 0, (const uint8_t*)slab,
                              L, hq, hst, idx, w, K, E, shared_w, sc, y);
}

// ----------------------------------------------------------------------------
// RMS renorm between stacked layers
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ y, int H, float eps, float* __restrict__ x)
{
    __shared__ double part[4];
    const int b = blockIdx.x;
    const float* yb = y + (long long)b * H;
    double ss = 0.0;
    for (int c = threadIdx.x; c < H; c += 256) ss += (double)yb[c] * (double)yb[c];
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const double tot = part[0] + part[1] + part[2] + part[3];
    const float inv = (float)(1.0 / sqrt(tot / H + (double)eps));
    __syncthreads();
    for (int c = threadIdx.x; c < H; c += 256) x[(long long)b * H + c] = yb[c] * inv;
}

void launch_rmsnorm(const float* y, int B, int H, float eps, float* x, hipStream_t s)
{
    hipLaunchKernelGGL(k_rmsnorm, dim3(B), dim3(256), 0, s, y, H, eps, x);
}

}  // namespace moe
