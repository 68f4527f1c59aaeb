// grouped.hip - batched decode (B > 1 tokens per call): token -> expert grouping
// and MFMA dequant-GEMMs that read each active expert's weights once per call.
//
// Pages (titles as published):
//   [LLMAPIS] llmapis.com, "Flash-MoE：把 397B MoE 真正跑进消费级笔记本，意味着
//             '大模型本地化'开始从演示走向系统工程"
//   [MFFB]    f.mffb.com.cn, Flash-MoE article ("HN上281票 ... 8200行纯C代码 ...")
//
// The pages decode one token at a time and fetch only the experts the router
// selects ([LLMAPIS] section 深度分析; [MFFB] section Flash-MoE关键参数, about 27 MB
// of experts per layer and token).  With B tokens per call the tokens that select
// the same expert share its read: the B*K assignments are grouped by expert (a
// stable counting sort), every active expert's codes are dequantized once into
// fp16 MFMA operands, and the whole group of tokens is multiplied against them.
//
// Kernels:
//   k_router_tiled   fp64-accumulated logits of many tokens, split over H
//   k_topk_slices    sums the H-slice partials in a fixed order, then softmax / top-K;
//                    blocks beside the selecting ones write the token operands
//   k_group          stable counting sort of the assignments + the MFMA work list
//   k_prep_tokens    token activations -> fp16 MFMA operands + chunk sums (+ GEMV operands)
//   k_grouped_mfma   gate/up (+ SwiGLU) or down dequant-GEMM over (group, 128 rows, K chunk)
//   k_fixup          SwiGLU of gate/up tiles whose K chunks two blocks shared
//   k_gemv_gateup    gate/up (+ SwiGLU) of the small groups as integer (v_dot8) GEMVs
//   k_hconvert       h of every entry -> fp16 with the entry's power-of-two scale + group stats
//   k_gemv_down      down of the small groups as fp16 (v_dot2) GEMVs
//   k_combine        per-token routing-weighted sum of the down outputs
#include <hip/hip_ext.h>

#include <mutex>

#include "common.h"
#include "grouped.h"
#include "topk.h"

namespace moe {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));  // native vector: copies stay in registers

constexpr int GM_GROUP = 32;         // most tokens of one MFMA work-list group
#ifndef MOE_GV_TOKENS
#define MOE_GV_TOKENS 2
#endif
constexpr int GV_TOKENS = MOE_GV_TOKENS;  // an expert with fewer tokens than this runs as a GEMV group
constexpr int GV_GROUP = 2;  // most tokens of one GEMV group of an expert flagged as out of the matrix cores' range
// most tokens of any GEMV group when experts below gv_t tokens run as GEMV groups
__host__ __device__ constexpr int gv_max_tokens(int gv_t) { return gv_t - 1 > GV_GROUP ? gv_t - 1 : GV_GROUP; }
constexpr int GM_MAX_BLOCKS = 1024;  // most blocks of a stream-split launch
constexpr int GM_MAX_DEVICES = 64;   // devices whose launch shapes are cached

__device__ inline f4 mfma16(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }


// ----------------------------------------------------------------------------
// The MFMA token operand: v = x scaled by the power of two that puts the token's
// largest |x| in [2^13, 2^14); per chunk of 32 columns its mean rounded to fp16,
// m, and each element's deviation v - m rounded to fp16, in chunk order: element c
// lands in chunk P = (c / 32 % 2) * G + c / 64 (the code chunks' order in a row),
// dword dd = c % 32 / 8, at xh[(t * 2G + P) * 4 + dd] element (r % 4) * 2 + r / 4
// for r = c % 8 (the pair order the packed codes unpack to), so a step's 4 chunks
// are 256 contiguous bytes.  For the MFMA kernel's chunk term, xsum[t * 2G + P]
// holds the chunk's sum of the unrounded v, as fp16 hi + lo of 2^-5 times it, and
// the fp16 pair (2m, 2m).  The rounding error of an element is then relative to its
// deviation from the chunk mean, so a token whose elements are (nearly) equal does
// not carry one rounding error, of one sign, into every column of a row.
// ----------------------------------------------------------------------------
// 2^5: the chunk term's fp16 operands are 2^5 b, 2^5 * 8 s and 2^-5 * chunk sum
constexpr float GM_CT = 32.f;

__device__ inline int token_exponent(float amax)
{
    int e = 0;
    if (amax > 0.f && amax <= 3.4e38f) {
        e = ilogbf(amax) - 13;
        e = e < -110 ? -110 : (e > 113 ? 113 : e);
    }
    return e;
}
__device__ inline uint32_t hi_lo_pair(float v)
{
    const _Float16 h = (_Float16)v, l = (_Float16)(v - (float)h);
    return __builtin_bit_cast(uint32_t, h2{h, l});
}
// Element c of token row xt; the 32 columns of a chunk must be 32 consecutive
// lanes of one wave, all calling together (c % 32 == lane % 32).
__device__ inline void token_operand(const float* __restrict__ xt, int c, float inv, int G, uint16_t* __restrict__ out,
                                     uint2* __restrict__ sums)
{
    const float v = xt[c] * inv;
    const int P = ((c >> 5) & 1) * G + (c >> 6), dd = (c >> 3) & 3, r = c & 7;
    const float sum = group_reduce(v, OpAdd(), 32);  // every lane of the chunk gets the same sum
    const _Float16 m = (_Float16)(sum * (1.f / 32.f));
    out[((long long)P * 4 + dd) * 8 + (r & 3) * 2 + (r >> 2)] = __builtin_bit_cast(uint16_t, (_Float16)(v - (float)m));
    if ((c & 31) == 0) {
        const _Float16 m2 = m + m;  // exact
        sums[P] = make_uint2(hi_lo_pair(sum * (1.f / GM_CT)), __builtin_bit_cast(uint32_t, h2{m2, m2}));
    }
}

// ----------------------------------------------------------------------------
// Logits of B tokens: a block computes a tile of 32 experts x 32 tokens over a
// 256-column slice of H; each thread keeps 2 x 2 outputs, accumulating the exact
// fp32 products in fp64.  partial[slice][b][e]; k_topk_slices adds the slices in
// slice order, so the logits do not depend on the launch.
// ----------------------------------------------------------------------------
constexpr int RT_E = 32, RT_B = 32, RT_SLICE = 256, RT_CHUNK = 64, RT_PITCH = RT_E + 2;

__global__ __launch_bounds__(256) void k_router_tiled(const float* __restrict__ x, int B, const float* __restrict__ W,
                                                      int H, int E, double* __restrict__ partial)
{
    __shared__ float ws[RT_CHUNK][RT_PITCH];
    __shared__ float xs[RT_CHUNK][RT_PITCH];
    const int e0 = blockIdx.x * RT_E, b0 = blockIdx.y * RT_B, split = blockIdx.z;
    const int tid = threadIdx.x;
    const int te = (tid & 15) * 2, tb = (tid >> 4) * 2;  // this thread's 2 experts x 2 tokens
    double a00 = 0.0, a01 = 0.0, a10 = 0.0, a11 = 0.0;
    const int c_begin = split * RT_SLICE, c_end = min(H, c_begin + RT_SLICE);  // H % 64 == 0
    for (int c0 = c_begin; c0 < c_end; c0 += RT_CHUNK) {
        // stage W[e0 .. e0+32)[c0 .. c0+64) and x[b0 .. b0+32)[c0 .. c0+64) as [column][row]
        float wv[8], xv[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int t = tid + 256 * q, r = t >> 6, c = t & 63;
            wv[q] = W[(long long)min(e0 + r, E - 1) * H + c0 + c];
            xv[q] = x[(long long)min(b0 + r, B - 1) * H + c0 + c];
        }
        __syncthreads();  // the previous chunk's reads are done
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int t = tid + 256 * q, r = t >> 6, c = t & 63;
            ws[c][r] = wv[q];
            xs[c][r] = xv[q];
        }
        __syncthreads();
#pragma unroll 16
        for (int c = 0; c < RT_CHUNK; ++c) {
            const float2 w2 = *reinterpret_cast<const float2*>(&ws[c][te]);
            const float2 x2 = *reinterpret_cast<const float2*>(&xs[c][tb]);
            const double w0 = w2.x, w1 = w2.y, x0 = x2.x, x1 = x2.y;
            a00 = fma(w0, x0, a00);
            a01 = fma(w0, x1, a01);
            a10 = fma(w1, x0, a10);
            a11 = fma(w1, x1, a11);
        }
    }
    double* out = partial + (long long)split * B * E;
    const int e = e0 + te, b = b0 + tb;
    if (e < E && b < B) out[(long long)b * E + e] = a00;
    if (e < E && b + 1 < B) out[(long long)(b + 1) * E + e] = a01;
    if (e + 1 < E && b < B) out[(long long)b * E + e + 1] = a10;
    if (e + 1 < E && b + 1 < B) out[(long long)(b + 1) * E + e + 1] = a11;
}

// Blocks (t, 0), one per token: the token's logits are the H-slice partials
// added in slice order, then the bias (a fixed order, so they do not depend on
// the launch); they go to LDS and wave 0 selects the top-K.  Beside them, when
// the FFNs need token operands: block (t, 1) writes token t's MFMA operand and
// chunk sums (as k_prep_tokens), blocks (t, y >= 2) its GEMV operand for the GEMV
// groups, one wave per group.  The selecting blocks alone would hold 64 CUs.
constexpr int TS_CHUNK = 16;       // slice loads in flight per thread
constexpr int TS_GEMV_BLOCKS = 4;  // blocks per token writing the GEMV operand

__global__ __launch_bounds__(512) void k_topk_slices(const double* __restrict__ partial, int nslice,
                                                     const float* __restrict__ bias, int B, int E, int K, int renorm,
                                                     int32_t* __restrict__ idx, float* __restrict__ w, TokenPrep P)
{
    __shared__ double lg[1024];  // E <= 1024
    __shared__ float red[8];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const float* xt = P.x + (long long)b * P.H;
    if (blockIdx.y == 1) {  // the MFMA operand and its chunk sums
        float m = 0.f;
        for (int c = tid; c < P.H; c += 512) m = fmaxf(m, fabsf(xt[c]));
        m = wave_max(m);
        if (lane == 0) red[wave] = m;
        __syncthreads();
        float amax = red[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) amax = fmaxf(amax, red[i]);
        const int e = token_exponent(amax);
        const float inv = exp2i_f(-e);
        if (tid == 0) P.xscale[b] = exp2i_f(e);
        const int G = P.H / 64;
        uint16_t* out = reinterpret_cast<uint16_t*>(P.xh + (long long)b * 2 * G * 4);
        for (int c = tid; c < P.H; c += 512) token_operand(xt, c, inv, G, out, P.xsum + (long long)b * 2 * G);
        return;
    }
    if (blockIdx.y >= 2) {  // the operand of the GEMV groups
        const int G = P.H / 64, step = 8 * (gridDim.y - 2);
        for (int g = (blockIdx.y - 2) * 8 + wave; g < G; g += step) prep_group<4>(P.x, G, b, g, lane, P.xq, P.xst);
        return;
    }
    const long long BE = (long long)B * E;
    for (int e = tid; e < E; e += 512) {
        const double* p = partial + (long long)b * E + e;
        double s = 0.0;
        for (int s0 = 0; s0 < nslice; s0 += TS_CHUNK) {
            double v[TS_CHUNK];
#pragma unroll
            for (int j = 0; j < TS_CHUNK; ++j) v[j] = p[min(s0 + j, nslice - 1) * BE];
#pragma unroll
            for (int j = 0; j < TS_CHUNK; ++j)
                if (s0 + j < nslice) s += v[j];
        }
        lg[e] = s + (bias ? (double)bias[e] : 0.0);
    }
    __syncthreads();
    if (tid >= 64) return;
    double lv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) lv[j] = lg[min(tid + 64 * j, E - 1)];
    int id;
    float wt;
    topk_select<32, 16>(lv, E, K, renorm, tid, id, wt);
    if (tid < K) {
        idx[(long long)b * K + tid] = id;
        w[(long long)b * K + tid] = wt;
    }
}

int router_splits(int H) { return (H + RT_SLICE - 1) / RT_SLICE; }

void launch_route_batched(const float* x, int B, const float* W, const float* bias, int H, int E, int K, int renorm,
                          double* partial, int32_t* idx, float* w, const TokenPrep& P, hipStream_t s, Timing t)
{
    const dim3 grid((E + RT_E - 1) / RT_E, (B + RT_B - 1) / RT_B, router_splits(H));
    hipExtLaunchKernelGGL(k_router_tiled, grid, dim3(256), 0, s, t.start, t.stop, 0, x, B, W, H, E, partial);
    TokenPrep Q = P;
    Q.x = x;
    Q.H = H;
    const int ny = 1 + (P.xh ? 1 + (P.xq ? TS_GEMV_BLOCKS : 0) : 0);  // selection, MFMA operand, GEMV operand
    hipLaunchKernelGGL(k_topk_slices, dim3(B, ny), dim3(512), 0, s, partial, router_splits(H), bias, B, E, K, renorm,
                       idx, w, Q);
}

// ----------------------------------------------------------------------------
// Grouping: stable counting sort of the B*K assignments (slot i = b*K + k holds
// expert idx[i]) by expert id, in one block.  The block counts the slots of
// every expert (LDS atomics) and scans the counts; then wave 0 walks the slots
// 64 at a time in slot order: lanes naming the same expert find each other with
// ballots over the id bits, take consecutive places after the expert's running
// position in lane order, and the last of them advances it.  Every expert's
// list therefore keeps slot order.  Slots whose id is outside [0, E) are left out.
//
// The work list of the MFMA kernels cuts every expert's entries into groups of
// at most GM_GROUP tokens (the shared expert's B entries first, then the routed
// experts by id), so that every group is one pass of the dequant-GEMM.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_group(const int32_t* __restrict__ idx, int B, int K, int E, int gv_t,
                                                 const int32_t* __restrict__ flags, GroupOut O)
{
    __shared__ int sidx[MOE_MAX_B * MOE_MAX_K];
    __shared__ int cnt[MOE_MAX_E];
    __shared__ int wsum[3][16];
    const int tid = threadIdx.x, lane = tid & 63;
    const int n = B * K;
    const bool work = O.grp_u != nullptr;
    for (int e = tid; e < E; e += 1024) cnt[e] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 1024) {
        const int e = idx[i];
        sidx[i] = e;
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
        else if (work) O.slot_pos[i] = -1;
    }
    __syncthreads();
    const int c = tid < E ? cnt[tid] : 0;
    // an expert with fewer than gv_t tokens is one GEMV group, a larger one is
    // cut into MFMA groups of at most GM_GROUP tokens; an expert flagged as holding
    // scales or biases beyond the matrix cores' range is cut into GEMV groups of at
    // most GV_GROUP tokens whatever its count (the GEMV applies them in fp32)
    const int gsz = gv_t > 1 ? GV_GROUP : 1;
    const bool fl = flags != nullptr && gv_t > 1 && tid < E && flags[tid] != 0;
    const int fm = (!fl && c >= gv_t) ? (c + GM_GROUP - 1) / GM_GROUP : 0;
    const int fg = fl ? (c + gsz - 1) / gsz : ((c > 0 && c < gv_t) ? 1 : 0);
    // exclusive scans of the counts and of both group counts over the block
    int sc = c, sm = fm, sg = fg;
    for (int off = 1; off < 64; off <<= 1) {
        const int oc = __shfl_up(sc, off, 64), om = __shfl_up(sm, off, 64), og = __shfl_up(sg, off, 64);
        if (lane >= off) {
            sc += oc;
            sm += om;
            sg += og;
        }
    }
    if (lane == 63) {
        wsum[0][tid >> 6] = sc;
        wsum[1][tid >> 6] = sm;
        wsum[2][tid >> 6] = sg;
    }
    __syncthreads();
    int pc = 0, pm = 0, pg = 0;
    for (int q = 0; q < (tid >> 6); ++q) {
        pc += wsum[0][q];
        pm += wsum[1][q];
        pg += wsum[2][q];
    }
    const int excl_c = pc + sc - c, excl_m = pm + sm - fm, excl_g = pg + sg - fg;
    // the shared expert (all B tokens, entries 0 .. B-1) leads its list
    const bool shared_gemv = B < gv_t || (flags != nullptr && gv_t > 1 && flags[E] != 0);
    const int vsm = shared_gemv ? 0 : (B + GM_GROUP - 1) / GM_GROUP, vsg = shared_gemv ? (B + gsz - 1) / gsz : 0;
    if (tid < E) {
        O.offsets[tid] = excl_c;
        cnt[tid] = excl_c;  // running position of expert tid
        if (work) {
            for (int j = 0; j < fm; ++j) {
                O.act_expert[vsm + excl_m + j] = tid;
                O.act_off[vsm + excl_m + j] = B + excl_c + j * GM_GROUP;
                O.act_n[vsm + excl_m + j] = min(GM_GROUP, c - j * GM_GROUP);
            }
            for (int j = 0; j < fg; ++j) {
                O.gv_expert[vsg + excl_g + j] = tid;
                O.gv_off[vsg + excl_g + j] = B + excl_c + j * gsz;
                O.gv_n[vsg + excl_g + j] = fl ? min(gsz, c - j * gsz) : c;
            }
        }
    }
    if (tid == E - 1) {
        O.offsets[E] = excl_c + c;
        if (work) {
            O.grp_u[0] = vsm + excl_m + fm;  // MFMA groups
            O.grp_u[1] = vsg + excl_g + fg;  // GEMV groups
        }
    }
    if (work) {
        for (int j = tid; j < vsm; j += 1024) {
            O.act_expert[j] = E;
            O.act_off[j] = j * GM_GROUP;
            O.act_n[j] = min(GM_GROUP, B - j * GM_GROUP);
        }
        for (int j = tid; j < vsg; j += 1024) {
            O.gv_expert[j] = E;
            O.gv_off[j] = j * gsz;
            O.gv_n[j] = min(gsz, B - j * gsz);
        }
        for (int b = tid; b < B; b += 1024) O.ent_token[b] = b;
    }
    __syncthreads();
    if (tid >= 64) return;
    const uint64_t lt = (1ull << lane) - 1ull;
    for (int base = 0; base < n; base += 64) {
        const int i = base + lane;
        const int e = i < n ? sidx[i] : -1;
        const bool ok = e >= 0 && e < E;
        uint64_t peers = __ballot(ok);
#pragma unroll
        for (int bit = 0; bit < 10; ++bit) {  // E <= 1024
            const uint64_t m = __ballot((e >> bit) & 1);
            peers &= ((e >> bit) & 1) ? m : ~m;
        }
        if (ok) {
            const int rank = __popcll(peers & lt);
            const int pos = cnt[e] + rank;
            O.tokens[pos] = i / K;
            O.slots[pos] = i;
            if (work) {
                O.ent_token[B + pos] = i / K;
                O.slot_pos[i] = B + pos;
            }
            if ((peers >> lane) == 1ull) cnt[e] = pos + 1;  // the last lane of the group
        }
    }
}

int gemv_tokens(const Layout& L) { return (L.bits == 4 && L.Gh <= 64 && L.Gi <= 64) ? GV_TOKENS : 1; }

void launch_group(const int32_t* idx, int B, int K, int E, int gv_tokens, const int32_t* flags, const GroupOut& O,
                  hipStream_t s)
{
    hipLaunchKernelGGL(k_group, dim3(1), dim3(1024), 0, s, idx, B, K, E, gv_tokens, flags, O);
}

// flags[e] = 1 if record e holds a group whose scale or bias the matrix-core path
// cannot take (|s| >= 256, |b| >= 2048, or not finite), else 0; one block per record.
// The scale/bias areas alternate (s, b) bf16 pairs, so element parity tells them apart.
__global__ __launch_bounds__(256) void k_expert_ranges(Layout L, const uint8_t* __restrict__ slab,
                                                       int32_t* __restrict__ flags)
{
    const uint8_t* rec = slab + (long long)blockIdx.x * L.record;
    const long long n_gu = (long long)L.I * L.Sh * 8 / 16, n_dn = (long long)L.H * L.Si * 4 / 16;
    const uint4* gu = reinterpret_cast<const uint4*>(rec + L.off_gu_sb);
    const uint4* dn = reinterpret_cast<const uint4*>(rec + L.off_d_sb);
    auto bad = [](uint4 v) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        int r = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float sc = fabsf(bf16_lo(w[k])), bi = fabsf(bf16_hi(w[k]));
            r |= !(sc < 256.f) || !(bi < 2048.f);  // also true for NaN
        }
        return r;
    };
    int any = 0;
    for (long long i = threadIdx.x; i < n_gu; i += 256) any |= bad(gu[i]);
    for (long long i = threadIdx.x; i < n_dn; i += 256) any |= bad(dn[i]);
    any = __syncthreads_or(any);
    if (threadIdx.x == 0) flags[blockIdx.x] = any ? 1 : 0;
}

void launch_expert_ranges(const Layout& L, const void* slab, int n, int32_t* flags, hipStream_t s)
{
    hipLaunchKernelGGL(k_expert_ranges, dim3(n), dim3(256), 0, s, L, (const uint8_t*)slab, flags);
}

// ----------------------------------------------------------------------------
// Token operands of the gate/up GEMM (token_operand: x * 2^-e in fp16, chunk
// order, and the chunk sums) when the caller brings the routing.
// ----------------------------------------------------------------------------

// Blocks (t, y >= 1) write token t's GEMV operand instead (the single-token
// kernels' 4-bit operand: digit planes of a per-group fixed point + group stats)
// for the GEMV groups, one wave per group.
constexpr int PT_GEMV_BLOCKS = 4;

__global__ __launch_bounds__(256) void k_prep_tokens(const float* __restrict__ x, int H, uint4* __restrict__ xh,
                                                     uint2* __restrict__ xsum, float* __restrict__ xscale,
                                                     uint4* __restrict__ xq, float4* __restrict__ xst)
{
    __shared__ float red[4];
    const int t = blockIdx.x, tid = threadIdx.x;
    if (blockIdx.y > 0) {
        const int G = H / 64, step = 4 * (gridDim.y - 1);
        for (int g = (blockIdx.y - 1) * 4 + (tid >> 6); g < G; g += step) prep_group<4>(x, G, t, g, tid & 63, xq, xst);
        return;
    }
    const float* xt = x + (long long)t * H;
    float m = 0.f;
    for (int c = tid; c < H; c += 256) m = fmaxf(m, fabsf(xt[c]));
    m = wave_max(m);
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const int e = token_exponent(amax);
    const float inv = exp2i_f(-e);
    if (tid == 0) xscale[t] = exp2i_f(e);
    const int G = H / 64;
    uint16_t* out = reinterpret_cast<uint16_t*>(xh + (long long)t * 2 * G * 4);
    for (int c = tid; c < H; c += 256) token_operand(xt, c, inv, G, out, xsum + (long long)t * 2 * G);
}

// ----------------------------------------------------------------------------
// Dword w of a 16-byte chunk of a 4-bit row (8 codes) -> the fp16 MFMA operand
// s * (q - 8) of its 8 weights in the order (c0, c4, c1, c5, c2, c6, c3, c7).
// OR-ing the fp16 pattern of 1024 into the masked code pair (c_t, c_t+4) gives
// (1024 + q_a, 1024 + q_b) for t = 0, 2 (mask 0x000F000F on w, on w >> 8) and
// (1024 + 16 q_a, 1024 + 16 q_b) for t = 1, 3 (mask 0x00F000F0): subtracting 1032,
// or scaling by 1/16 and subtracting 72, gives q - 8 exactly.  |q - 8| <= 8 has at
// most 3 significant bits and a bf16 scale at most 8, so the product fits fp16's
// 11 and is exact (for 2^-14 <= |s| < 2^13): the weights s*q + b = s*(q - 8) +
// (b + 8 s) reach the MFMA unrounded, the group's b + 8 s being added apart, times
// the token operand's chunk sum.
// ----------------------------------------------------------------------------
__device__ inline h8 dequant_dword_q4(uint32_t w, h2 s2, const Masks& M)
{
    const h2 k1032 = {(_Float16)1032.f, (_Float16)1032.f};
    const h2 k16 = {(_Float16)0.0625f, (_Float16)0.0625f}, k72 = {(_Float16)-72.f, (_Float16)-72.f};
    const uint32_t w8 = w >> 8;
    const h2 q0 = __builtin_bit_cast(h2, (w & M.m4a) | M.magic) - k1032;
    const h2 q1 = __builtin_elementwise_fma(__builtin_bit_cast(h2, (w & M.m4b) | M.magic), k16, k72);
    const h2 q2 = __builtin_bit_cast(h2, (w8 & M.m4a) | M.magic) - k1032;
    const h2 q3 = __builtin_elementwise_fma(__builtin_bit_cast(h2, (w8 & M.m4b) | M.magic), k16, k72);
    const h2 p0 = q0 * s2, p1 = q1 * s2, p2 = q2 * s2, p3 = q3 * s2;
    return h8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// 2-bit records: a group is one 16-byte chunk whose code k (column 64 g + k) sits
// at bits 2k, so the 32 columns of the 4-bit chunk (half h, group g) are the
// chunk's bytes 8h .. 8h + 7, and dword d of that 4-bit chunk (columns 8d .. 8d+7
// of the half) is the 16-bit field d of those 8 bytes.  Copying the field's high
// byte up by 8 bits puts codes r and r + 4 of the dword into the two 16-bit halves
// at bit 2r, so the 2-bit masks yield the pairs in the order the 4-bit unpacking
// gives (codes 0 and 4, 1 and 5, 2 and 6, 3 and 7); the fp16 values 1024 + 4^r q
// become q - 2 exactly (the 2-bit codes' centre, where the 4-bit ones use 8), and
// times s exactly.  The chunk term then carries b + 2 s.
__device__ inline h8 dequant_field_q2(uint32_t x16, h2 s2, const Masks& M)
{
    const h2 k1026 = {(_Float16)1026.f, (_Float16)1026.f};
    const h2 k4 = {(_Float16)0.25f, (_Float16)0.25f}, k258 = {(_Float16)-258.f, (_Float16)-258.f};
    const h2 k16 = {(_Float16)0.0625f, (_Float16)0.0625f}, k66 = {(_Float16)-66.f, (_Float16)-66.f};
    const h2 k64 = {(_Float16)0.015625f, (_Float16)0.015625f}, k18 = {(_Float16)-18.f, (_Float16)-18.f};
    const uint32_t y = x16 | (x16 << 8);
    const h2 q0 = __builtin_bit_cast(h2, (y & M.m2[0]) | M.magic) - k1026;
    const h2 q1 = __builtin_elementwise_fma(__builtin_bit_cast(h2, (y & M.m2[1]) | M.magic), k4, k258);
    const h2 q2 = __builtin_elementwise_fma(__builtin_bit_cast(h2, (y & M.m2[2]) | M.magic), k16, k66);
    const h2 q3 = __builtin_elementwise_fma(__builtin_bit_cast(h2, (y & M.m2[3]) | M.magic), k64, k18);
    const h2 p0 = q0 * s2, p1 = q1 * s2, p2 = q2 * s2, p3 = q3 * s2;
    return h8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// 3-bit records: the low two bits of a unit's codes form a 2-bit chunk, so field x16
// is taken as at 2 bits; the unit's high-bit dword hi[h] covers the 32 columns of
// 4-bit chunk half h.  For dword d of that half, high_bits_q3 moves the high bits of
// codes r and r + 4 (r < 4) next to their low fields, to bits 2r + 2 and 2r + 18 (the
// single-token order keeps them at bits 2i + 2 / 2i + 3 of the 16-bit half of the
// 16-column dword, i = the code's place in it), and dequant_field_q3 ORs them in:
// 1024 + 4^r q, then q - 4 exactly (the 3-bit codes' centre), times s exactly.  The
// chunk term carries b + 4 s.
__device__ inline uint32_t high_bits_q3(uint32_t W, int d)
{
    const uint32_t S = ((d >> 1) & 1) ? __builtin_amdgcn_alignbit(W, W, 8) : W;
    return (d & 1) ? (((S >> 16) & 0x154u) | ((S >> 1) & 0x1540000u)) : ((S & 0x154u) | ((S << 15) & 0x1540000u));
}

__device__ inline h8 dequant_field_q3(uint32_t x16, uint32_t hb, h2 s2, const Masks& M)
{
    const h2 k1028 = {(_Float16)1028.f, (_Float16)1028.f};
    const h2 k4 = {(_Float16)0.25f, (_Float16)0.25f}, k260 = {(_Float16)-260.f, (_Float16)-260.f};
    const h2 k16 = {(_Float16)0.0625f, (_Float16)0.0625f}, k68 = {(_Float16)-68.f, (_Float16)-68.f};
    const h2 k64 = {(_Float16)0.015625f, (_Float16)0.015625f}, k20 = {(_Float16)-20.f, (_Float16)-20.f};
    const uint32_t y = x16 | (x16 << 8);
    const h2 q0 = __builtin_bit_cast(h2, (y & M.m2[0]) | M.magic | (hb & M.m3[0])) - k1028;
    const h2 q1 = __builtin_elementwise_fma(__builtin_bit_cast(h2, (y & M.m2[1]) | M.magic | (hb & M.m3[1])), k4, k260);
    const h2 q2 = __builtin_elementwise_fma(__builtin_bit_cast(h2, (y & M.m2[2]) | M.magic | (hb & M.m3[2])), k16, k68);
    const h2 q3 = __builtin_elementwise_fma(__builtin_bit_cast(h2, (y & M.m2[3]) | M.magic | (hb & M.m3[3])), k64, k20);
    const h2 p0 = q0 * s2, p1 = q1 * s2, p2 = q2 * s2, p3 = q3 * s2;
    return h8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Sum over a lane's 32 codes of q - C (C = 8, 4, 2: the width's centre): 4-bit, the
// nibbles of 4 dwords; 2-bit, the crumbs of 2 dwords; 3-bit, those crumbs (the low
// bits) plus 4 per set high bit.  Byte sums by v_sad_u8 against zero.
template <int BITS, typename CW>
__device__ inline int code_sum_centered(const CW& c, uint32_t hi)
{
    uint32_t acc = 0u;
    if constexpr (BITS == 4) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            acc = __builtin_amdgcn_sad_u8(c[d] & 0x0F0F0F0Fu, 0u, acc);
            acc = __builtin_amdgcn_sad_u8((c[d] >> 4) & 0x0F0F0F0Fu, 0u, acc);
        }
        return (int)acc - 8 * 32;
    } else {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const uint32_t t = (c[d] & 0x33333333u) + ((c[d] >> 2) & 0x33333333u);  // nibbles: pair sums
            acc = __builtin_amdgcn_sad_u8(t & 0x0F0F0F0Fu, 0u, acc);
            acc = __builtin_amdgcn_sad_u8((t >> 4) & 0x0F0F0F0Fu, 0u, acc);
        }
        if constexpr (BITS == 3) return (int)acc + 4 * __builtin_popcount(hi) - 4 * 32;
        return (int)acc - 2 * 32;
    }
}

// The chunk term (b + 8 s) * sum: one MFMA per tile and step whose K slots of a
// lane's chunk hold (b', b', s', s') against (X_hi, X_lo, X_hi, X_lo), with
// b' = 2^5 b and s' = 2^5 * 8 s (exact in fp16 for |b| < 2^11 and |s| < 2^8) and
// X = 2^-5 * the token operand's sum over the chunk's 32 columns (below 2^15 for
// operands below 2^15), split into fp16 hi + lo.  The codes q - 8 average about
// zero, so the rounding of the token operand they multiply adds no error of one
// sign to every row; the part of each weight that does not average out, b + 8 s,
// meets the sum of the unrounded x (gate/up) or of the operand itself (down).

// ----------------------------------------------------------------------------
// Grouped dequant-GEMM.  A block of 8 waves owns a tile of 128 rows of one
// group's expert (16 rows per wave) and multiplies it by the group's tokens
// (at most 32: two 16-token MFMA tiles).  K advances 128 columns (4 chunks of
// 32 columns) per step: lane (i, kk) of a wave holds chunk gm_chunk(step, kk) of
// its row i (4-bit: 16 code bytes; 2-bit: the 8 bytes of a half group), turns it
// into the exact fp16 operand s*(q - 8) (2-bit: s*(q - 2)), and MFMA d (16 x 16 x
// 32) takes dword d of the four lanes' chunks against the token operands of the
// same 32 columns, staged in LDS as [tt][kk][token][d]; one more MFMA per step
// adds (b + 8 s) times each chunk's token-operand sum, staged beside them.  Both
// operands are stored in chunk order, so a step's 4 chunks of one token (x) or
// entry (h) are 256 contiguous bytes.
//
// Work split: the units (group, tile, K chunk) in that order are cut into
// gridDim.x equal contiguous ranges, one per block.  Gate/up tiles are whole
// units while they number at most one per block; beyond that each is cut into
// GM_KC_GATEUP K chunks so the ranges still balance, and a tile whose K chunks
// fall into two blocks is finished by k_fixup from the blocks' partial sums.
//
// Pipelining: each step first loads the next step's token operands (cache-
// resident) into registers, then the weights of step + 3 (HBM) into a 4-slot
// register ring; gfx9 counts outstanding vector loads in issue order, so the
// LDS hand-over waits only for the token operands and the weight loads stay in
// flight across the barrier.
//
// MODE_GATEUP: rows are gate/up row pairs; token operand x scaled per token by a
//   power of two and rounded to fp16, with the chunk sums of the unrounded x;
//   writes h = silu(g) * u of each entry in fp32 in the pair-layout order
//   hb[entry][dword d < 8][G_i][8].
// MODE_DOWN: rows are down rows (one K chunk per tile); token operand h scaled
//   per entry by a power of two and rounded to fp16; writes the entry's output
//   row part[entry][H] in fp32.
// ----------------------------------------------------------------------------
enum { MODE_GATEUP = 0, MODE_DOWN = 1 };
constexpr int GM_WAVES = 8, GM_ROWS = GM_WAVES * 16, GM_TT = 2, GM_THREADS = GM_WAVES * 64;
constexpr int GM_KC_GATEUP = 4;  // K chunks per gate/up tile when tiles outnumber the blocks

// K chunks per gate/up tile of a launch: whole tiles when every block gets at
// most one (no partial sums, nothing for k_fixup), else GM_KC_GATEUP so that the
// equal ranges still balance.  Uniform for the launch: both kernels derive it alike.
__device__ inline int gm_kc(int tiles_total, int nb) { return tiles_total <= nb ? 1 : GM_KC_GATEUP; }

struct GroupedArgs {
    const uint8_t* slab;
    Layout L;
    const int32_t* grp_u;
    const int32_t* act_expert;
    const int32_t* act_off;
    const int32_t* act_n;
    const int32_t* gv_expert;
    const int32_t* gv_off;
    const int32_t* gv_n;
    const int32_t* n_ent;   // offsets[E]: routed entries placed (entries B .. B + n_ent - 1)
    const int32_t* ent_token;
    const uint4* xh;        // gate/up operand: x * 2^-e(token) as fp16 in chunk order [token][2 G_h][4]
    const uint2* xsum;      // per chunk: 2^-5 * sum of x * 2^-e as fp16 (hi, lo), and the pair (2m, 2m)
    const float* xscale;
    float* hb;       // gate/up output: h in fp32, pair-layout order [entry][8][G_i][8]
    const uint4* hb16;     // down operand: h * 2^-e(entry) as fp16 pairs in chunk order [entry][2 G_i][4]
    const float* hscale;   // 2^e(entry)
    float* part;     // MODE_DOWN output
    float* split;    // MODE_GATEUP partial sums [2 * gridDim.x][2][GM_GROUP][GM_ROWS]
};

template <int MODE>
struct GmShape {
    static constexpr int NM = (MODE == MODE_GATEUP) ? 2 : 1;  // matrices per row: gate + up | down
    static constexpr int RING = (MODE == MODE_GATEUP) ? 3 : 4;  // weight ring slots (loads run RING-1 steps ahead)
    static constexpr int NSTG = GM_TT * 4 * 4 * 16;           // 16-byte token-operand elements staged per step
    static_assert(NSTG == GM_THREADS, "one staged element per thread");
    // LDS of a stage: rows (tt, k2, token) of 5 elements: the 4 dwords' operands, then
    // the chunk sum; the odd pitch keeps the reads of 16 tokens free of bank conflicts
    static constexpr int NLDS = GM_TT * 4 * 16 * 5;
};

__host__ __device__ inline int gm_tiles(const Layout& L, int mode) { return ((mode == MODE_GATEUP ? L.I : L.H) + GM_ROWS - 1) / GM_ROWS; }
__host__ __device__ inline int gm_steps(const Layout& L, int mode) { return (2 * (mode == MODE_GATEUP ? L.Gh : L.Gi) + 3) / 4; }
int grouped_tiles(const Layout& L, int down) { return gm_tiles(L, down ? MODE_DOWN : MODE_GATEUP); }
int grouped_gateup_chunks() { return GM_KC_GATEUP; }
int grouped_group_tokens() { return GM_GROUP; }
// first unit of block b when T units are cut into nb ranges (T * nb < 2^32)
__device__ inline int gm_lo(int b, int T, int nb) { return (int)(((uint32_t)b * (uint32_t)T) / (uint32_t)nb); }
// Logical index of block b of an nb-block launch.  The dispatcher deals blocks to
// the 8 XCDs in turn (block b to XCD b % 8); this gives each XCD a contiguous run of
// logical indices, so the consecutive units of one group (its tiles and K chunks,
// which all read the group's token operands) mostly run under one XCD's L2 instead
// of pulling the operands into all eight.  A bijection on [0, nb): XCD x holds
// blocks x, x + 8, ... and takes logical indices from the sum of the counts below x.
constexpr int GM_XCDS = 8, GM_RUN = 4;
__device__ inline int gm_logical(int b, int nb)
{
    // runs of GM_RUN logical indices per XCD, dealt in turn; a partial last round keeps b
    const int round = GM_XCDS * GM_RUN, full = nb - nb % round;
    if (b >= full) return b;
    const int base = b - b % round, j = b % round;  // j = position within the round: XCD j % 8, slot j / 8
    return base + (j % GM_XCDS) * GM_RUN + j / GM_XCDS;
}

// the block whose range holds unit x
__device__ inline int gm_blk(int x, int T, int nb)
{
    return (int)((((uint32_t)x + 1u) * (uint32_t)nb - 1u) / (uint32_t)T);
}

// h = silu(g * xs) * (u * xs) of entry ent at input column `row` of the down
// GEMM, stored in fp32 in the pair-layout order
__device__ inline void store_h(const GroupedArgs& A, int ent, int row, float g, float u, float xs)
{
    g *= xs;
    u *= xs;
    const float h = g / (1.f + __expf(-g)) * u;
    float* hrow = A.hb + (long long)ent * 64 * A.L.Gi;
    const int grp = row >> 6, cc = row & 63, dd = cc >> 3, r = cc & 7;
    hrow[((long long)dd * A.L.Gi + grp) * 8 + (r & 3) * 2 + (r >> 2)] = h;
}

// The chunk (4-bit chunk order P = h G + g: columns 64 g + 32 h .. + 31) that K slot k
// of step ks multiplies; past the row end, the last chunk with *pad set (zero weights).
// 4-bit: chunks 4 ks .. 4 ks + 3, 64 contiguous code bytes of a row.  2-bit: both halves
// of groups 2 ks and 2 ks + 1, 32 contiguous code bytes, so a row's 2-bit codes are read
// in order and each 128-byte line in consecutive steps.  The contraction does not depend
// on the order; the token operand of slot k is staged from the same chunk.
template <int BITS>
__device__ inline int gm_chunk(int ks, int k, int G, bool* pad)
{
    if (BITS == 4) {  // (3-bit rows: the low-bit chunks, in the 2-bit order)
        const int P = 4 * ks + k;
        *pad = P >= 2 * G;
        return min(P, 2 * G - 1);
    }
    const int g = 2 * ks + (k >> 1);
    *pad = g >= G;
    return (k & 1) * G + min(g, G - 1);
}

template <int MODE, int BITS>
__global__ __launch_bounds__(GM_THREADS) __attribute__((amdgpu_waves_per_eu(4))) void k_grouped_mfma(GroupedArgs A)
{
    using S = GmShape<MODE>;
    constexpr int NM = S::NM, RING = S::RING;
    __shared__ u4 bs[2][S::NLDS];

    const Layout& L = A.L;
    const int G = (MODE == MODE_GATEUP) ? L.Gh : L.Gi;
    const int NR = (MODE == MODE_GATEUP) ? L.I : L.H;
    const int tiles = gm_tiles(L, MODE);
    const int nsteps = gm_steps(L, MODE);
    const int nb = gridDim.x, blk = gm_logical(blockIdx.x, nb);
    const int KC = (MODE == MODE_GATEUP) ? gm_kc(A.grp_u[0] * tiles, nb) : 1;
    const int T = A.grp_u[0] * tiles * KC;
    const int lo = gm_lo(blk, T, nb), hi = gm_lo(blk + 1, T, nb);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i = lane & 15, kk = lane >> 4;
    const Masks M = load_masks();

    // a lane's codes of one chunk: 16 bytes (4-bit) or the 8 bytes of its half of a 2-bit chunk
    typedef uint32_t cw_t __attribute__((ext_vector_type(BITS == 4 ? 4 : 2)));
    struct WRegs {
        cw_t c[NM];
        uint32_t sb[NM];
        uint32_t hi[NM];  // 3-bit: the high-bit dword of the lane's 32 columns
    };

    for (int x = lo; x < hi;) {
        const int tau = x / KC, kc0 = x - tau * KC, kc1 = min(KC, kc0 + (hi - x));
        const int u = tau / tiles, tile = tau - u * tiles;
        const int k_begin = kc0 * nsteps / KC, k_end = kc1 * nsteps / KC;
        const int e = A.act_expert[u];
        const int ent0 = A.act_off[u], n = A.act_n[u];  // 1 <= n <= GM_GROUP
        const int ntt = (n + 15) / 16;
        // addresses: uniform base + 32-bit byte offset (a record, the token and h
        // operands are each far below 4 GiB)
        const uint8_t* rec = A.slab + (long long)e * L.record;
        const int row = min(tile * GM_ROWS + wave * 16 + i, NR - 1);
        const uint32_t row_off = (uint32_t)(row * 2 * L.hb);  // gate/up; down chunks go through d_chunk_off
        const uint32_t sb_off = (MODE == MODE_GATEUP) ? (uint32_t)(L.off_gu_sb + (long long)row * L.Sh * 8)
                                                      : (uint32_t)(L.off_d_sb + (long long)row * L.Si * 4);
        const uint32_t up_off = (uint32_t)L.hb;
        const char* tok_base = (MODE == MODE_GATEUP) ? (const char*)A.xh : (const char*)A.hb16;

        // Stage element t = threadIdx.x = ((tt*16 + j)*4 + k2)*4 + d: dword d of chunk
        // gm_chunk(step, k2) of the tile's token j (gate/up: x of the entry's token, down: h
        // of the entry), so 16 consecutive lanes read a step's 256 contiguous bytes of
        // one operand row.  It lands in LDS row (tt*4 + k2)*16 + j, whose last slot takes
        // the chunk sum for the chunk-term MFMA: gate/up loads the one the token-operand
        // writer stored; down adds the row's 4 elements across its 4 threads.  Chunks
        // past the row end (2G not a multiple of 4) read a valid chunk and get zero weights.
        const int st_d = threadIdx.x & 3, st_k2 = (threadIdx.x >> 2) & 3;
        const int st_row = (((threadIdx.x >> 8) * 4 + st_k2) * 16 + ((threadIdx.x >> 4) & 15)) * 5;
        int st_src, st_sum;
        {
            const int m = min((threadIdx.x >> 8) * 16 + ((threadIdx.x >> 4) & 15), n - 1);
            const int orow = (MODE == MODE_GATEUP) ? A.ent_token[ent0 + m] : ent0 + m;
            st_src = orow * 8 * G + st_d;
            st_sum = orow * 2 * G;
        }
        struct Stage {
            u4 v;
            uint2 cs;  // gate/up: the row's chunk sum and mean pair
        };
        auto stage_load = [&](int ks, Stage& S) {
            bool stpad;  // a padded slot stages a valid chunk; its weights are zero
            const int P = gm_chunk<BITS>(ks, st_k2, G, &stpad);
            (void)stpad;
            S.v = *reinterpret_cast<const u4*>(tok_base + (uint32_t)(st_src + P * 4) * 16u);
            if (MODE == MODE_GATEUP) S.cs = A.xsum[st_sum + P];
        };
        auto stage_store = [&](int buf, const Stage& S) {
            bs[buf][st_row + st_d] = S.v;
            uint2 cs;
            if (MODE == MODE_GATEUP) {
                cs = S.cs;
            } else {
                float sum = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) sum = dot2(S.v[e], 0x3C003C00u, sum);  // fp16 (1, 1)
                cs = make_uint2(hi_lo_pair(group_reduce(sum, OpAdd(), 4) * (1.f / GM_CT)), 0u);  // h: no mean term
            }
            if (st_d == 0) bs[buf][st_row + 4] = u4{cs.x, cs.y, 0u, 0u};
        };
        auto weight_load = [&](int ks, WRegs& W) {
            bool wpad;  // the step applies the zero weights of a padded slot
            const int P = gm_chunk<BITS>(ks, kk, G, &wpad), g = P >= G ? P - G : P;
            (void)wpad;
            // 4-bit: chunk P; 2-bit: half P / G of chunk g
            const uint32_t co = (BITS == 4) ? ((MODE == MODE_GATEUP) ? row_off + (uint32_t)P * 16u
                                                                     : (uint32_t)(L.off_d_codes + d_chunk_off(L, row, P)))
                                            : ((MODE == MODE_GATEUP) ? row_off + (uint32_t)g * 16u
                                                                     : (uint32_t)(L.off_d_codes + d_chunk_off(L, row, g))) +
                                                  (P >= G ? 8u : 0u);
            W.c[0] = *reinterpret_cast<const cw_t*>(rec + co);
            if constexpr (BITS == 3) {
                // the high-bit dword of half P / G of unit g
                const uint32_t ho = ((MODE == MODE_GATEUP)
                                         ? row_off + (uint32_t)(16 * G + 8 * g)
                                         : (uint32_t)(L.off_d_codes + d_chunk_off(L, row, G + (g >> 1)) + 8 * (g & 1))) +
                                    (P >= G ? 4u : 0u);
                W.hi[0] = *reinterpret_cast<const uint32_t*>(rec + ho);
                if (MODE == MODE_GATEUP) W.hi[NM - 1] = *reinterpret_cast<const uint32_t*>(rec + (ho + up_off));
            }
            if (MODE == MODE_GATEUP) {
                W.c[NM - 1] = *reinterpret_cast<const cw_t*>(rec + (co + up_off));
                const uint2 v = *reinterpret_cast<const uint2*>(rec + (sb_off + (uint32_t)(g >> L.gs) * 8u));
                W.sb[0] = v.x;
                W.sb[NM - 1] = v.y;
            } else {
                W.sb[0] = *reinterpret_cast<const uint32_t*>(rec + (sb_off + (uint32_t)(g >> L.gs) * 4u));
            }
        };

        // scale of this lane's output column in each token tile: the token's x scale
        // (gate/up) or the entry's h scale (down)
        float xs_lane[GM_TT];
#pragma unroll
        for (int tt = 0; tt < GM_TT; ++tt) {
            const int ent = ent0 + min(tt * 16 + i, n - 1);
            xs_lane[tt] = (MODE == MODE_GATEUP) ? A.xscale[A.ent_token[ent]] : A.hscale[ent];
        }

        f4 acc[NM][GM_TT];
#pragma unroll
        for (int mm = 0; mm < NM; ++mm)
#pragma unroll
            for (int tt = 0; tt < GM_TT; ++tt) acc[mm][tt] = f4{0.f, 0.f, 0.f, 0.f};

        // Step ks: token operands of step ks + 2 -> registers (Sp), weights of step
        // ks + RING - 1 -> the ring slot step ks - 1 used (Wp), multiply step ks
        // (weights Wc, token operands in LDS stage ks & 1), then store the token
        // operands of step ks + 1 (Sc, loaded one step earlier) into the other stage.
        // The loads are unconditional (past the segment end they repeat its last
        // step): the waits for them then stay exact, where a skipped load would make
        // every later wait assume nothing else is in flight and drain the ring.
        auto step = [&](int ks, const WRegs& Wc, WRegs& Wp, const Stage& Sc, Stage& Sp) {
            stage_load(min(ks + 2, k_end - 1), Sp);
            __builtin_amdgcn_sched_barrier(0);
            weight_load(min(ks + RING - 1, k_end - 1), Wp);
            __builtin_amdgcn_sched_barrier(0);
            const u4* buf = bs[(ks - k_begin) & 1];
            bool pad;  // chunk past the row end: zero weights
            (void)gm_chunk<BITS>(ks, kk, G, &pad);
            h2 s2[NM];
            h8 cw[NM];  // the chunk term's weight operand
#pragma unroll
            for (int mm = 0; mm < NM; ++mm) {
                const uint32_t sb = pad ? 0u : Wc.sb[mm];
                const float s = bf16_lo(sb);
                // the codes' centre: 8 (4-bit), 4 (3-bit) or 2 (2-bit), so q - C averages about zero
                constexpr float C = BITS == 4 ? 8.f : (BITS == 3 ? 4.f : 2.f);
                const _Float16 sh = (_Float16)s, bh = (_Float16)(bf16_hi(sb) * GM_CT), s8 = (_Float16)(s * (C * GM_CT));
                s2[mm] = h2{sh, sh};
                _Float16 qh = (_Float16)0.f, ql = (_Float16)0.f;
                if constexpr (MODE == MODE_GATEUP) {
                    // the token operand is the chunk mean m plus deviations: the mean's share,
                    // m * s * Q with Q = sum of (q - C) over the lane's 32 codes, rides in the
                    // chunk term as (Q s / 2) in fp16 hi + lo against (2m, 2m), all exact
                    const float qs = (float)code_sum_centered<BITS>(Wc.c[mm], BITS == 3 ? Wc.hi[mm] : 0u) * s * 0.5f;
                    qh = (_Float16)qs;
                    ql = (_Float16)(qs - (float)qh);
                }
                cw[mm] = h8{bh, bh, s8, s8, qh, ql, (_Float16)0.f, (_Float16)0.f};
            }
            // (b + 8 s) of each lane's chunk times the token operand's chunk sum
#pragma unroll
            for (int tt = 0; tt < GM_TT; ++tt) {
                if (tt < ntt) {
                    const int r = (tt * 4 + kk) * 16 + i;
                    const u4 cv = buf[r * 5 + 4];  // (chunk sum hi, lo; the mean pair)
                    const h8 bx = __builtin_bit_cast(h8, u4{cv.x, cv.x, cv.y, 0u});
#pragma unroll
                    for (int mm = 0; mm < NM; ++mm) acc[mm][tt] = mfma16(cw[mm], bx, acc[mm][tt]);
                }
            }
            // dword-major: the token operands of dword d + 1 are read from LDS while
            // the MFMAs of dword d run, and only one dword's weights are live
            h8 bv[2][GM_TT];
            auto bread = [&](int d, h8 (&b)[GM_TT]) {
#pragma unroll
                for (int tt = 0; tt < GM_TT; ++tt)
                    if (tt < ntt) b[tt] = __builtin_bit_cast(h8, buf[((tt * 4 + kk) * 16 + i) * 5 + d]);
            };
            bread(0, bv[0]);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                if (d + 1 < 4) bread(d + 1, bv[(d + 1) & 1]);
                h8 a[NM];
#pragma unroll
                for (int mm = 0; mm < NM; ++mm) {
                    if constexpr (BITS == 4)
                        a[mm] = dequant_dword_q4(Wc.c[mm][d], s2[mm], M);
                    else if constexpr (BITS == 3)
                        a[mm] = dequant_field_q3((d & 1) ? Wc.c[mm][d >> 1] >> 16 : Wc.c[mm][d >> 1] & 0xFFFFu,
                                                 high_bits_q3(Wc.hi[mm], d), s2[mm], M);
                    else
                        a[mm] = dequant_field_q2((d & 1) ? Wc.c[mm][d >> 1] >> 16 : Wc.c[mm][d >> 1] & 0xFFFFu, s2[mm], M);
                }
#pragma unroll
                for (int tt = 0; tt < GM_TT; ++tt) {
                    if (tt < ntt) {
#pragma unroll
                        for (int mm = 0; mm < NM; ++mm) acc[mm][tt] = mfma16(a[mm], bv[d & 1][tt], acc[mm][tt]);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (ks + 1 < k_end) {
                stage_store((ks + 1 - k_begin) & 1, Sc);
                __syncthreads();
            }
        };

        WRegs R0, R1, R2, R3;
        Stage S0, S1;
        {
            __syncthreads();  // LDS reads of the previous segment are done
            // a segment holds at least one step (grouped_supported: nsteps >= KC)
            stage_load(k_begin, S0);
            stage_load(min(k_begin + 1, k_end - 1), S1);
            __builtin_amdgcn_sched_barrier(0);
            weight_load(k_begin, R0);
            weight_load(min(k_begin + 1, k_end - 1), R1);
            if (RING == 4) weight_load(min(k_begin + 2, k_end - 1), R2);
            __builtin_amdgcn_sched_barrier(0);
            stage_store(0, S0);
            __syncthreads();
        }
        // token operands alternate between S1 (steps ks + 1 with ks even) and S0
        if (RING == 4) {
            for (int ks = k_begin; ks < k_end; ks += 4) {
                step(ks, R0, R3, S1, S0);
                if (ks + 1 >= k_end) break;
                step(ks + 1, R1, R0, S0, S1);
                if (ks + 2 >= k_end) break;
                step(ks + 2, R2, R1, S1, S0);
                if (ks + 3 >= k_end) break;
                step(ks + 3, R3, R2, S0, S1);
            }
        } else {
            for (int ks = k_begin; ks < k_end; ks += 6) {
                step(ks, R0, R2, S1, S0);
                if (ks + 1 >= k_end) break;
                step(ks + 1, R1, R0, S0, S1);
                if (ks + 2 >= k_end) break;
                step(ks + 2, R2, R1, S1, S0);
                if (ks + 3 >= k_end) break;
                step(ks + 3, R0, R2, S0, S1);
                if (ks + 4 >= k_end) break;
                step(ks + 4, R1, R0, S1, S0);
                if (ks + 5 >= k_end) break;
                step(ks + 5, R2, R1, S0, S1);
            }
        }

        // lane (i, kk) holds D[row 4*kk + v][token i] of each token tile
        const int rbase = tile * GM_ROWS + wave * 16 + 4 * kk;
        const bool whole = (kc0 == 0 && kc1 == KC);
        float* sp = nullptr;
        if (MODE == MODE_GATEUP && !whole)  // slot 2b: the block's first segment, 2b + 1: its last
            sp = A.split + (long long)(2 * blk + (x == lo ? 0 : 1)) * 2 * GM_GROUP * GM_ROWS;
#pragma unroll
        for (int tt = 0; tt < GM_TT; ++tt) {
            const int m = tt * 16 + i;
            if (tt >= ntt || m >= n) continue;
            const int ent = ent0 + m;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = rbase + v;
                if (r >= NR) continue;
                if (MODE == MODE_GATEUP) {
                    if (whole) {
                        store_h(A, ent, r, acc[0][tt][v], acc[NM - 1][tt][v], xs_lane[tt]);
                    } else {
                        const int rl = r - tile * GM_ROWS;
                        sp[(0 * GM_GROUP + m) * GM_ROWS + rl] = acc[0][tt][v];
                        sp[(1 * GM_GROUP + m) * GM_ROWS + rl] = acc[NM - 1][tt][v];
                    }
                } else {
                    A.part[(long long)ent * L.H + r] = xs_lane[tt] * acc[0][tt][v];
                }
            }
        }
        x += kc1 - kc0;
    }
}

// Gate/up tiles whose K chunks were split between blocks: sum the blocks'
// partial sums in K order, then SwiGLU.  Block b handles the tile in which its
// range starts, when that start is inside a tile and no lower block starts
// inside the same tile.
// Block-uniform; 256 threads.
__device__ inline void fixup_block(const GroupedArgs& A, int nb, int b)
{
    const int tiles = gm_tiles(A.L, MODE_GATEUP);
    const int KC = gm_kc(A.grp_u[0] * tiles, nb);
    if (KC == 1) return;  // whole tiles: nothing was split
    const int T = A.grp_u[0] * tiles * KC;
    const int s0 = gm_lo(b, T, nb);
    if (s0 >= T || s0 % KC == 0) return;
    const int tau = s0 / KC;
    if (gm_lo(b - 1, T, nb) > tau * KC) return;  // a lower block starts inside this tile
    const int u = tau / tiles, tile = tau - u * tiles;
    const int ent0 = A.act_off[u], n = A.act_n[u];
    const int b_lo = gm_blk(tau * KC, T, nb), b_hi = gm_blk((tau + 1) * KC - 1, T, nb);
    // the tile's partial slots in K order (at most KC blocks share a tile)
    int slots[GM_KC_GATEUP], ns = 0;
    for (int bb = b_lo; bb <= b_hi && ns < KC; ++bb) {
        const int l0 = gm_lo(bb, T, nb);
        if (l0 == gm_lo(bb + 1, T, nb)) continue;  // empty range
        slots[ns++] = (bb == b_lo && l0 < tau * KC) ? 2 * bb + 1 : 2 * bb;
    }
    __shared__ float xs_tok[GM_GROUP];
    if (threadIdx.x < n) xs_tok[threadIdx.x] = A.xscale[A.ent_token[ent0 + threadIdx.x]];
    __syncthreads();
    // 4 elements per thread and pass, their loads issued together
    for (int t0 = threadIdx.x; t0 < n * GM_ROWS; t0 += 4 * 256) {
        float g[4] = {0.f, 0.f, 0.f, 0.f}, up[4] = {0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < ns; ++j) {
            const float* sp = A.split + (long long)slots[j] * 2 * GM_GROUP * GM_ROWS;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int t = min(t0 + q * 256, n * GM_ROWS - 1);
                const int m = t / GM_ROWS, rl = t - m * GM_ROWS;
                g[q] += sp[(0 * GM_GROUP + m) * GM_ROWS + rl];
                up[q] += sp[(1 * GM_GROUP + m) * GM_ROWS + rl];
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int t = t0 + q * 256;
            const int m = t / GM_ROWS, rl = t - m * GM_ROWS;
            const int r = tile * GM_ROWS + rl;
            if (t < n * GM_ROWS && r < A.L.I) store_h(A, ent0 + m, r, g[q], up[q], xs_tok[m]);
        }
    }
    __syncthreads();  // xs_tok is free for the block's next tile
}

__global__ __launch_bounds__(256) void k_fixup(GroupedArgs A, int nb) { fixup_block(A, nb, blockIdx.x); }

// The down operand: each entry's h scaled by the power of two that puts its
// largest |h| in [2^14, 2^15), as fp16 pairs in chunk order (the 4 dwords of
// code chunk c = j * G_i + g, j = 0, 1, are the uint4 of pairs 16j .. 16j+15 of
// group g, so a down step's 4 chunks are contiguous), so a token whose h is tiny
// everywhere (saturated SiLU) keeps its relative precision; and, for the dot2
// GEMV, each group's stats (C = 1024 * sum_p (pair sum) / t(p), S = sum h, scale)
// of the rounded values.  One block per entry.
__global__ __launch_bounds__(256) void k_hconvert(const float* __restrict__ hb, const int32_t* __restrict__ n_ent,
                                                  int B, int I, uint4* __restrict__ hb16, float* __restrict__ hscale,
                                                  float4* __restrict__ hstats)
{
    __shared__ float red[4];
    __shared__ float poff[1024], psum[1024];  // per pair-layout uint4 (I <= 8192)
    const int ent = blockIdx.x;
    if (ent >= B + n_ent[0]) return;  // uniform for the block
    const int nu = I / 8, Gi = I / 64;  // pair-layout uint4 of the entry: [8][Gi]
    const float4* src = reinterpret_cast<const float4*>(hb) + (long long)ent * nu * 2;
    float m = 0.f;
    for (int u = threadIdx.x; u < nu; u += 256) m = fmaxf(m, absmax8(src[2 * u], src[2 * u + 1]));
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    const int e = h_exponent(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
    const float inv = exp2i_f(-e), sc = exp2i_f(e);
    for (int u = threadIdx.x; u < nu; u += 256) {
        const uint4 pv = h_pairs(src[2 * u], src[2 * u + 1], inv);
        const int j = u / Gi, gg = u - j * Gi;  // uint4 u = j * Gi + g holds pairs 4j .. 4j+3 of group g
        hb16[(long long)ent * nu + ((j >> 2) * Gi + gg) * 4 + (j & 3)] = pv;  // chunk order
        const uint32_t pr[4] = {pv.x, pv.y, pv.z, pv.w};
        float off = 0.f, sum = 0.f;
#pragma unroll
        for (int el = 0; el < 4; ++el) {
            const h2 hh = __builtin_bit_cast(h2, pr[el]);
            const float ps = (float)hh.x + (float)hh.y;
            off = fmaf(pair_class_inv(4, 4 * j + el), ps, off);
            sum += ps;
        }
        poff[u] = off;
        psum[u] = sum;
    }
    __syncthreads();
    for (int g = threadIdx.x; g < Gi; g += 256) {
        float off = 0.f, sum = 0.f;
        for (int j = 0; j < 8; ++j) {
            off += poff[j * Gi + g];
            sum += psum[j * Gi + g];
        }
        hstats[(long long)ent * Gi + g] = make_float4(1024.f * off, sc * sum, sc, 0.f);
    }
    if (threadIdx.x == 0) hscale[ent] = sc;
}

// ----------------------------------------------------------------------------
// Small groups (fewer than GV_TOKENS tokens): GEMVs, each weight row read once
// and multiplied by every token of the group; the matrix cores would pad such a
// group to 16 tokens.  Gate/up takes the single-token kernels' integer operand
// (xq / xst: digit planes, v_dot8 against the codes as signed nibbles); down
// takes the fp16 h the matrix cores also read, with the codes as exact fp16
// patterns (v_dot2) and the stats k_hconvert writes.  The group fold is the
// single-token kernels'.  Work items (group, block of rows) are cut
// into equal contiguous ranges, one per block.
// ----------------------------------------------------------------------------
constexpr int GV_WAVES = 4;
constexpr int GV_META = 32;  // most GEMV groups one block's item range may touch (the grid is sized for it)

// The block's groups (expert, first entry, tokens) in LDS, read once up front so
// that no wait on them ever drains the weight loads in flight.  Returns the
// first group of the range.
__device__ inline int gv_meta(const GroupedArgs& A, int lo, int hi, int rb, int (*meta)[GV_META])
{
    const int v0 = lo / rb, nv = min((hi - 1) / rb - v0 + 1, GV_META);
    if (threadIdx.x < nv) {
        meta[0][threadIdx.x] = A.gv_expert[v0 + threadIdx.x];
        meta[1][threadIdx.x] = A.gv_off[v0 + threadIdx.x];
        meta[2][threadIdx.x] = A.gv_n[v0 + threadIdx.x];
    }
    __syncthreads();
    return v0;
}

// Stage the group's n operand vectors in LDS: per vector 8*G uint4 of pairs
// (vector m's pairs at pairs[m*8*G ..]) then G float4 stats.
__device__ inline void gv_stage(uint4* lds, int n, int G, const int32_t* vec_of, int vec0, const uint4* pairs,
                                const float4* stats)
{
    const int nx = 9 * G;
    for (int t = threadIdx.x; t < n * nx; t += 64 * GV_WAVES) {
        const int m = t / nx, k = t - m * nx;
        const long long vec = vec_of ? vec_of[vec0 + m] : vec0 + m;
        lds[t] = k < 8 * G ? pairs[vec * 8 * G + k] : __builtin_bit_cast(uint4, stats[vec * G + (k - 8 * G)]);
    }
}

// One lane's share of a gate/up row pair (gate codes, up codes, scales) or of a down row.
struct GvGateUp {
    uint4 c[4];
    uint2 sb;
};
struct GvDown {
    uint4 c[2];
    uint32_t sb;
};

// gate/up of the small groups: h = silu(W_g x) * (W_u x) per token of the group.
// Work item = (group, GV_WAVES row passes); each block walks a contiguous range of
// items, the next item's weights in flight while the current one is computed.
__global__ __launch_bounds__(64 * GV_WAVES) void k_gemv_gateup(GroupedArgs A, const uint4* __restrict__ xq,
                                                               const float4* __restrict__ xst, int nb_fix)
{
    static_assert(64 * GV_WAVES == 256, "the split-tile fixup runs on 256-thread blocks");
    // first the MFMA launch's split-tile fixups (nothing when its tiles were whole)
    for (int fb = blockIdx.x; fb < nb_fix; fb += gridDim.x) fixup_block(A, nb_fix, fb);
    extern __shared__ uint4 xs[];  // [n][9*G]
    const Layout& L = A.L;
    const int G = L.Gh, LPR = lanes_per_row(G), RPP = 64 / LPR;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane / LPR, gl = lane & (LPR - 1);
    const bool gv = gl < G;
    const int g = gv ? gl : G - 1;
    const int rows_pi = GV_WAVES * RPP;
    const int rb = (L.I + rows_pi - 1) / rows_pi;
    const int T = A.grp_u[1] * rb;
    const int lo = gm_lo(blockIdx.x, T, gridDim.x), hi = gm_lo(blockIdx.x + 1, T, gridDim.x);
    if (lo >= hi) return;  // uniform for the block
    __shared__ int meta[3][GV_META];
    const int v0 = gv_meta(A, lo, hi, rb, meta);
    auto mv = [&](int f, int v) { return __builtin_amdgcn_readfirstlane(meta[f][min(v - v0, GV_META - 1)]); };
    const Masks M = load_masks();
    // loads are unconditional (item and row clamped) so that waits stay exact
    auto load = [&](GvGateUp& w, int it) {
        it = min(it, hi - 1);
        const int v = it / rb;
        const int r = min((it - v * rb) * rows_pi + wave * RPP + sub, L.I - 1);
        const uint8_t* rec = A.slab + (long long)mv(0, v) * L.record;
        const uint8_t* base = rec + (long long)r * 2 * L.hb;
        w.c[0] = *reinterpret_cast<const uint4*>(base + g * 16);
        w.c[1] = *reinterpret_cast<const uint4*>(base + (G + g) * 16);
        w.c[2] = *reinterpret_cast<const uint4*>(base + L.hb + g * 16);
        w.c[3] = *reinterpret_cast<const uint4*>(base + L.hb + (G + g) * 16);
        w.sb = *reinterpret_cast<const uint2*>(rec + L.off_gu_sb + ((long long)r * L.Sh + (g >> L.gs)) * 8);
    };
    int v_prev = -1;
    auto work = [&](const GvGateUp& w, int it, GvGateUp& next) {
        const int v = it / rb;
        const int ent0 = mv(1, v), n = mv(2, v);
        if (v != v_prev) {    // uniform: every thread walks the same items
            __syncthreads();  // every wave is done with the previous group's operands
            gv_stage(xs, n, G, A.ent_token, ent0, xq, xst);
            __syncthreads();
            v_prev = v;
        }
        load(next, it + 1);
        const int r = (it - v * rb) * rows_pi + wave * RPP + sub;
        for (int m = 0; m < n; ++m) {
            const uint4* xv = xs + m * 9 * G;
            uint4 xp[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) xp[j] = xv[j * G + g];
            const float4 st = __builtin_bit_cast(float4, xv[8 * G + g]);
            float ga = fmaf(bf16_lo(w.sb.x) * st.z, group_dot_q4(M, w.c[0], w.c[1], xp) - st.x, bf16_hi(w.sb.x) * st.y);
            float ua = fmaf(bf16_lo(w.sb.y) * st.z, group_dot_q4(M, w.c[2], w.c[3], xp) - st.x, bf16_hi(w.sb.y) * st.y);
            ga = lane_group_sum(gv ? ga : 0.f, LPR);
            ua = lane_group_sum(gv ? ua : 0.f, LPR);
            if (gl == 0 && r < L.I) store_h(A, ent0 + m, r, ga, ua, 1.f);
        }
    };
    GvGateUp wa, wb;
    load(wa, lo);
    for (int it = lo; it < hi; it += 2) {
        work(wa, it, wb);
        if (it + 1 >= hi) break;
        work(wb, it + 1, wa);
    }
}

// down of the small groups: part[entry] = W_d h_entry, h as the scaled fp16
// pairs and per-group stats written by k_hconvert.
__global__ __launch_bounds__(64 * GV_WAVES) void k_gemv_down(GroupedArgs A, const float4* __restrict__ hstats)
{
    extern __shared__ uint4 hs[];  // [n][9*G]
    const Layout& L = A.L;
    const int G = L.Gi, LPR = lanes_per_row(G), RPP = 64 / LPR;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane / LPR, gl = lane & (LPR - 1);
    const bool gv = gl < G;
    const int g = gv ? gl : G - 1;
    const int rows_pi = GV_WAVES * RPP;
    const int rb = (L.H + rows_pi - 1) / rows_pi;
    const int T = A.grp_u[1] * rb;
    const int lo = gm_lo(blockIdx.x, T, gridDim.x), hi = gm_lo(blockIdx.x + 1, T, gridDim.x);
    if (lo >= hi) return;
    __shared__ int meta[3][GV_META];
    const int v0 = gv_meta(A, lo, hi, rb, meta);
    auto mv = [&](int f, int v) { return __builtin_amdgcn_readfirstlane(meta[f][min(v - v0, GV_META - 1)]); };
    const Masks M = load_masks();
    auto load = [&](GvDown& w, int it) {
        it = min(it, hi - 1);
        const int v = it / rb;
        const int r = min((it - v * rb) * rows_pi + wave * RPP + sub, L.H - 1);
        const uint8_t* rec = A.slab + (long long)mv(0, v) * L.record;
        const uint8_t* base = rec + L.off_d_codes;
        w.c[0] = *reinterpret_cast<const uint4*>(base + d_chunk_off(L, r, g));
        w.c[1] = *reinterpret_cast<const uint4*>(base + d_chunk_off(L, r, G + g));
        w.sb = *reinterpret_cast<const uint32_t*>(rec + L.off_d_sb + ((long long)r * L.Si + (g >> L.gs)) * 4);
    };
    int v_prev = -1;
    auto work = [&](const GvDown& w, int it, GvDown& next) {
        const int v = it / rb;
        const int ent0 = mv(1, v), n = mv(2, v);
        if (v != v_prev) {
            __syncthreads();
            gv_stage(hs, n, G, nullptr, ent0, A.hb16, hstats);
            __syncthreads();
            v_prev = v;
        }
        load(next, it + 1);
        const int r = (it - v * rb) * rows_pi + wave * RPP + sub;
        for (int m = 0; m < n; ++m) {
            const uint4* hv = hs + m * 9 * G;
            uint4 hp[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) hp[j] = hv[((j >> 2) * G + g) * 4 + (j & 3)];
            const float4 sv = __builtin_bit_cast(float4, hv[8 * G + g]);
            float acc = fmaf(bf16_lo(w.sb) * sv.z, group_dot_q4_f16(M, w.c[0], w.c[1], hp) - sv.x, bf16_hi(w.sb) * sv.y);
            acc = lane_group_sum(gv ? acc : 0.f, LPR);
            if (gl == 0 && r < L.H) A.part[(long long)(ent0 + m) * L.H + r] = acc;
        }
    };
    GvDown wa, wb;
    load(wa, lo);
    for (int it = lo; it < hi; it += 2) {
        work(wa, it, wb);
        if (it + 1 >= hi) break;
        work(wb, it + 1, wa);
    }
}

// y[t][r] = sum_k w[t][k] * part[entry of slot t*K+k][r] + shared_w * part[t][r],
// in slot order with the shared expert last; a slot whose expert id was invalid
// makes the token's row NaN.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ part, const int32_t* __restrict__ slot_pos,
                                                 const float* __restrict__ w, int K, int H, float shared_w,
                                                 float* __restrict__ y)
{
    const int t = blockIdx.y;
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= H) return;
    float acc = 0.f;
    for (int k = 0; k < K; ++k) {
        const int pos = slot_pos[t * K + k];
        const float v = part[(long long)max(pos, 0) * H + r];
        acc = (pos >= 0) ? fmaf(w[t * K + k], v, acc) : __builtin_nanf("");
    }
    y[(long long)t * H + r] = fmaf(shared_w, part[(long long)t * H + r], acc);
}

bool grouped_supported(const Layout& L, int B, int K)
{
    // every gate/up K chunk of a tile must hold at least one step (H >= 448)
    return (L.bits >= 2 && L.bits <= 4) && B >= 2 && B <= MOE_MAX_B && K <= MOE_MAX_K && L.H % 64 == 0 && L.I % 64 == 0 &&
           gm_steps(L, MODE_GATEUP) >= GM_KC_GATEUP;
}

// most work-list groups of either list a call can produce: the shared expert's B entries
// and every expert's entries cut into GEMV groups of at most 2 (experts flagged as out of the
// matrix cores' range) or into MFMA groups of at most GM_GROUP
static int max_groups(int B, int K, int E) { return (B + 1) / 2 + min(E, B * K) + (B * K + 1) / 2 + 1; }

size_t grouped_workspace_bytes(const Layout& L, int B, int K, int E)
{
    const size_t ents = (size_t)B * K + B, V = max_groups(B, K, E);
    size_t n = 0;
    auto add = [&](size_t bytes) { n += (bytes + 255) & ~(size_t)255; };
    add(sizeof(double) * router_splits(L.H) * B * E);  // partial logits
    add(sizeof(int32_t) * (E + 1));                    // offsets
    add(sizeof(int32_t) * B * K);                      // tokens
    add(sizeof(int32_t) * B * K);                      // slots
    add(sizeof(int32_t) * 4);                          // number of groups
    for (int l = 0; l < 6; ++l) add(sizeof(int32_t) * V);  // act_expert, act_off, act_n, gv_expert, gv_off, gv_n
    add(sizeof(int32_t) * ents);                       // ent_token
    add(sizeof(int32_t) * B * K);                      // slot_pos
    add(16ull * B * 2 * L.Gh * 4);                     // xh
    add(8ull * B * 2 * L.Gh);                          // xsum
    add(sizeof(float) * B);                            // xscale
    add(4ull * ents * L.I);                            // hb (fp32)
    add(2ull * ents * L.I);                            // hb16
    add(sizeof(float) * ents);                         // hscale
    add(16ull * ents * L.Gi);                          // hstats
    add(sizeof(float) * ents * L.H);                   // part
    add(sizeof(float) * 2ull * GM_MAX_BLOCKS * 2 * GM_GROUP * GM_ROWS);  // split tiles
    return n;
}

GroupedWork carve_grouped(void* base, const Layout& L, int B, int K, int E)
{
    const size_t ents = (size_t)B * K + B, V = max_groups(B, K, E);
    char* p = (char*)base;
    auto take = [&](size_t bytes) {
        char* r = p;
        p += (bytes + 255) & ~(size_t)255;
        return (void*)r;
    };
    GroupedWork W;
    W.partial = (double*)take(sizeof(double) * router_splits(L.H) * B * E);
    W.g.offsets = (int32_t*)take(sizeof(int32_t) * (E + 1));
    W.g.tokens = (int32_t*)take(sizeof(int32_t) * B * K);
    W.g.slots = (int32_t*)take(sizeof(int32_t) * B * K);
    W.g.grp_u = (int32_t*)take(sizeof(int32_t) * 4);
    W.g.act_expert = (int32_t*)take(sizeof(int32_t) * V);
    W.g.act_off = (int32_t*)take(sizeof(int32_t) * V);
    W.g.act_n = (int32_t*)take(sizeof(int32_t) * V);
    W.g.gv_expert = (int32_t*)take(sizeof(int32_t) * V);
    W.g.gv_off = (int32_t*)take(sizeof(int32_t) * V);
    W.g.gv_n = (int32_t*)take(sizeof(int32_t) * V);
    W.g.ent_token = (int32_t*)take(sizeof(int32_t) * ents);
    W.g.slot_pos = (int32_t*)take(sizeof(int32_t) * B * K);
    W.xh = (uint4*)take(16ull * B * 2 * L.Gh * 4);
    W.xsum = (uint2*)take(8ull * B * 2 * L.Gh);
    W.xscale = (float*)take(sizeof(float) * B);
    W.hb = (float*)take(4ull * ents * L.I);
    W.hb16 = (uint4*)take(2ull * ents * L.I);
    W.hscale = (float*)take(sizeof(float) * ents);
    W.hstats = (float4*)take(16ull * ents * L.Gi);
    W.part = (float*)take(sizeof(float) * ents * L.H);
    W.split = (float*)take(sizeof(float) * 2ull * GM_MAX_BLOCKS * 2 * GM_GROUP * GM_ROWS);
    return W;
}

// blocks of the stream split: as many as stay resident together (the work is cut
// into equal ranges, so all of them must run at once), at most GM_MAX_BLOCKS
static int resident_blocks(int dev, const void* kernel, int threads)
{
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1)
        per_cu = 1;
    return max(1, min(GM_MAX_BLOCKS, cus * per_cu));
}

// Block counts of the four stream-split launches on the calling thread's current
// device.  Computed once per device under a lock and only then published, so a
// thread never sees a partly filled entry; callers on several threads and devices
// are safe.
GroupedBlocks grouped_blocks()
{
    static std::mutex mu;
    static GroupedBlocks cache[GM_MAX_DEVICES];
    static bool filled[GM_MAX_DEVICES];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    const int slot = dev < GM_MAX_DEVICES ? dev : -1;
    std::lock_guard<std::mutex> lock(mu);
    if (slot >= 0 && filled[slot]) return cache[slot];
    GroupedBlocks n;
    n.gateup = resident_blocks(dev, (const void*)k_grouped_mfma<MODE_GATEUP, 4>, GM_THREADS);
    n.down = resident_blocks(dev, (const void*)k_grouped_mfma<MODE_DOWN, 4>, GM_THREADS);
    n.gateup2 = resident_blocks(dev, (const void*)k_grouped_mfma<MODE_GATEUP, 2>, GM_THREADS);
    n.down2 = resident_blocks(dev, (const void*)k_grouped_mfma<MODE_DOWN, 2>, GM_THREADS);
    n.gateup3 = resident_blocks(dev, (const void*)k_grouped_mfma<MODE_GATEUP, 3>, GM_THREADS);
    n.down3 = resident_blocks(dev, (const void*)k_grouped_mfma<MODE_DOWN, 3>, GM_THREADS);
    n.gemv_gateup = resident_blocks(dev, (const void*)k_gemv_gateup, 64 * GV_WAVES);
    n.gemv_down = resident_blocks(dev, (const void*)k_gemv_down, 64 * GV_WAVES);
    if (slot >= 0) {
        cache[slot] = n;
        filled[slot] = true;
    }
    return n;
}

void launch_ffn_grouped(const Layout& L, const void* slab, const GroupedWork& W, const float* x, const float* w,
                        float shared_w, int B, int K, int E, uint4* xq, float4* xst, bool prepped, float* y,
                        hipStream_t s, Timing tg, Timing td)
{
    const GroupedBlocks nb = grouped_blocks();
    const int nb_gu = L.bits == 2 ? nb.gateup2 : (L.bits == 3 ? nb.gateup3 : nb.gateup);
    const int nb_dn = L.bits == 2 ? nb.down2 : (L.bits == 3 ? nb.down3 : nb.down);
    const int nb_gvu = nb.gemv_gateup, nb_gvd = nb.gemv_down;
    const int gv_t = gemv_tokens(L);
    const bool gv = gv_t > 1;

    if (!prepped)
        hipLaunchKernelGGL(k_prep_tokens, dim3(B, gv ? 1 + PT_GEMV_BLOCKS : 1), dim3(256), 0, s, x, L.H, W.xh,
                           W.xsum, W.xscale, xq, xst);
    GroupedArgs A;
    A.slab = (const uint8_t*)slab;
    A.L = L;
    A.grp_u = W.g.grp_u;
    A.act_expert = W.g.act_expert;
    A.act_off = W.g.act_off;
    A.act_n = W.g.act_n;
    A.gv_expert = W.g.gv_expert;
    A.gv_off = W.g.gv_off;
    A.gv_n = W.g.gv_n;
    A.n_ent = W.g.offsets + E;
    A.ent_token = W.g.ent_token;
    A.xh = W.xh;
    A.xsum = W.xsum;
    A.xscale = W.xscale;
    A.hb = W.hb;
    A.hb16 = W.hb16;
    A.hscale = W.hscale;
    A.part = W.part;
    A.split = W.split;
    // the GEMV groups' operands in LDS: up to gv_max_tokens vectors of 9 * G uint4
    const int gv_n = gv ? gv_max_tokens(gv_t) : 0;
    const size_t lds_gu = 16ull * 9 * L.Gh * gv_n, lds_dn = 16ull * 9 * L.Gi * gv_n;
    // a block's item range spans at most ceil(V / nb) + 1 groups: keep that below GV_META
    const int v_max = max_groups(B, K, E), nb_meta = (v_max + GV_META - 3) / (GV_META - 2);
    const int nbu = max(nb_gvu, nb_meta), nbd = max(nb_gvd, nb_meta);

    // gate/up phase, timed as a whole (MFMA groups, split-tile fixup, GEMV groups):
    // together they read every active expert's gate/up rows once
    if (tg.start) (void)hipEventRecord(tg.start, s);
    if (L.bits == 2)
        hipLaunchKernelGGL((k_grouped_mfma<MODE_GATEUP, 2>), dim3(nb_gu), dim3(GM_THREADS), 0, s, A);
    else if (L.bits == 3)
        hipLaunchKernelGGL((k_grouped_mfma<MODE_GATEUP, 3>), dim3(nb_gu), dim3(GM_THREADS), 0, s, A);
    else
        hipLaunchKernelGGL((k_grouped_mfma<MODE_GATEUP, 4>), dim3(nb_gu), dim3(GM_THREADS), 0, s, A);
    if (gv)  // the GEMV kernel runs the split-tile fixups first
        hipLaunchKernelGGL(k_gemv_gateup, dim3(nbu), dim3(64 * GV_WAVES), lds_gu, s, A, (const uint4*)xq,
                           (const float4*)xst, nb_gu);
    else
        hipLaunchKernelGGL(k_fixup, dim3(nb_gu), dim3(256), 0, s, A, nb_gu);
    if (tg.stop) (void)hipEventRecord(tg.stop, s);

    hipLaunchKernelGGL(k_hconvert, dim3(B * K + B), dim3(256), 0, s, W.hb, A.n_ent, B, L.I, W.hb16, W.hscale,
                       W.hstats);

    // down phase, timed as a whole
    if (td.start) (void)hipEventRecord(td.start, s);
    if (L.bits == 2)
        hipLaunchKernelGGL((k_grouped_mfma<MODE_DOWN, 2>), dim3(nb_dn), dim3(GM_THREADS), 0, s, A);
    else if (L.bits == 3)
        hipLaunchKernelGGL((k_grouped_mfma<MODE_DOWN, 3>), dim3(nb_dn), dim3(GM_THREADS), 0, s, A);
    else
        hipLaunchKernelGGL((k_grouped_mfma<MODE_DOWN, 4>), dim3(nb_dn), dim3(GM_THREADS), 0, s, A);
    if (gv) hipLaunchKernelGGL(k_gemv_down, dim3(nbd), dim3(64 * GV_WAVES), lds_dn, s, A, (const float4*)W.hstats);
    if (td.stop) (void)hipEventRecord(td.stop, s);
    hipLaunchKernelGGL(k_combine, dim3((L.H + 255) / 256, B), dim3(256), 0, s, W.part, W.g.slot_pos, w, K, L.H,
                       shared_w, y);
}

}  // namespace moe
