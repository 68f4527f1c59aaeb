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
//   k_topk_split     sums the split partials in a fixed order, then top-K
//   k_group          stable counting sort of the assignments + the MFMA work list
//   k_prep_tokens    token activations -> fp16 hi + lo MFMA operands
//   k_grouped_mfma   gate/up (+ SwiGLU) or down dequant-GEMM per (expert, 128 rows)
//   k_combine        per-token routing-weighted sum of the down outputs
#include <hip/hip_ext.h>

#include "common.h"
#include "grouped.h"
#include "topk.h"

namespace moe {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));  // native vector: copies stay in registers

__device__ inline f4 mfma16(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// ----------------------------------------------------------------------------
// Logits of B tokens: a block computes a tile of 32 experts x 32 tokens over a
// 512-column slice of H; each thread keeps 2 x 2 outputs, accumulating the exact
// fp32 products in fp64.  partial[split][b][e]; k_topk_split adds the slices in
// slice order, so the logits do not depend on the launch.
// ----------------------------------------------------------------------------
constexpr int RT_E = 32, RT_B = 32, RT_SLICE = 512, RT_CHUNK = 64;

__global__ __launch_bounds__(256) void k_router_tiled(const float* __restrict__ x, int B, const float* __restrict__ W,
                                                      int H, int E, double* __restrict__ partial)
{
    __shared__ float ws[RT_CHUNK][RT_E + 1];
    __shared__ float xs[RT_CHUNK][RT_B + 1];
    const int e0 = blockIdx.x * RT_E, b0 = blockIdx.y * RT_B, split = blockIdx.z;
    const int tid = threadIdx.x;
    const int te = (tid & 15) * 2, tb = (tid >> 4) * 2;  // this thread's 2 experts x 2 tokens
    double acc[2][2] = {{0.0, 0.0}, {0.0, 0.0}};
    const int c_begin = split * RT_SLICE, c_end = min(H, c_begin + RT_SLICE);
    for (int c0 = c_begin; c0 < c_end; c0 += RT_CHUNK) {
        // stage W[e0 .. e0+32)[c0 .. c0+64) and x[b0 .. b0+32)[c0 .. c0+64) as [column][row]
        for (int t = tid; t < RT_CHUNK * RT_E; t += 256) {
            const int r = t / RT_CHUNK, c = t - r * RT_CHUNK;
            const int e = min(e0 + r, E - 1), b = min(b0 + r, B - 1), cc = min(c0 + c, H - 1);
            ws[c][r] = W[(long long)e * H + cc];
            xs[c][r] = x[(long long)b * H + cc];
        }
        __syncthreads();
        const int nc = min(RT_CHUNK, c_end - c0);
        for (int c = 0; c < nc; ++c) {
            const double w0 = ws[c][te], w1 = ws[c][te + 1];
            const double x0 = xs[c][tb], x1 = xs[c][tb + 1];
            acc[0][0] = fma(w0, x0, acc[0][0]);
            acc[0][1] = fma(w0, x1, acc[0][1]);
            acc[1][0] = fma(w1, x0, acc[1][0]);
            acc[1][1] = fma(w1, x1, acc[1][1]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = e0 + te + i, b = b0 + tb + j;
            if (e < E && b < B) partial[((long long)split * B + b) * E + e] = acc[i][j];
        }
}

// one wave per token: logits = sum of the slice partials (slice order) + bias, then top-K
__global__ __launch_bounds__(256) void k_topk_split(const double* __restrict__ partial, int nsplit,
                                                    const float* __restrict__ bias, int B, int E, int K, int renorm,
                                                    double* __restrict__ logits, int32_t* __restrict__ idx,
                                                    float* __restrict__ w)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int b = blockIdx.x * 4 + wave;
    if (b >= B) return;
    double lv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int e = min(lane + 64 * j, E - 1);
        double s = 0.0;
        for (int sp = 0; sp < nsplit; ++sp) s += partial[((long long)sp * B + b) * E + e];
        lv[j] = s + (bias ? (double)bias[e] : 0.0);
        if (logits && lane + 64 * j < E) logits[(long long)b * E + lane + 64 * j] = lv[j];
    }
    int id;
    float wt;
    topk_select<32, 16>(lv, E, K, renorm, lane, id, wt);
    if (lane < K) {
        idx[(long long)b * K + lane] = id;
        w[(long long)b * K + lane] = wt;
    }
}

int router_splits(int H) { return (H + RT_SLICE - 1) / RT_SLICE; }

void launch_route_batched(const float* x, int B, const float* W, const float* bias, int H, int E, int K, int renorm,
                          double* partial, double* logits, int32_t* idx, float* w, hipStream_t s, Timing t)
{
    const dim3 grid((E + RT_E - 1) / RT_E, (B + RT_B - 1) / RT_B, router_splits(H));
    hipExtLaunchKernelGGL(k_router_tiled, grid, dim3(256), 0, s, t.start, t.stop, 0, x, B, W, H, E, partial);
    hipLaunchKernelGGL(k_topk_split, dim3((B + 3) / 4), dim3(256), 0, s, partial, router_splits(H), bias, B, E, K,
                       renorm, logits, idx, w);
}

// ----------------------------------------------------------------------------
// Grouping: stable counting sort of the B*K assignments (slot i = b*K + k holds
// expert idx[i]) by expert id, in one block.  Thread e owns expert e: it counts
// the slots naming e, the block scans the counts, and thread e then walks the
// slots in order and places its own, so every expert's list keeps slot order.
// Slots whose id is outside [0, E) are left out.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_group(const int32_t* __restrict__ idx, int B, int K, int E, GroupOut O)
{
    __shared__ int sidx[MOE_MAX_B * MOE_MAX_K];
    __shared__ int wsum[2][16];
    const int tid = threadIdx.x;
    const int n = B * K;
    for (int i = tid; i < n; i += 1024) sidx[i] = idx[i];
    __syncthreads();
    int c = 0;
    if (tid < E)
        for (int i = 0; i < n; ++i) c += (sidx[i] == tid) ? 1 : 0;
    const int f = c > 0 ? 1 : 0;
    // exclusive scans of the counts and of the active flags over the block
    int sc = c, sf = f;
    for (int off = 1; off < 64; off <<= 1) {
        const int oc = __shfl_up(sc, off, 64), of = __shfl_up(sf, off, 64);
        if ((tid & 63) >= off) {
            sc += oc;
            sf += of;
        }
    }
    if ((tid & 63) == 63) {
        wsum[0][tid >> 6] = sc;
        wsum[1][tid >> 6] = sf;
    }
    __syncthreads();
    int pc = 0, pf = 0;
    for (int q = 0; q < (tid >> 6); ++q) {
        pc += wsum[0][q];
        pf += wsum[1][q];
    }
    const int excl_c = pc + sc - c, excl_f = pf + sf - f;
    const bool work = O.grp_u != nullptr;
    if (tid < E) O.offsets[tid] = excl_c;
    if (tid == E - 1) {
        const int total = excl_c + c, U = excl_f + f;
        O.offsets[E] = total;
        if (work) {
            // work list: the shared expert (every token) first, then the routed experts by id
            O.grp_u[0] = U;
            O.act_expert[0] = E;
            O.act_off[0] = 0;
            O.act_off[U + 1] = B + total;
        }
    }
    if (tid < E && f) {
        if (work) {
            O.act_expert[1 + excl_f] = tid;
            O.act_off[1 + excl_f] = B + excl_c;
        }
        int pos = excl_c;
        for (int i = 0; i < n; ++i) {
            if (sidx[i] != tid) continue;
            O.tokens[pos] = i / K;
            O.slots[pos] = i;
            if (work) {
                O.ent_token[B + pos] = i / K;
                O.slot_pos[i] = B + pos;
            }
            ++pos;
        }
    }
    if (work) {
        for (int b = tid; b < B; b += 1024) O.ent_token[b] = b;
        for (int i = tid; i < n; i += 1024) {
            const int e = sidx[i];
            if (e < 0 || e >= E) O.slot_pos[i] = -1;
        }
    }
}

void launch_group(const int32_t* idx, int B, int K, int E, const GroupOut& O, hipStream_t s)
{
    hipLaunchKernelGGL(k_group, dim3(1), dim3(1024), 0, s, idx, B, K, E, O);
}

// ----------------------------------------------------------------------------
// Token operands of the gate/up GEMM: x * 2^-e (one power-of-two scale per
// token, so that the largest |x| lands in [2^14, 2^15)) split into fp16 hi and
// lo = fp16(v - hi), in the pair order the packed codes unpack to.
//   xhl[(t * G + g) * 16 + hl * 8 + d]: uint4 holding dword d's 8 columns of
//   group g (d = 0..7; columns 8d + (0,4,1,5,2,6,3,7)), hl = 0 hi, 1 lo.
// ----------------------------------------------------------------------------
__device__ inline float exp2i(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

__global__ __launch_bounds__(256) void k_prep_tokens(const float* __restrict__ x, int H, uint4* __restrict__ xhl,
                                                     float* __restrict__ xscale)
{
    __shared__ float red[4];
    const int t = blockIdx.x, tid = threadIdx.x;
    const float* xt = x + (long long)t * H;
    float m = 0.f;
    for (int c = tid; c < H; c += 256) m = fmaxf(m, fabsf(xt[c]));
    m = wave_max(m);
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int e = 0;
    if (amax > 0.f && amax <= 3.4e38f) {
        e = ilogbf(amax) - 14;
        e = e < -110 ? -110 : (e > 113 ? 113 : e);
    }
    const float inv = exp2i(-e);
    if (tid == 0) xscale[t] = exp2i(e);
    const int G = H / 64;
    uint16_t* out = reinterpret_cast<uint16_t*>(xhl + (long long)t * G * 16);
    for (int c = tid; c < H; c += 256) {
        const float v = xt[c] * inv;
        const _Float16 hi = (_Float16)v;
        const _Float16 lo = (_Float16)(v - (float)hi);
        const int g = c >> 6, cc = c & 63, d = cc >> 3, r = cc & 7;
        const long long o = ((long long)g * 16 + d) * 8 + (r & 3) * 2 + (r >> 2);
        out[o] = __builtin_bit_cast(uint16_t, hi);
        out[o + 64] = __builtin_bit_cast(uint16_t, lo);
    }
}

// ----------------------------------------------------------------------------
// One 16-byte chunk of a 4-bit row (32 codes) -> fp16 MFMA operands: out[d]
// holds the 8 weights s*q + b of the chunk's dword d in the order
// (c0, c4, c1, c5, c2, c6, c3, c7).  OR-ing the fp16 pattern of 1024 into a
// masked code pair gives (1024 + q_a, 1024 + q_b); subtracting 1024 is exact and
// one fused multiply-add gives s*q + b, rounded once to fp16.
// ----------------------------------------------------------------------------
__device__ inline void dequant_chunk_q4(uint4 c, uint32_t sb, h8 (&out)[4])
{
    const _Float16 s = (_Float16)bf16_lo(sb), b = (_Float16)bf16_hi(sb);
    const h2 s2 = {s, s}, b2 = {b, b};
    const h2 k1024 = {(_Float16)1024.f, (_Float16)1024.f};
    const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        h2 p[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t bits = ((wd[d] >> (4 * t)) & 0x000F000Fu) | 0x64006400u;
            const h2 q = __builtin_bit_cast(h2, bits) - k1024;
            p[t] = __builtin_elementwise_fma(q, s2, b2);
        }
        out[d] = h8{p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
    }
}

// ----------------------------------------------------------------------------
// Grouped dequant-GEMM.  A work item is (active expert u, tile of 128 rows): a
// block of 4 waves, 32 rows per wave as two 16-row MFMA tiles, multiplies the
// item's rows by the expert's tokens, up to 64 at a time (four 16-token tiles).
// K advances 128 columns (4 chunks of 16 bytes) per step: lane (i, kk) of a wave
// holds chunk 4*step + kk of row i of each tile, and MFMA d (16 x 16 x 32)
// takes dword d of the four lanes' chunks against the token operands of the
// same 32 columns, staged in LDS as [tt][kk][d][hl][token].
//
// gfx9 counts outstanding vector loads in issue order, so each step issues the
// next step's token operands (cache-resident) before the next step's weight
// chunks (HBM); the LDS hand-over waits only for the former, and the barrier
// leaves the weight loads in flight: the weights stream one step ahead.
//
// MODE_GATEUP: rows are gate/up row pairs; token operand x as fp16 hi + lo;
//   writes h = silu(g) * u of each entry as fp16(h / 256) in the pair layout
//   hb[entry][dword d < 8][G_i] (uint4 of 4 pairs).
// MODE_DOWN: rows are down rows; token operand h (fp16); writes the entry's
//   output row part[entry][H] in fp32.
// ----------------------------------------------------------------------------
enum { MODE_GATEUP = 0, MODE_DOWN = 1 };
constexpr int GM_WAVES = 4, GM_TT = 4, GM_ROWS = GM_WAVES * 32;

struct GroupedArgs {
    const uint8_t* slab;
    Layout L;
    const int32_t* grp_u;
    const int32_t* act_expert;
    const int32_t* act_off;
    const int32_t* ent_token;
    const uint4* xhl;
    const float* xscale;
    uint4* hb;
    float* part;
};

template <int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_grouped_mfma(GroupedArgs A)
{
    constexpr int NM = (MODE == MODE_GATEUP) ? 2 : 1;  // matrices per row: gate + up | down
    constexpr int HL = (MODE == MODE_GATEUP) ? 2 : 1;  // token operand parts: hi + lo | h
    constexpr int NSTG = GM_TT * 4 * 4 * HL * 16;      // uint4 staged per step
    constexpr int PER_T = NSTG / 256;
    __shared__ u4 bs[2][NSTG];

    const Layout& L = A.L;
    const int G = (MODE == MODE_GATEUP) ? L.Gh : L.Gi;
    const int NR = (MODE == MODE_GATEUP) ? L.I : L.H;
    const int tiles = (NR + GM_ROWS - 1) / GM_ROWS;
    const int n_items = (A.grp_u[0] + 1) * tiles;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i = lane & 15, kk = lane >> 4;
    const int nsteps = (2 * G + 3) / 4;  // 2 chunks per group, 4 chunks per step

    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int u = item / tiles, tile = item - u * tiles;
        const int e = A.act_expert[u];
        const int ent0 = A.act_off[u], n = A.act_off[u + 1] - ent0;
        const int rbase = tile * GM_ROWS + wave * 32;
        const uint8_t* rec = A.slab + (long long)e * L.record;

        const uint8_t* rowp[2];
        const uint8_t* sbp[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int row = min(rbase + 16 * rt + i, NR - 1);
            if (MODE == MODE_GATEUP) {
                rowp[rt] = rec + (long long)row * 2 * L.hb;
                sbp[rt] = rec + L.off_gu_sb + (long long)row * G * 8;
            } else {
                rowp[rt] = rec + L.off_d_codes + (long long)row * L.ib;
                sbp[rt] = rec + L.off_d_sb + (long long)row * G * 4;
            }
        }

        for (int p0 = 0; p0 < n; p0 += 16 * GM_TT) {
            const int ntt = min(GM_TT, (n - p0 + 15) / 16);

            // token operands of step ks: element t = ((tt*4 + k2)*4 + d)*HL*16 + hl*16 + j.
            // src[q]: the element's fixed part (token or entry row, hl, d); the step adds
            // the chunk's group and half.  Chunks past the row end (2G not a multiple
            // of 4) read a valid chunk; their weights are zeroed below.
            int src[PER_T];
            int k2q[PER_T];
#pragma unroll
            for (int q = 0; q < PER_T; ++q) {
                const int t = threadIdx.x + 256 * q;
                const int j = t & 15, r1 = t >> 4;
                const int hl = (HL == 2) ? (r1 & 1) : 0, r2 = r1 / HL;
                const int d = r2 & 3, tt = r2 >> 4;
                k2q[q] = (r2 >> 2) & 3;
                const int m = min(p0 + tt * 16 + j, n - 1);
                if (MODE == MODE_GATEUP)
                    src[q] = A.ent_token[ent0 + m] * G * 16 + hl * 8 + d;
                else
                    src[q] = (ent0 + m) * 8 * G + d * G;
            }
            const u4* xhl = reinterpret_cast<const u4*>(A.xhl);
            const u4* hbv = reinterpret_cast<const u4*>(A.hb);
            auto stage_load = [&](int ks, u4 (&st)[PER_T]) {
#pragma unroll
                for (int q = 0; q < PER_T; ++q) {
                    const int P = min(4 * ks + k2q[q], 2 * G - 1);
                    const int jh = P >= G ? 1 : 0, g = P - jh * G;
                    if (MODE == MODE_GATEUP)
                        st[q] = xhl[src[q] + g * 16 + jh * 4];
                    else
                        st[q] = hbv[src[q] + jh * 4 * G + g];
                }
            };
            struct WRegs {
                uint4 c[2][NM];
                uint32_t sb[2][NM];
            };
            auto weight_load = [&](int ks, WRegs& W) {
                const int P = min(4 * ks + kk, 2 * G - 1), g = P >= G ? P - G : P;
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    W.c[rt][0] = *reinterpret_cast<const uint4*>(rowp[rt] + (long long)P * 16);
                    if (MODE == MODE_GATEUP) {
                        W.c[rt][NM - 1] = *reinterpret_cast<const uint4*>(rowp[rt] + L.hb + (long long)P * 16);
                        const uint2 v = *reinterpret_cast<const uint2*>(sbp[rt] + (long long)g * 8);
                        W.sb[rt][0] = v.x;
                        W.sb[rt][NM - 1] = v.y;
                    } else {
                        W.sb[rt][0] = *reinterpret_cast<const uint32_t*>(sbp[rt] + (long long)g * 4);
                    }
                }
            };

            f4 acc[2][NM][GM_TT];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int mm = 0; mm < NM; ++mm)
#pragma unroll
                    for (int tt = 0; tt < GM_TT; ++tt) acc[rt][mm][tt] = f4{0.f, 0.f, 0.f, 0.f};

            u4 st[PER_T];
            WRegs Wc, Wn;
            __syncthreads();  // LDS reads of the previous item or pass are done
            stage_load(0, st);
            __builtin_amdgcn_sched_barrier(0);
            weight_load(0, Wc);
#pragma unroll
            for (int q = 0; q < PER_T; ++q) bs[0][threadIdx.x + 256 * q] = st[q];
            __syncthreads();

            for (int ks = 0; ks < nsteps; ++ks) {
                const bool more = ks + 1 < nsteps;
                if (more) {
                    stage_load(ks + 1, st);
                    __builtin_amdgcn_sched_barrier(0);
                    weight_load(ks + 1, Wn);
                }
                __builtin_amdgcn_sched_barrier(0);
                const u4* buf = bs[ks & 1];
                const bool pad = 4 * ks + kk >= 2 * G;  // chunk past the row end: zero weights
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    h8 a[NM][4];
#pragma unroll
                    for (int mm = 0; mm < NM; ++mm) dequant_chunk_q4(Wc.c[rt][mm], pad ? 0u : Wc.sb[rt][mm], a[mm]);
#pragma unroll
                    for (int tt = 0; tt < GM_TT; ++tt) {
                        if (tt < ntt) {
#pragma unroll
                            for (int d = 0; d < 4; ++d)
#pragma unroll
                                for (int hl = 0; hl < HL; ++hl) {
                                    const h8 bv =
                                        __builtin_bit_cast(h8, buf[(((tt * 4 + kk) * 4 + d) * HL + hl) * 16 + i]);
#pragma unroll
                                    for (int mm = 0; mm < NM; ++mm)
                                        acc[rt][mm][tt] = mfma16(a[mm][d], bv, acc[rt][mm][tt]);
                                }
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                if (more) {
#pragma unroll
                    for (int q = 0; q < PER_T; ++q) bs[(ks + 1) & 1][threadIdx.x + 256 * q] = st[q];
                    __syncthreads();
                    Wc = Wn;
                }
            }

            // lane (i, kk) holds D[row 4*kk + v][token i] of each tile
#pragma unroll
            for (int tt = 0; tt < GM_TT; ++tt) {
                const int m = p0 + tt * 16 + i;
                if (tt >= ntt || m >= n) continue;
                const int ent = ent0 + m;
                if (MODE == MODE_GATEUP) {
                    const float xs = A.xscale[A.ent_token[ent]];
                    uint16_t* hrow = reinterpret_cast<uint16_t*>(A.hb + (long long)ent * 8 * L.Gi);
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int row = rbase + 16 * rt + 4 * kk + v;
                            if (row >= NR) continue;
                            const float gg = acc[rt][0][tt][v] * xs, uu = acc[rt][NM - 1][tt][v] * xs;
                            const float h = gg / (1.f + __expf(-gg)) * uu;
                            const int grp = row >> 6, cc = row & 63, dd = cc >> 3, r = cc & 7;
                            hrow[((long long)dd * L.Gi + grp) * 8 + (r & 3) * 2 + (r >> 2)] =
                                __builtin_bit_cast(uint16_t, (_Float16)(h * (1.f / 256.f)));
                        }
                } else {
                    float* prow = A.part + (long long)ent * L.H;
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int row = rbase + 16 * rt + 4 * kk + v;
                            if (row < NR) prow[row] = 256.f * acc[rt][0][tt][v];
                        }
                }
            }
        }
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
    return L.bits == 4 && B >= 2 && B <= MOE_MAX_B && K <= MOE_MAX_K && L.H % 64 == 0 && L.I % 64 == 0;
}

size_t grouped_workspace_bytes(const Layout& L, int B, int K, int E)
{
    const size_t ents = (size_t)B * K + B;
    size_t n = 0;
    auto add = [&](size_t bytes) { n += (bytes + 255) & ~(size_t)255; };
    add(sizeof(double) * router_splits(L.H) * B * E);  // partial logits
    add(sizeof(int32_t) * (E + 1));                    // offsets
    add(sizeof(int32_t) * B * K);                      // tokens
    add(sizeof(int32_t) * B * K);                      // slots
    add(sizeof(int32_t) * 4);                          // U
    add(sizeof(int32_t) * (E + 1));                    // act_expert
    add(sizeof(int32_t) * (E + 2));                    // act_off
    add(sizeof(int32_t) * ents);                       // ent_token
    add(sizeof(int32_t) * B * K);                      // slot_pos
    add(16ull * B * L.Gh * 16);                        // xhl
    add(sizeof(float) * B);                            // xscale
    add(2ull * ents * L.I);                            // hb
    add(sizeof(float) * ents * L.H);                   // part
    return n;
}

GroupedWork carve_grouped(void* base, const Layout& L, int B, int K, int E)
{
    const size_t ents = (size_t)B * K + B;
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
    W.g.act_expert = (int32_t*)take(sizeof(int32_t) * (E + 1));
    W.g.act_off = (int32_t*)take(sizeof(int32_t) * (E + 2));
    W.g.ent_token = (int32_t*)take(sizeof(int32_t) * ents);
    W.g.slot_pos = (int32_t*)take(sizeof(int32_t) * B * K);
    W.xhl = (uint4*)take(16ull * B * L.Gh * 16);
    W.xscale = (float*)take(sizeof(float) * B);
    W.hb = (uint4*)take(2ull * ents * L.I);
    W.part = (float*)take(sizeof(float) * ents * L.H);
    return W;
}

int grouped_grid(const Layout& L, int B, int K, int E, int mode)
{
    const int max_u = min(E, B * K) + 1;
    const int NR = mode == MODE_GATEUP ? L.I : L.H;
    return max_u * ((NR + GM_ROWS - 1) / GM_ROWS);
}

void launch_ffn_grouped(const Layout& L, const void* slab, const GroupedWork& W, const float* x, const float* w,
                        float shared_w, int B, int K, int E, float* y, hipStream_t s, Timing tg, Timing td)
{
    hipLaunchKernelGGL(k_prep_tokens, dim3(B), dim3(256), 0, s, x, L.H, W.xhl, W.xscale);
    GroupedArgs A;
    A.slab = (const uint8_t*)slab;
    A.L = L;
    A.grp_u = W.g.grp_u;
    A.act_expert = W.g.act_expert;
    A.act_off = W.g.act_off;
    A.ent_token = W.g.ent_token;
    A.xhl = W.xhl;
    A.xscale = W.xscale;
    A.hb = W.hb;
    A.part = W.part;
    hipExtLaunchKernelGGL(k_grouped_mfma<MODE_GATEUP>, dim3(grouped_grid(L, B, K, E, MODE_GATEUP)), dim3(256), 0, s,
                          tg.start, tg.stop, 0, A);
    hipExtLaunchKernelGGL(k_grouped_mfma<MODE_DOWN>, dim3(grouped_grid(L, B, K, E, MODE_DOWN)), dim3(256), 0, s,
                          td.start, td.stop, 0, A);
    hipLaunchKernelGGL(k_combine, dim3((L.H + 255) / 256, B), dim3(256), 0, s, W.part, W.g.slot_pos, w, K, L.H,
                       shared_w, y);
}

}  // namespace moe
