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
// Decode attention on the matrix cores.  For one KV head g the per query heads
// of its group (at most 16, padded with zero rows) form the 16-wide side of the
// MFMAs, over sub-tiles of 16 cached positions:
//   scores  S^T [16 positions x 16 heads] = K [16 x d] . Q^T [d x 16]
//           (v_mfma_f32_16x16x32_bf16, d / 32 steps)
//   values  O   [16 heads x 16 columns]  += P [16 x 16 positions] . V [16 x 16]
//           (v_mfma_f32_16x16x16_bf16, one per 16 columns)
// The contraction index of either product only has to be labelled the same way
// on both operands, so each operand is loaded in its natural layout:
//   - K: lane (j, r) (j = lane % 16, r = lane / 16) reads row j of the sub-tile;
//     its chunk c (8 elements) is chunk 4c + r of the row, so the four lanes of a
//     row read 64 contiguous bytes per load.  q carries the same labels; it is
//     prepared once per block (scaled by log2(e)/sqrt(d), split into bf16 hi + lo)
//     and read from LDS.
//   - P: the score product leaves lane (j, r) with head j at positions 4r..4r+3,
//     which is exactly the A operand of the value product.
//   - V: lane (j, r) reads rows 4r..4r+3; for d >= 128 its columns are
//     128 w + 8 j + (0..7), so the 16 lanes of a row read 256 contiguous bytes per
//     load (d = 64: columns 4 j + (0..3)).  Pairing rows in registers gives one B
//     operand per column: value MFMA u yields one column per lane j.
// q and the weights p are fp32, each split into bf16 hi + lo (relative residual
// about 2^-17) and multiplied twice; K and V are exact bf16, the products exact,
// the sums fp32.
//
// Work split: a block of AT_WAVES waves covers AT_WAVES * R sub-tiles of one KV
// head (wave w takes sub-tiles w, w + AT_WAVES, ...); two waves share a SIMD.  A
// wave issues the next sub-tile's K loads as soon as the score MFMAs have read its
// K registers, and the V loads once the value MFMAs have read V, so its loads are
// in flight while it computes.  It keeps, per head, a reference
// maximum M, the weight sum L and O, all relative to M: weights are 2^(s - M), and
// M (with L and O) moves only when a score exceeds it by more than 2^AT_SLACK, so
// the weights stay below 2^AT_SLACK and O is rarely rescaled; the result does not
// depend on the reference.  The waves merge in LDS and the block writes one
// partial (M, L, O) per query head; the combine kernel merges the partials.
// Scores are in the log2 domain throughout.
// ----------------------------------------------------------------------------
constexpr int AT_SUB = 16;      // positions per sub-tile
constexpr int AT_WAVES = 4;     // waves per block
constexpr int AT_MAX_PER = 16;  // query heads per KV head
constexpr int AT_TARGET_BLOCKS = 256;
constexpr int AT_MAX_NBLK = 1024;  // most partials per head
constexpr float AT_SLACK = 8.f;

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef short s4v __attribute__((ext_vector_type(4)));
typedef float fl2 __attribute__((ext_vector_type(2)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

__device__ inline f4v mfma_k32(u4v a, u4v b, f4v c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, a), __builtin_bit_cast(bf8, b), c, 0, 0, 0);
}
__device__ inline f4v mfma_k16(u2v a, u2v b, f4v c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4v, a), __builtin_bit_cast(s4v, b), c, 0, 0, 0);
}

// (x0, x1) -> packed bf16 hi and lo terms: x = hi + lo + O(2^-17 |x|), each term
// rounded to nearest even by the hardware conversion; returns (hi, lo)
__device__ inline uint2 split_pair(float x0, float x1)
{
    const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(fl2{x0, x1}, bf2));
    const float r0 = x0 - __uint_as_float(hi << 16), r1 = x1 - __uint_as_float(hi & 0xFFFF0000u);
    return make_uint2(hi, __builtin_bit_cast(uint32_t, __builtin_convertvector(fl2{r0, r1}, bf2)));
}

// op over the four 16-lane rows of a wave (lanes j, j + 16, j + 32, j + 48)
template <typename Op>
__device__ inline float across_rows(float v, Op op)
{
    float a, b;
    swap<false>(v, a, b);
    v = op(a, b);
    swap<true>(v, a, b);
    return op(a, b);
}

struct AttnPlan {
    int R;     // sub-tiles per wave
    int nblk;  // blocks per KV head
};

__host__ __device__ inline AttnPlan attn_plan(int n_kv, int T)
{
    const long long st = (T + AT_SUB - 1) / AT_SUB;
    long long R = (long long)n_kv * st / ((long long)AT_WAVES * AT_TARGET_BLOCKS);
    if (R < 1) R = 1;
    long long nblk = (st + AT_WAVES * R - 1) / (AT_WAVES * R);
    if (nblk > AT_MAX_NBLK) {
        R = (st + AT_WAVES * AT_MAX_NBLK - 1) / (AT_WAVES * AT_MAX_NBLK);
        nblk = (st + AT_WAVES * R - 1) / (AT_WAVES * R);
    }
    AttnPlan p;
    p.R = (int)R;
    p.nblk = (int)nblk;
    return p;
}

// V column of value MFMA u in lane j
template <int VC>
__device__ inline int v_col(int u, int j)
{
    return VC >= 8 ? (u >> 3) * 128 + 8 * j + (u & 7) : VC * j + u;
}

template <int D>
struct AttnTile {
    static constexpr int KC = D / 32;  // 16-byte K chunks per lane = score MFMAs (x2 for hi, lo)
    static constexpr int VC = D / 16;  // V columns per lane = value MFMAs (x2)
    static constexpr int VW = VC / 2;  // dwords per V row and lane
    u4v k[KC];                         // K row p0 + j, chunks 4c + r
    uint32_t v[4][VW];                 // V rows p0 + 4r + e, the lane's columns
};

template <int D>
__device__ inline void attn_load_k(AttnTile<D>& t, const uint16_t* __restrict__ Kg, int p0, int T, int j, int r)
{
    const u4v* kp = reinterpret_cast<const u4v*>(Kg + (long long)min(p0 + j, T - 1) * D) + r;
#pragma unroll
    for (int c = 0; c < AttnTile<D>::KC; ++c) t.k[c] = kp[4 * c];
}

template <int D>
__device__ inline void attn_load_v(AttnTile<D>& t, const uint16_t* __restrict__ Vg, int p0, int T, int j, int r)
{
    constexpr int VC = AttnTile<D>::VC, VW = AttnTile<D>::VW;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint16_t* vp = Vg + (long long)min(p0 + 4 * r + e, T - 1) * D;
        if constexpr (VW == 2) {
            const uint2 w = *reinterpret_cast<const uint2*>(vp + VC * j);
            t.v[e][0] = w.x;
            t.v[e][1] = w.y;
        } else {
#pragma unroll
            for (int w4 = 0; w4 < VW / 4; ++w4) {
                const uint4 w = *reinterpret_cast<const uint4*>(vp + 128 * w4 + 8 * j);
                t.v[e][4 * w4 + 0] = w.x;
                t.v[e][4 * w4 + 1] = w.y;
                t.v[e][4 * w4 + 2] = w.z;
                t.v[e][4 * w4 + 3] = w.w;
            }
        }
    }
}

// partials: O [n_q][nblk][D] floats, then (M, L) [n_q][nblk][2]
template <int D>
__global__ __launch_bounds__(64 * AT_WAVES) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_partial(int n_q, int n_kv, int T, int R,
                                                               const float* __restrict__ q,
                                                               const uint16_t* __restrict__ K,
                                                               const uint16_t* __restrict__ V,
                                                               float* __restrict__ part_o,
                                                               float* __restrict__ part_ml)
{
    constexpr int KC = AttnTile<D>::KC, VC = AttnTile<D>::VC;
    __shared__ u4v q_s[2][KC][64];  // hi, lo operands per (chunk, lane)
    __shared__ float ml_s[AT_WAVES][2][16];
    __shared__ float o_s[2][4 * VC * 64];

    const int g = blockIdx.y, blk = blockIdx.x, nblk = gridDim.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, j = lane & 15, r = lane >> 4;
    const int per = n_q / n_kv;
    const long long st = (T + AT_SUB - 1) / AT_SUB;
    const uint16_t* Kg = K + (long long)g * T * D;
    const uint16_t* Vg = V + (long long)g * T * D;

    // q first (its wait then does not wait for the cache loads behind it)
    constexpr int QE = (KC * 64 + 64 * AT_WAVES - 1) / (64 * AT_WAVES);  // q entries per thread
    float4 qa[QE], qb[QE];
#pragma unroll
    for (int x = 0; x < QE; ++x) {
        const int e = min((int)threadIdx.x + x * 64 * AT_WAVES, KC * 64 - 1);
        const int c = e >> 6, l = e & 63;
        const float* qp = q + (long long)(g * per + min(l & 15, per - 1)) * D + 8 * (4 * c + (l >> 4));
        qa[x] = *reinterpret_cast<const float4*>(qp);
        qb[x] = *reinterpret_cast<const float4*>(qp + 4);
    }
    long long sub = (long long)blk * R * AT_WAVES + wave;  // the wave's first sub-tile
    AttnTile<D> t;
    attn_load_k<D>(t, Kg, (int)(min(sub, st - 1) * AT_SUB), T, j, r);
    attn_load_v<D>(t, Vg, (int)(min(sub, st - 1) * AT_SUB), T, j, r);
    __builtin_amdgcn_sched_barrier(0);

    // q operands: entry (c, l) holds head l % 16, elements 8 (4c + l / 16) + (0..7),
    // scaled by log2(e)/sqrt(d) and split
    {
        const float sc = 1.4426950408889634f * rsqrtf((float)D);
#pragma unroll
        for (int x = 0; x < QE; ++x) {
            const int e = threadIdx.x + x * 64 * AT_WAVES;
            if (e >= KC * 64) break;
            const int c = e >> 6, l = e & 63;
            const float z = (l & 15) < per ? sc : 0.f;
            const float4 a = qa[x], b = qb[x];
            const uint2 s0 = split_pair(a.x * z, a.y * z), s1 = split_pair(a.z * z, a.w * z);
            const uint2 s2 = split_pair(b.x * z, b.y * z), s3 = split_pair(b.z * z, b.w * z);
            q_s[0][c][l] = u4v{s0.x, s1.x, s2.x, s3.x};
            q_s[1][c][l] = u4v{s0.y, s1.y, s2.y, s3.y};
        }
    }
    __syncthreads();

    float M = -INFINITY, L = 0.f;  // head j
    f4v O[VC];                     // heads 4r + i, columns v_col(u, j)
#pragma unroll
    for (int u = 0; u < VC; ++u) O[u] = f4v{0.f, 0.f, 0.f, 0.f};

    for (int it = 0; it < R && sub < st; ++it) {
        const int p0 = (int)sub * AT_SUB;
        const long long nx = sub + AT_WAVES;
        const bool more = it + 1 < R && nx < st;
        // scores, two accumulator chains
        f4v a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KC; c += 2) {
            a0 = mfma_k32(t.k[c], q_s[0][c][lane], a0);
            if (c + 1 < KC) a1 = mfma_k32(t.k[c + 1], q_s[0][c + 1][lane], a1);
            a0 = mfma_k32(t.k[c], q_s[1][c][lane], a0);
            if (c + 1 < KC) a1 = mfma_k32(t.k[c + 1], q_s[1][c + 1][lane], a1);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (more) attn_load_k<D>(t, Kg, (int)nx * AT_SUB, T, j, r);
        __builtin_amdgcn_sched_barrier(0);
        float s[4];  // position p0 + 4r + i, head j
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = (p0 + 4 * r + i < T) ? a0[i] + a1[i] : -INFINITY;
        float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        mx = across_rows(mx, OpMax());
        if (__builtin_amdgcn_ballot_w64(mx > M + AT_SLACK)) {  // a head's reference moves
            const float Mn = mx > M + AT_SLACK ? mx : M;
            const float f = __builtin_amdgcn_exp2f(M - Mn);  // 1 where M stays, 0 from -inf
            L *= f;
            M = Mn;
            if (it > 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float fi = __shfl(f, 4 * r + i);
#pragma unroll
                    for (int u = 0; u < VC; ++u) O[u][i] *= fi;
                }
            }
        }
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(s[i] - M);
        L += across_rows((p[0] + p[1]) + (p[2] + p[3]), OpAdd());
        const uint2 p01 = split_pair(p[0], p[1]), p23 = split_pair(p[2], p[3]);
        const u2v phi = {p01.x, p23.x}, plo = {p01.y, p23.y};
#pragma unroll
        for (int u = 0; u < VC; ++u) {
            const uint32_t x0 = t.v[0][u >> 1], x1 = t.v[1][u >> 1], x2 = t.v[2][u >> 1], x3 = t.v[3][u >> 1];
            const u2v b = (u & 1) ? u2v{(x0 >> 16) | (x1 & 0xFFFF0000u), (x2 >> 16) | (x3 & 0xFFFF0000u)}
                                  : u2v{(x0 & 0xFFFFu) | (x1 << 16), (x2 & 0xFFFFu) | (x3 << 16)};
            O[u] = mfma_k16(phi, b, O[u]);
            O[u] = mfma_k16(plo, b, O[u]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (more) attn_load_v<D>(t, Vg, (int)nx * AT_SUB, T, j, r);
        __builtin_amdgcn_sched_barrier(0);
        sub = nx;
    }

    // merge the waves: block reference and sum per head, each wave's O scaled to it
    if (r == 0) {
        ml_s[wave][0][j] = M;
        ml_s[wave][1][j] = L;
    }
    __syncthreads();
    float fself[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * r + i;
        float Mb = ml_s[0][0][m];
#pragma unroll
        for (int w = 1; w < AT_WAVES; ++w) Mb = fmaxf(Mb, ml_s[w][0][m]);
        fself[i] = __builtin_amdgcn_exp2f(ml_s[wave][0][m] - Mb);  // 0 for a wave without positions
    }
#pragma unroll
    for (int u = 0; u < VC; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[u][i] *= fself[i];
    // tree sum: waves 2, 3 -> 0, 1 -> 0; slot (i, u, lane) is conflict-free
    auto put = [&](int buf) {
#pragma unroll
        for (int u = 0; u < VC; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) o_s[buf][(i * VC + u) * 64 + lane] = O[u][i];
    };
    auto add = [&](int buf) {
#pragma unroll
        for (int u = 0; u < VC; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) O[u][i] += o_s[buf][(i * VC + u) * 64 + lane];
    };
    if (wave >= 2) put(wave - 2);
    __syncthreads();
    if (wave < 2) add(wave);
    __syncthreads();
    if (wave == 1) put(0);
    __syncthreads();
    if (wave != 0) return;
    add(0);
    const long long hb = (long long)g * per;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * r + i;
        if (m >= per) continue;
        float* op = part_o + ((hb + m) * nblk + blk) * D;
#pragma unroll
        for (int u = 0; u < VC; u += 4)
            *reinterpret_cast<float4*>(op + v_col<VC>(u, j)) = make_float4(O[u][i], O[u + 1][i], O[u + 2][i], O[u + 3][i]);
    }
    if (r == 0 && j < per) {
        float Mb = ml_s[0][0][j], Lb = 0.f;
#pragma unroll
        for (int w = 1; w < AT_WAVES; ++w) Mb = fmaxf(Mb, ml_s[w][0][j]);
#pragma unroll
        for (int w = 0; w < AT_WAVES; ++w) Lb += ml_s[w][1][j] * __builtin_amdgcn_exp2f(ml_s[w][0][j] - Mb);
        float* mp = part_ml + ((hb + j) * nblk + blk) * 2;
        mp[0] = Mb;
        mp[1] = Lb;
    }
}

// One block per (query head, 64 columns), 16 waves; wave w merges the partials
// w, w + 16, ... for its lane's column, 8 at a time with the loads issued together,
// and the waves meet in LDS.
constexpr int AC_WAVES = 16;
constexpr int AC_BATCH = 8;

__global__ __launch_bounds__(64 * AC_WAVES) void k_attn_combine(int D, int nblk, const float* __restrict__ part_o,
                                                               const float* __restrict__ part_ml,
                                                               float* __restrict__ o)
{
    __shared__ float red[AC_WAVES][3][64];
    const int h = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const float* ph = part_o + (long long)h * nblk * D + blockIdx.y * 64 + lane;
    const float* mh = part_ml + (long long)h * nblk * 2;
    float M = -INFINITY, L = 0.f, A = 0.f;
    for (int b0 = wave; b0 < nblk; b0 += AC_WAVES * AC_BATCH) {
        float x[AC_BATCH], m[AC_BATCH], l[AC_BATCH];
#pragma unroll
        for (int k = 0; k < AC_BATCH; ++k) {
            const int b = b0 + k * AC_WAVES;
            const bool ok = b < nblk;
            x[k] = ok ? ph[(long long)b * D] : 0.f;
            m[k] = ok ? mh[2 * b] : -INFINITY;
            l[k] = ok ? mh[2 * b + 1] : 0.f;
        }
        float mc = m[0];
#pragma unroll
        for (int k = 1; k < AC_BATCH; ++k) mc = fmaxf(mc, m[k]);
        const float Mn = fmaxf(M, mc);  // finite: partial b0 exists
        const float f = __builtin_amdgcn_exp2f(M - Mn);
        A *= f;
        L *= f;
#pragma unroll
        for (int k = 0; k < AC_BATCH; ++k) {
            const float w = __builtin_amdgcn_exp2f(m[k] - Mn);
            A = fmaf(x[k], w, A);
            L = fmaf(l[k], w, L);
        }
        M = Mn;
    }
    red[wave][0][lane] = M;
    red[wave][1][lane] = L;
    red[wave][2][lane] = A;
    __syncthreads();
    if (wave != 0) return;
    float Mb = red[0][0][lane];
#pragma unroll
    for (int w = 1; w < AC_WAVES; ++w) Mb = fmaxf(Mb, red[w][0][lane]);
    float Lb = 0.f, Ab = 0.f;
#pragma unroll
    for (int w = 0; w < AC_WAVES; ++w) {
        const float f = __builtin_amdgcn_exp2f(red[w][0][lane] - Mb);  // 0 for a wave without partials
        Lb = fmaf(red[w][1][lane], f, Lb);
        Ab = fmaf(red[w][2][lane], f, Ab);
    }
    o[(long long)h * D + blockIdx.y * 64 + lane] = Ab / Lb;
}

size_t attn_workspace_bytes(int n_q, int n_kv, int d, int T)
{
    const AttnPlan p = attn_plan(n_kv, T);
    return (size_t)n_q * p.nblk * (d + 2) * 4;
}

int attn_max_per() { return AT_MAX_PER; }

void launch_attn_decode(int n_q, int n_kv, int d, int T, const float* q, const uint16_t* K, const uint16_t* V,
                        float* part, float* o, hipStream_t s)
{
    const AttnPlan p = attn_plan(n_kv, T);
    float* part_o = part;
    float* part_ml = part + (size_t)n_q * p.nblk * d;
    const dim3 grid(p.nblk, n_kv), blk(64 * AT_WAVES);
    switch (d) {
    case 64: hipLaunchKernelGGL(k_attn_partial<64>, grid, blk, 0, s, n_q, n_kv, T, p.R, q, K, V, part_o, part_ml); break;
    case 128: hipLaunchKernelGGL(k_attn_partial<128>, grid, blk, 0, s, n_q, n_kv, T, p.R, q, K, V, part_o, part_ml); break;
    default: hipLaunchKernelGGL(k_attn_partial<256>, grid, blk, 0, s, n_q, n_kv, T, p.R, q, K, V, part_o, part_ml); break;
    }
    hipLaunchKernelGGL(k_attn_combine, dim3(n_q, d / 64), dim3(64 * AC_WAVES), 0, s, d, p.nblk, part_o, part_ml, o);
}

}  // namespace moe
