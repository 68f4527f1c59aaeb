// common.h - packed expert layout and device helpers shared by the gfx950 kernels.
//
// Packed record of one expert (bits = 4 or 2, G_h = H/64, G_i = I/64 groups per row),
// byte-for-byte the same size as the canonical expert:
//   [gu_codes]  I row pairs, each [gate row codes (H*bits/8 B) | up row codes (H*bits/8 B)]
//   [gu_sb]     I x G_h entries of 8 B: bf16 (gate scale, gate bias, up scale, up bias)
//   [d_codes]   H rows of I*bits/8 B, in panels of 16 rows (d_chunk_off below)
//   [d_sb]      H x G_i entries of 4 B: bf16 (scale, bias)
// Inside a row the codes of group g are split into 16-byte chunks; chunk j of
// group g sits at chunk position j*G + g (4-bit: 2 chunks per group, 2-bit: 1),
// so that 64 lanes working on 64 consecutive groups issue fully contiguous
// 16-byte loads.  A gate/up row's chunks are contiguous.  The down rows are
// stored in panels of 16 rows: each row's chunks are cut into units of 4 chunks
// (64 bytes), and unit u of the panel's 16 rows is stored as 16 consecutive runs,
// row 0 first, so that 64 bytes of 16 consecutive rows (a step of the grouped
// MFMA kernel) are one contiguous kilobyte and 4 consecutive rows (a wave of the
// single-token down kernel) are contiguous per unit.  A row shorter than 64
// bytes leaves the panel row-major.  Within a chunk the codes keep the canonical order (low bits =
// lower column), which puts columns (c, c+4) (4-bit) or (c, c+8) (2-bit) in the
// two 16-bit halves of a dword: masking one field of each half and OR-ing in the
// fp16 pattern of 1024 turns two codes into the fp16 pair (1024 + t*q_a, 1024 + t*q_b)
// with t a power of two, ready for v_dot2 against an fp16 pair of activations.
//
// Activation operand ("prep") of a vector v split in groups of 64:
//   q  [8][G] uint4: 32 fp16 pairs per group; pair p of group g is element p%4
//                    of uint4 (p/4)*G + g.  Pair p holds v_h at columns
//                    4-bit: (8*(p/4) + p%4, +4);  2-bit: (16*(p/8) + p%8, +8),
//                    where v_h = fp16(v * 2^-e_g) with a power-of-two per-group scale.
//   st [G]    float4: (C_g, S_g, 2^e_g, 0) with S_g = sum of v over the group and
//                    C_g = 1024 * sum_p (v_h pair sum) / t(p) + mid * sum_c (v_h - v 2^-e_g):
//                    the offset the fp16 code patterns add to the dot products, plus
//                    the code midpoint (7.5 or 1.5) times the group's rounding error.
// Per group and row:  sum_c (s*q_c + b) v_c ~= s * 2^e_g * (sum_t acc_t / t - C_g) + b * S_g,
// where sum_t acc_t / t - C_g = sum_c (q_c - mid) v_h,c + mid * sum_c v_c 2^-e_g: the
// fp16 rounding of v only meets the zero-mean part of the codes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

struct Layout {
    int bits, H, I, Gh, Gi;
    long long hb, ib;  // code bytes per gate/up row and per down row
    long long off_gu_sb, off_d_codes, off_d_sb, record;
};

__host__ __device__ inline Layout make_layout(int bits, int H, int I)
{
    Layout L;
    L.bits = bits;
    L.H = H;
    L.I = I;
    L.Gh = H / 64;
    L.Gi = I / 64;
    L.hb = (long long)H * bits / 8;
    L.ib = (long long)I * bits / 8;
    L.off_gu_sb = 2LL * I * L.hb;
    L.off_d_codes = L.off_gu_sb + 8LL * I * L.Gh;
    L.off_d_sb = L.off_d_codes + (long long)H * L.ib;
    L.record = L.off_d_sb + 4LL * H * L.Gi;
    return L;
}

// Byte offset, from the start of d_codes, of chunk position P of down row r:
// panel r / 16, unit P / 4 (the units before it are full, 16 x 64 bytes), then the
// row's run in the unit (64 bytes, or what is left of a shorter row), then the chunk.
__host__ __device__ inline long long d_chunk_off(const Layout& L, int r, int P)
{
    const int u = P >> 2;
    const long long w = (L.ib - 64LL * u) < 64 ? (L.ib - 64LL * u) : 64;
    return (long long)(r >> 4) * 16 * L.ib + (long long)u * 1024 + (long long)(r & 15) * w + (P & 3) * 16;
}

// lanes cooperating on one row: G rounded up to a power of two, at most 64
__host__ __device__ inline int lanes_per_row(int G)
{
    int l = 1;
    while (l < G && l < 64) l <<= 1;
    return l;
}

__device__ inline float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Opaque register constants: keeps the masks in SGPRs and the fp16 pattern in a
// VGPR so each code pair costs a single v_and_or_b32 (gfx9 VOP3 takes no literals).
struct Masks {
    uint32_t magic, m4a, m4b, m2[5];
};

__device__ inline Masks load_masks()
{
    Masks m;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m.magic));
    asm volatile("s_mov_b32 %0, 0xf000f" : "=s"(m.m4a));
    asm volatile("s_mov_b32 %0, 0xf000f0" : "=s"(m.m4b));
    asm volatile("s_mov_b32 %0, 0x30003" : "=s"(m.m2[0]));
    asm volatile("s_mov_b32 %0, 0xc000c" : "=s"(m.m2[1]));
    asm volatile("s_mov_b32 %0, 0x300030" : "=s"(m.m2[2]));
    asm volatile("s_mov_b32 %0, 0xc000c0" : "=s"(m.m2[3]));
    asm volatile("s_mov_b32 %0, 0x3000300" : "=s"(m.m2[4]));
    return m;
}

__device__ inline float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
}

// 4-bit: one group = two 16-byte chunks c0 (columns 0..31) and c1 (32..63);
// xp = the group's 8 uint4 of activation pairs.  Returns sum_t acc_t / t.
__device__ inline float group_dot_q4(const Masks& M, uint4 c0, uint4 c1, const uint4* xp)
{
    const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    float a1 = 0.f, a16 = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
        const uint32_t v = w[d], v8 = v >> 8;
        const uint4 x = xp[d];
        a1 = dot2((v & M.m4a) | M.magic, x.x, a1);
        a16 = dot2((v & M.m4b) | M.magic, x.y, a16);
        a1 = dot2((v8 & M.m4a) | M.magic, x.z, a1);
        a16 = dot2((v8 & M.m4b) | M.magic, x.w, a16);
    }
    return fmaf(a16, 0.0625f, a1);
}

// 2-bit: one group = one 16-byte chunk (4 dwords of 16 codes).
__device__ inline float group_dot_q2(const Masks& M, uint4 c0, const uint4* xp)
{
    const uint32_t w[4] = {c0.x, c0.y, c0.z, c0.w};
    float a1 = 0.f, a4 = 0.f, a16 = 0.f, a64 = 0.f, a256 = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t v = w[d], v10 = v >> 10;
        const uint4 x0 = xp[2 * d], x1 = xp[2 * d + 1];
        a1 = dot2((v & M.m2[0]) | M.magic, x0.x, a1);
        a4 = dot2((v & M.m2[1]) | M.magic, x0.y, a4);
        a16 = dot2((v & M.m2[2]) | M.magic, x0.z, a16);
        a64 = dot2((v & M.m2[3]) | M.magic, x0.w, a64);
        a256 = dot2((v & M.m2[4]) | M.magic, x1.x, a256);
        a1 = dot2((v10 & M.m2[0]) | M.magic, x1.y, a1);
        a4 = dot2((v10 & M.m2[1]) | M.magic, x1.z, a4);
        a16 = dot2((v10 & M.m2[2]) | M.magic, x1.w, a16);
    }
    float r = fmaf(a256, 1.f / 256.f, a64 * (1.f / 64.f));
    r = fmaf(a16, 1.f / 16.f, r);
    r = fmaf(a4, 0.25f, r);
    return r + a1;
}

// divisor t of pair p (see the prep layout above)
__device__ inline float pair_class_inv(int bits, int p)
{
    if (bits == 4) return (p & 1) ? 0.0625f : 1.f;
    switch (p & 7) {
    case 0: case 5: return 1.f;
    case 1: case 6: return 0.25f;
    case 2: case 7: return 0.0625f;
    case 3: return 1.f / 64.f;
    default: return 1.f / 256.f;
    }
}

// ---- h between the gate/up and down kernels.  h is written in fp32 in the
// element order of the fp16 pair layout above (the 8 values of pair-layout
// uint4 u sit at floats 8u .. 8u+7).  The down kernels scale each expert's h by
// a power of two taken from its largest |h| and round it to fp16 pairs, so a
// token whose h is tiny everywhere (saturated SiLU) keeps its relative precision.
__device__ inline float exp2i_f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// exponent e with max|h| * 2^-e in [2^14, 2^15); 0 for zero or non-finite maxima
__device__ inline int h_exponent(float amax)
{
    if (!(amax > 0.f) || !(amax <= 3.4e38f)) return 0;
    const int e = ilogbf(amax) - 14;
    return e < -110 ? -110 : (e > 113 ? 113 : e);
}

__device__ inline uint4 h_pairs(float4 a, float4 b, float inv)
{
    const h2 p0 = {(_Float16)(a.x * inv), (_Float16)(a.y * inv)};
    const h2 p1 = {(_Float16)(a.z * inv), (_Float16)(a.w * inv)};
    const h2 p2 = {(_Float16)(b.x * inv), (_Float16)(b.y * inv)};
    const h2 p3 = {(_Float16)(b.z * inv), (_Float16)(b.w * inv)};
    return make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                      __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
}

__device__ inline float absmax8(float4 a, float4 b)
{
    return fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                 fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
}

// ---- cross-lane exchange without LDS: DPP for partners inside a row of 16
// lanes, gfx950 permlane16/32 swaps across rows.  Every step combines a lane
// with its partner as op(own, partner), so for commutative ops all lanes of a
// group end with bit-identical results.
template <int CTRL>
__device__ inline uint32_t dpp32(uint32_t v)
{
    // every pattern used here reads inside the lane's row, so every lane is
    // written and the destination needs no initial value
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ inline float xchg(float v) { return __uint_as_float(dpp32<CTRL>(__float_as_uint(v))); }
template <int CTRL>
__device__ inline double xchg(double v)
{
    uint2 u = __builtin_bit_cast(uint2, v);
    u.x = dpp32<CTRL>(u.x);
    u.y = dpp32<CTRL>(u.y);
    return __builtin_bit_cast(double, u);
}

template <bool ROW32>
__device__ inline void swap_u32(uint32_t v, uint32_t& a, uint32_t& b)
{
    if (ROW32) {
        auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        a = p[0];
        b = p[1];
    } else {
        auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        a = p[0];
        b = p[1];
    }
}
template <bool ROW32>
__device__ inline void swap(float v, float& a, float& b)
{
    uint32_t x, y;
    swap_u32<ROW32>(__float_as_uint(v), x, y);
    a = __uint_as_float(x);
    b = __uint_as_float(y);
}
template <bool ROW32>
__device__ inline void swap(double v, double& a, double& b)
{
    uint2 u = __builtin_bit_cast(uint2, v), p, q;
    swap_u32<ROW32>(u.x, p.x, q.x);
    swap_u32<ROW32>(u.y, p.y, q.y);
    a = __builtin_bit_cast(double, p);
    b = __builtin_bit_cast(double, q);
}

// all-reduce over aligned groups of `width` lanes (a power of two <= 64)
template <typename T, typename Op>
__device__ inline T group_reduce(T v, Op op, int width)
{
    if (width > 1) v = op(v, xchg<0xB1>(v));   // quad_perm [1,0,3,2]
    if (width > 2) v = op(v, xchg<0x4E>(v));   // quad_perm [2,3,0,1]
    if (width > 4) v = op(v, xchg<0x141>(v));  // row_half_mirror
    if (width > 8) v = op(v, xchg<0x140>(v));  // row_mirror
    if (width > 16) {
        T a, b;
        swap<false>(v, a, b);
        v = op(a, b);
    }
    if (width > 32) {
        T a, b;
        swap<true>(v, a, b);
        v = op(a, b);
    }
    return v;
}

struct OpAdd {
    template <typename T>
    __device__ T operator()(T a, T b) const { return a + b; }
};
struct OpMax {
    __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

template <typename T>
__device__ inline T wave_sum(T v) { return group_reduce(v, OpAdd(), 64); }
__device__ inline float wave_max(float v) { return group_reduce(v, OpMax(), 64); }
__device__ inline float lane_group_sum(float v, int width) { return group_reduce(v, OpAdd(), width); }

// ---- token prep (the operand layout at the top of this file): one wave per
// (vector, group) writes the group's fp16 pairs and its stats (C, S, 2^e).
template <int BITS>
__device__ inline void prep_group(const float* __restrict__ v, int G, int vec, int g, int lane, uint4* __restrict__ q,
                                  float4* __restrict__ st, float scale = 1.f)
{
    const float val = v[(long long)vec * G * 64 + g * 64 + lane] * scale;
    const float amax = wave_max(fabsf(val));
    int e = 0;
    if (amax > 0.f && amax <= 3.4e38f) {
        e = ilogbf(amax) - 14;  // amax * 2^-e in [2^14, 2^15)
        e = e < -110 ? -110 : (e > 113 ? 113 : e);
    }
    const float vs = val * exp2i_f(-e);  // exact power-of-two scaling
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
    if (lane == 0) st[(long long)vec * G + g] = make_float4(C, S, exp2i_f(e), 0.f);
}

}  // namespace moe
