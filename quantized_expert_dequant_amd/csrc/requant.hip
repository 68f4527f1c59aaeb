// requant.hip - offline requantization of 4-bit experts to 2-bit on the GPU.
//
// Pages (titles as published):
//   [CLAUDAY] clauday.com, "Flash-MoE: Running a 397B Parameter Model on a MacBook
//             with Pure C and Metal"
//   [LLMAPIS] llmapis.com, "Flash-MoE：把 397B MoE 真正跑进消费级笔记本，意味着
//             '大模型本地化'开始从演示走向系统工程"
//
// The pages report that the experts were requantized from 4-bit to 2-bit, the
// expert files shrinking from 209 GB to 120 GB ([CLAUDAY]; [LLMAPIS] section
// 数据和技术细节), and give no procedure.  This library's reading is a per-group
// min/max affine refit of the dequantized 4-bit weights: for the weights of a
// group (64, 128 or 256), w_c = s4 q4_c + b4 (exact in double), b2 = bf16(min w), s2 =
// bf16((max w - min w) / 3), q2_c = clamp(rint((w_c - b2) / s2), 0, 3) (0 when
// s2 = 0 or when the quotient is not a number), every operation in IEEE double and bf16() one rounding of the double
// to the nearest bf16, ties to even.  The integer codes follow from these
// operations alone, so any implementation that performs them gets the same codes.
//
// Input and output are in the canonical format (moe_pack_experts): the output is
// a 2-bit canonical expert set of the same shape, ready to be packed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace moe {

// Nearest bf16 of a double, ties to even, by integer arithmetic on the double's
// bits: the 53-bit significand is cut to the bf16 quantum of its binade (8
// significant bits; 2^-133 below 2^-126), rounded half to even on the dropped
// bits, and the kept count becomes the bf16 bits directly (a carry into the next
// binade, or out of the subnormals, lands in the exponent field by addition).
__device__ inline uint16_t bf16_nearest_even(double v)
{
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
    if (a > 0x7FF0000000000000ull) return 0x7FC0;          // NaN
    if (a == 0x7FF0000000000000ull) return sign | 0x7F80;  // infinity
    const int bexp = (int)(a >> 52);
    if (bexp == 0) return sign;  // double subnormals lie far below half the smallest bf16
    const int e = bexp - 1023;                             // v = M * 2^(e - 52), M in [2^52, 2^53)
    const uint64_t M = (a & 0xFFFFFFFFFFFFFull) | (1ull << 52);
    const int qe = e >= -126 ? e - 7 : -133;               // the bf16 quantum of this binade
    const int shift = qe - (e - 52);                       // dropped significand bits, >= 45
    if (shift >= 54) return sign;                          // below half the quantum
    uint64_t R = M >> shift;
    const uint64_t rem = M & ((1ull << shift) - 1ull), half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (R & 1ull))) R += 1ull;
    uint32_t bits;
    if (e >= -126)
        bits = (uint32_t)((e + 127) << 7) + (uint32_t)R - 128u;  // R in [128, 256]
    else
        bits = (uint32_t)R;                                        // subnormal, R in [0, 128]
    if (bits >= 0x7F80u) bits = 0x7F80u;                           // past the largest bf16
    return (uint16_t)(sign | bits);
}

__device__ inline double bf16_to_f64(uint16_t b) { return (double)__uint_as_float((uint32_t)b << 16); }

// One thread per group of 64 << gs weights: 32 << gs bytes of 4-bit codes in, 16 << gs
// bytes of 2-bit codes out, in units of 64 weights (two passes: the extremes, then the
// codes).  Group t of expert j: gate groups [0, I*Sh), up groups [I*Sh, 2*I*Sh), down
// groups after (Sh, Si: groups per gate/up and per down row).
__global__ __launch_bounds__(256) void k_requant(int H, int I, int gs, const uint8_t* __restrict__ gate4,
                                                 const uint8_t* __restrict__ up4, const uint8_t* __restrict__ down4,
                                                 const uint16_t* __restrict__ s4, const uint16_t* __restrict__ b4,
                                                 uint8_t* __restrict__ gate2, uint8_t* __restrict__ up2,
                                                 uint8_t* __restrict__ down2, uint16_t* __restrict__ s2,
                                                 uint16_t* __restrict__ b2)
{
    const int j = blockIdx.y, nu = 1 << gs;  // 64-weight units per group
    const long long Sh = (H / 64) >> gs, Si = (I / 64) >> gs;
    const long long ngu = (long long)I * Sh, ng = 2 * ngu + (long long)H * Si;
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= ng) return;
    // the group's 4-bit codes and 2-bit destination, canonical order
    const uint8_t* src;
    uint8_t* dst;
    if (t < 2 * ngu) {
        const bool up = t >= ngu;
        const long long gi = up ? t - ngu : t;  // r * Sh + group
        const long long off4 = (long long)j * I * (H / 2) + gi * 32 * nu, off2 = (long long)j * I * (H / 4) + gi * 16 * nu;
        src = (up ? up4 : gate4) + off4;
        dst = (up ? up2 : gate2) + off2;
    } else {
        const long long gi = t - 2 * ngu;  // r * Si + group
        src = down4 + (long long)j * H * (I / 2) + gi * 32 * nu;
        dst = down2 + (long long)j * H * (I / 4) + gi * 16 * nu;
    }
    const long long si = (long long)j * ng + t;
    const double s = bf16_to_f64(s4[si]), b = bf16_to_f64(b4[si]);
    double lo = 0.0, hi = 0.0;
    for (int u = 0; u < nu; ++u) {
        const uint4 c0 = *reinterpret_cast<const uint4*>(src + 32 * u), c1 = *reinterpret_cast<const uint4*>(src + 32 * u + 16);
        const uint32_t words[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int k = 0; k < 64; ++k) {
            const double w = s * (double)((words[k >> 3] >> (4 * (k & 7))) & 15u) + b;
            lo = (u == 0 && k == 0) ? w : fmin(lo, w);
            hi = (u == 0 && k == 0) ? w : fmax(hi, w);
        }
    }
    const uint16_t nb = bf16_nearest_even(lo), ns = bf16_nearest_even((hi - lo) / 3.0);
    const double bd = bf16_to_f64(nb), sd = bf16_to_f64(ns);
    for (int u = 0; u < nu; ++u) {
        const uint4 c0 = *reinterpret_cast<const uint4*>(src + 32 * u), c1 = *reinterpret_cast<const uint4*>(src + 32 * u + 16);
        const uint32_t words[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < 64; ++k) {
            const double w = s * (double)((words[k >> 3] >> (4 * (k & 7))) & 15u) + b;
            uint32_t q = 0u;
            if (sd != 0.0) {
                const double r = rint((w - bd) / sd);
                q = r >= 3.0 ? 3u : (r > 0.0 ? (uint32_t)r : 0u);  // a quotient that is not a number gives 0
            }
            out[k >> 4] |= q << (2 * (k & 15));
        }
        *reinterpret_cast<uint4*>(dst + 16 * u) = make_uint4(out[0], out[1], out[2], out[3]);
    }
    s2[si] = ns;
    b2[si] = nb;
}

void launch_requant_4to2(int H, int I, int group, int n, const uint8_t* gate4, const uint8_t* up4,
                         const uint8_t* down4, const uint16_t* s4, const uint16_t* b4, uint8_t* gate2, uint8_t* up2,
                         uint8_t* down2, uint16_t* s2, uint16_t* b2, hipStream_t s)
{
    const int gs = group >= 256 ? 2 : (group >= 128 ? 1 : 0);
    const long long ng = 2LL * I * ((H / 64) >> gs) + (long long)H * ((I / 64) >> gs);
    hipLaunchKernelGGL(k_requant, dim3((unsigned)((ng + 255) / 256), n), dim3(256), 0, s, H, I, gs, gate4, up4,
                       down4, s4, b4, gate2, up2, down2, s2, b2);
}

}  // namespace moe
