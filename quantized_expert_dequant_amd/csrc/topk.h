// topk.h - one wave selects the top-K of a token's logits (E <= 1024) and
// computes their softmax routing weights.  Used by the single-token router path
// and by the batched router.
#pragma once
#include "common.h"

namespace moe {

// Selection key of a logit: an order-preserving map of the double onto a
// 64-bit integer (larger logit, larger key) whose lowest 10 bits are replaced
// by 1023 - id.  One unsigned compare then ranks (logit desc, id asc); logits
// that agree to 2^-43 relative (below what fp64 summation order fixes) count
// as equal and go to the lower id.  Needs E <= 1024.
__device__ inline uint64_t select_key(double d, int id)
{
    const uint64_t u = (uint64_t)__double_as_longlong(d);
    const uint64_t k = (u >> 63) ? ~u : (u | 0x8000000000000000ull);
    return (k & ~1023ull) | (uint64_t)(1023 - id);
}
__device__ inline int key_id(uint64_t k) { return 1023 - (int)(k & 1023ull); }
__device__ inline double key_value(uint64_t k)  // the logit to within 2^-42 relative
{
    const uint64_t u = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
    return __longlong_as_double((long long)u);
}

// Load the logits a wave selects from: lane l holds ids l + 64 j, j < NL
// (clamped indices: every lane loads, the selection masks ids >= E).
template <int NL>
__device__ inline void topk_load(const double* __restrict__ lg, int E, int lane, double (&lv)[NL])
{
#pragma unroll
    for (int j = 0; j < NL; ++j) lv[j] = lg[min(lane + 64 * j, E - 1)];
}

struct OpU64Max {
    __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return b > a ? b : a; }
};

// Top-K of one token's E <= 64 * NL logits by one wave.  Lane k < K returns
// the k-th expert (rank order) and its routing weight; every lane sees the
// same selection.  All loops have compile-time trip counts, so the keys stay
// in registers.
template <int KMAX, int NL>
__device__ void topk_select(const double (&lv)[NL], int E, int K, int renorm, int lane, int& my_id, float& my_w)
{
    uint64_t key[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const int id = lane + 64 * j;
        key[j] = (id < E) ? select_key(lv[j], id) : 0ull;
    }
    uint64_t mine = 0ull, top = 0ull;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (k >= K) break;
        uint64_t t[NL];  // this lane's best remaining key: a tree over its candidates
#pragma unroll
        for (int j = 0; j < NL; ++j) t[j] = key[j];
#pragma unroll
        for (int w = 1; w < NL; w *= 2)
#pragma unroll
            for (int j = 0; j + w < NL; j += 2 * w) t[j] = t[j + w] > t[j] ? t[j + w] : t[j];
        const uint64_t best = group_reduce(t[0], OpU64Max(), 64);
#pragma unroll
        for (int j = 0; j < NL; ++j) key[j] = (key[j] == best) ? 0ull : key[j];  // keys are unique
        if (k == 0) top = best;
        if (lane == k) mine = best;
    }
    my_id = (lane < K) ? key_id(mine) : 0x7FFFFFFF;
    const double lmax = key_value(top);
    // softmax weights in fp32: exp of logit differences, renormalized over the K
    const float ew = (lane < K) ? __expf((float)(key_value(mine) - lmax)) : 0.f;
    float denom;
    if (renorm) {
        denom = wave_sum(ew);
    } else {
        float part = 0.f;
#pragma unroll
        for (int j = 0; j < NL; ++j)
            if (lane + 64 * j < E) part += __expf((float)(lv[j] - lmax));
        denom = wave_sum(part);
    }
    my_w = ew / denom;
}

}  // namespace moe
