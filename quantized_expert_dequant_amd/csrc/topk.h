// topk.h - one wave selects the top-K of a token's logits (E <= 1024) and
// computes their softmax routing weights.  Used by the single-token router path
// and by the batched router.
#pragma once
#include "common.h"

namespace moe {

// Selection value of a logit: the double itself with its lowest 10 mantissa
// bits replaced by a code of the id, so that fp64 max/min alone rank
// (logit desc, id asc): 1023 - id for a non-negative logit, id for a negative
// one (there a larger magnitude is a smaller value).  Logits that agree but for
// those bits (2^-43 relative, below what the fp64 summation order fixes) count
// as equal and go to the lower id.  -0 is made +0 first, so the two zeros are
// one logit.  The value is the logit to within 2^-42 relative.  Needs E <= 1024.
__device__ inline double select_val(double d, int id)
{
    const uint64_t u = (uint64_t)__double_as_longlong(d + 0.0);
    const uint64_t t = (u >> 63) ? (uint64_t)id : (uint64_t)(1023 - id);
    return __longlong_as_double((long long)((u & ~1023ull) | t));
}
__device__ inline int val_id(double v)
{
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const int t = (int)(u & 1023ull);
    return (u >> 63) ? t : 1023 - t;
}

// Load the logits a wave selects from: lane l holds ids l + 64 j, j < NL
// (clamped indices: every lane loads, the selection masks ids >= E).
template <int NL>
__device__ inline void topk_load(const double* __restrict__ lg, int E, int lane, double (&lv)[NL])
{
#pragma unroll
    for (int j = 0; j < NL; ++j) lv[j] = lg[min(lane + 64 * j, E - 1)];
}

// fp64 max / min of selection values: one v_max_f64 / v_min_f64 each (the
// compiler adds a quieting max only for inputs it cannot prove NaN-free: the
// built values and the values taken from other lanes)
__device__ inline double sel_max(double a, double b) { return fmax(a, b); }
__device__ inline double sel_min(double a, double b) { return fmin(a, b); }
constexpr double SEL_NONE = -1.7976931348623157e308;  // below every selection value of a real logit

struct OpSelMax {
    __device__ double operator()(double a, double b) const { return sel_max(a, b); }
};

// compare-exchange: a takes the larger value (DESC) or the smaller one
template <bool DESC>
__device__ inline void cmp_xchg(double& a, double& b)
{
    const double hi = sel_max(a, b), lo = sel_min(a, b);
    a = DESC ? hi : lo;
    b = DESC ? lo : hi;
}

// bitonic sort of v[0..N) into descending order (N a power of two)
template <int N>
__device__ inline void sort_desc(double* v)
{
#pragma unroll
    for (int k = 2; k <= N; k *= 2)
#pragma unroll
        for (int j = k / 2; j > 0; j /= 2)
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int l = i ^ j;
                if (l > i) {
                    if ((i & k) == 0)
                        cmp_xchg<true>(v[i], v[l]);
                    else
                        cmp_xchg<false>(v[i], v[l]);
                }
            }
}

// a[0..P) and b[0..P) sorted descending -> a = the P largest of both, sorted
// descending: max(a_i, b_{P-1-i}) is bitonic, then one bitonic merge
template <int P>
__device__ inline void merge_top(double* a, const double* b)
{
#pragma unroll
    for (int i = 0; i < P; ++i) a[i] = sel_max(a[i], b[P - 1 - i]);
#pragma unroll
    for (int j = P / 2; j > 0; j /= 2)
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int l = i ^ j;
            if (l > i) cmp_xchg<true>(a[i], a[l]);
        }
}

// The rounds of the top-K of one token's E <= 64 * NL logits by one wave.  Each
// lane first sorts its own candidates (it can give at most P = min(KMAX, NL) of
// the K), then every round takes the wave maximum of the lanes' heads and the
// lane that held it drops its head.  After `rounds` (<= KMAX) rounds every lane
// has `top` (the largest value) and `last` (the value of the last round), and
// lane k < rounds has `mine`, the value of round k.  All loops have compile-time
// trip counts, so the values stay in registers.
template <int KMAX, int NL>
__device__ inline void topk_rounds(const double (&lv)[NL], int E, int rounds, int lane, double& mine, double& top,
                                   double& last)
{
    constexpr int P = KMAX < NL ? KMAX : NL;
    constexpr int PP = (P <= 1) ? 1 : (P <= 2) ? 2 : (P <= 4) ? 4 : (P <= 8) ? 8 : 16;  // power of two >= P
    static_assert(NL % PP == 0, "candidates per lane: a multiple of the sorted run");
    double v[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const int id = lane + 64 * j;
        const double s = select_val(lv[j], id);
        v[j] = (id < E) ? s : SEL_NONE;
    }
    // this lane's P best, descending: sorted runs of PP merged pairwise
#pragma unroll
    for (int r = 0; r < NL; r += PP) sort_desc<PP>(v + r);
#pragma unroll
    for (int r = PP; r < NL; r += PP) merge_top<PP>(v, v + r);
    mine = 0.0;
    top = 0.0;
    last = 0.0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (k >= rounds) break;
        const double best = group_reduce(v[0], OpSelMax(), 64);
        const bool win = __double_as_longlong(v[0]) == __double_as_longlong(best);  // values are unique
#pragma unroll
        for (int i = 0; i + 1 < P; ++i) v[i] = win ? v[i + 1] : v[i];
        v[P - 1] = win ? SEL_NONE : v[P - 1];
        if (k == 0) top = best;
        if (lane == k) mine = best;
        last = best;
    }
}

// Top-K of one token's logits by one wave.  Lane k < K returns the k-th expert
// (rank order) and its routing weight; every lane sees the same selection.
template <int KMAX, int NL>
__device__ void topk_select(const double (&lv)[NL], int E, int K, int renorm, int lane, int& my_id, float& my_w)
{
    double mine, top, last;
    topk_rounds<KMAX, NL>(lv, E, K, lane, mine, top, last);
    my_id = (lane < K) ? val_id(mine) : 0x7FFFFFFF;
    // softmax weights in fp32: exp of logit differences, renormalized over the K
    const float ew = (lane < K) ? __expf((float)(mine - top)) : 0.f;
    float denom;
    if (renorm) {
        denom = wave_sum(ew);
    } else {
        float part = 0.f;
#pragma unroll
        for (int j = 0; j < NL; ++j)
            if (lane + 64 * j < E) part += __expf((float)(lv[j] - top));
        denom = wave_sum(part);
    }
    my_w = ew / denom;
}

// The expert of rank r < KMAX (0: the largest logit) alone: r + 1 rounds.
template <int KMAX, int NL>
__device__ inline int topk_nth(const double (&lv)[NL], int E, int r, int lane)
{
    double mine, top, last;
    topk_rounds<KMAX, NL>(lv, E, r + 1, lane, mine, top, last);
    return val_id(last);
}

}  // namespace moe
