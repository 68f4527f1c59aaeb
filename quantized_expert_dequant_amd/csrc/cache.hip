// cache.hip - tiered expert residency: an HBM cache of expert records over a
// backing store in pinned host memory, filled by the GPU itself.
//
// Pages (titles as published):
//   [LLMAPIS] llmapis.com, "Flash-MoE：把 397B MoE 真正跑进消费级笔记本，意味着
//             '大模型本地化'开始从演示走向系统工程"
//   [ACGFAV]  acgfav.com, "iPhone 17 Pro也能跑近400B大模型？Flash-MoE把端侧AI推到新极限"
//
// The pages' engine keeps only the active experts near the processor: per layer
// it reads the K selected experts (about 6.75 MB each) from the SSD and lets the
// OS page cache decide what stays in memory ([LLMAPIS] section 深度分析; [ACGFAV]
// section 到底做了什么).  Here the tiers are HBM and pinned host memory: every
// packed record of a layer lives in host memory, and `slots` records plus the
// shared expert live in HBM.  After the router has selected the experts, one
// block plans the call (hits refresh their slot's stamp; each miss takes the
// least recently used slot that this call does not use, ties to the lowest slot,
// misses in ascending expert id), a copy kernel pulls the missing records across
// PCIe straight from host memory, and the expert FFNs run on the cache with slot
// ids.  Everything is enqueued on the caller's stream: the host never waits for
// the routing, so a call can be captured in a HIP graph.
//
// State (device, caller-owned, moe_cache_state_bytes):
//   u64 counters[4]: hits, misses, bytes copied, calls   (offset 0)
//   u32 clock (calls so far + 1)                           (offset 32)
//   i32 slot_of[E], i32 expert_of[slots], u32 last_use[slots]  (from offset 64)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cache.h"
#include "topk.h"

namespace moe {

struct CacheView {
    unsigned long long* counters;
    uint32_t* clock;
    int32_t* slot_of;
    int32_t* expert_of;
    uint32_t* last_use;
};

__host__ __device__ inline size_t up256c(size_t n) { return (n + 255) & ~(size_t)255; }

size_t cache_state_bytes(int E, int slots)
{
    return 64 + up256c(4ull * E) + up256c(4ull * slots) + up256c(4ull * slots);
}

__host__ __device__ inline CacheView cache_view(void* state, int E, int slots)
{
    char* p = (char*)state;
    CacheView v;
    v.counters = (unsigned long long*)p;
    v.clock = (uint32_t*)(p + 32);
    v.slot_of = (int32_t*)(p + 64);
    v.expert_of = (int32_t*)(p + 64 + up256c(4ull * E));
    v.last_use = (uint32_t*)(p + 64 + up256c(4ull * E) + up256c(4ull * slots));
    return v;
}

__global__ __launch_bounds__(256) void k_cache_reset(void* state, int E, int slots)
{
    const CacheView v = cache_view(state, E, slots);
    const int t = blockIdx.x * 256 + threadIdx.x, nt = gridDim.x * 256;
    if (t < 4) v.counters[t] = 0ull;
    if (t == 0) *v.clock = 1u;
    for (int e = t; e < E; e += nt) v.slot_of[e] = -1;
    for (int s = t; s < slots; s += nt) {
        v.expert_of[s] = -1;
        v.last_use[s] = 0u;
    }
}

void launch_cache_reset(void* state, int E, int slots, hipStream_t s)
{
    int blocks = (max(E, slots) + 255) / 256;
    hipLaunchKernelGGL(k_cache_reset, dim3(blocks < 1 ? 1 : blocks), dim3(256), 0, s, state, E, slots);
}

// One block: the call's plan.  The selection idx [n] (n = B*K, ids outside [0, E)
// are passed through as -1) is given, or, with logits (B <= CP_ROUTE_MAX_B tokens),
// selected here first: wave b takes token b's top-K and softmax weights as the
// route-only kernel does, writes them to idx and w, and the plan reads them from
// LDS, which saves that launch.  Writes idx_slot [n], the copy list (expert, slot)
// [n] and its length at plan[0].  Needs E <= MOE_MAX_E and as many free slots as
// misses (the caller guarantees slots >= min(E, n)).
constexpr int CP_THREADS = 1024;
static_assert(CP_THREADS >= MOE_MAX_E, "one thread per expert in the miss scan");
static_assert(CP_ROUTE_MAX_B <= CP_THREADS / 64, "one wave per token selected in the plan");

__global__ __launch_bounds__(CP_THREADS) void k_cache_plan(int32_t* __restrict__ idx, int n, int E, int slots,
                                                          void* state, int32_t* __restrict__ idx_slot,
                                                          int32_t* __restrict__ plan, unsigned long long record,
                                                          const int32_t* __restrict__ flags,
                                                          int32_t* __restrict__ slot_flags,
                                                          const double* __restrict__ logits, int K, int renorm,
                                                          float* __restrict__ w)
{
    __shared__ uint32_t sel[MOE_MAX_E / 32];
    __shared__ int miss[MOE_MAX_E];
    __shared__ int n_miss, n_hit;
    __shared__ int wcount[CP_THREADS / 64];
    __shared__ int sidx[CP_ROUTE_MAX_B * MOE_MAX_K];
    __shared__ unsigned long long red_key[CP_THREADS / 64];
    const CacheView v = cache_view(state, E, slots);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t clock = *v.clock;
    const bool route = logits != nullptr;
    if (route && wave < n / K) {  // token `wave`'s selection (wave-uniform)
        int id;
        float wt;
        double lv[16];
        topk_load<16>(logits + (long long)wave * E, E, lane, lv);
        topk_select<32, 16>(lv, E, K, renorm, lane, id, wt);
        if (lane < K) {
            idx[wave * K + lane] = id;
            w[wave * K + lane] = wt;
            sidx[wave * K + lane] = id;
        }
    }
    for (int i = tid; i < MOE_MAX_E / 32; i += CP_THREADS) sel[i] = 0u;
    if (tid == 0) n_hit = 0;
    __syncthreads();
    auto idx_at = [&](int i) { return route ? sidx[i] : idx[i]; };
    for (int i = tid; i < n; i += CP_THREADS) {
        const int e = idx_at(i);
        if (e >= 0 && e < E) atomicOr(&sel[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
    // hits refresh their slot; each thread counts its own
    int hits = 0;
    for (int e = tid; e < E; e += CP_THREADS) {
        if (!((sel[e >> 5] >> (e & 31)) & 1u)) continue;
        const int s = v.slot_of[e];
        if (s >= 0) {
            v.last_use[s] = clock;
            ++hits;
        }
    }
    if (hits) atomicAdd(&n_hit, hits);
    __syncthreads();
    // the misses in ascending expert id: thread e tests expert e, each wave counts its
    // misses with a ballot, and a miss's place is the misses of the lower waves and lanes
    const bool is_miss = tid < E && ((sel[tid >> 5] >> (tid & 31)) & 1u) && v.slot_of[tid] < 0;
    const unsigned long long bal = __ballot(is_miss);
    if (lane == 0) wcount[wave] = __popcll(bal);
    __syncthreads();
    {
        int base = 0, total = 0;
        for (int q = 0; q < CP_THREADS / 64; ++q) {
            base += q < wave ? wcount[q] : 0;
            total += wcount[q];
        }
        if (is_miss) miss[base + __popcll(bal & ((1ull << lane) - 1ull))] = tid;
        if (tid == 0) n_miss = total;
    }
    __syncthreads();
    const int nm = n_miss;
    for (int m = 0; m < nm; ++m) {
        // the least recently used slot not used by this call: smallest (last_use, slot)
        unsigned long long best = ~0ull;
        for (int s = tid; s < slots; s += CP_THREADS) {
            const uint32_t lu = v.last_use[s];
            if (lu < clock) {
                const unsigned long long key = ((unsigned long long)lu << 32) | (unsigned)s;
                best = key < best ? key : best;
            }
        }
        for (int off = 32; off >= 1; off >>= 1) {
            const unsigned long long o = __shfl_xor(best, off);
            best = o < best ? o : best;
        }
        if (lane == 0) red_key[wave] = best;
        __syncthreads();
        if (tid == 0) {
            unsigned long long b = red_key[0];
            for (int w = 1; w < CP_THREADS / 64; ++w) b = red_key[w] < b ? red_key[w] : b;
            const int e = miss[m];
            if (b == ~0ull) {  // no free slot: the caller broke the slots >= n guarantee
                plan[1 + 2 * m] = e;
                plan[2 + 2 * m] = -1;
            } else {
                const int s = (int)(b & 0xFFFFFFFFu);
                const int old = v.expert_of[s];
                if (old >= 0) v.slot_of[old] = -1;
                v.expert_of[s] = e;
                v.slot_of[e] = s;
                v.last_use[s] = clock;
                plan[1 + 2 * m] = e;
                plan[2 + 2 * m] = s;
            }
        }
        __syncthreads();
    }
    for (int i = tid; i < n; i += CP_THREADS) {
        const int e = idx_at(i);
        idx_slot[i] = (e >= 0 && e < E) ? v.slot_of[e] : -1;
    }
    if (flags) {  // the range flags by slot, the shared expert's last
        for (int sl = tid; sl <= slots; sl += CP_THREADS) {
            const int e = sl < slots ? v.expert_of[sl] : E;
            slot_flags[sl] = e >= 0 ? flags[e] : 0;
        }
    }
    if (tid == 0) {
        plan[0] = nm;
        v.counters[0] += (unsigned long long)n_hit;
        v.counters[1] += (unsigned long long)nm;
        v.counters[2] += (unsigned long long)nm * record;
        v.counters[3] += 1ull;
        *v.clock = clock + 1u;
    }
}

// Copy the planned records: block (i, c) copies chunk c of copy i (if i < count)
// from the backing store (device-accessible host memory) into its slot.
constexpr int CC_CHUNK = 64 * 1024;  // bytes per block

__global__ __launch_bounds__(256) void k_cache_copy(const int32_t* __restrict__ plan, const uint8_t* __restrict__ src,
                                                    uint8_t* __restrict__ slab, long long record)
{
    const int i = blockIdx.y;
    if (i >= plan[0]) return;
    const int e = plan[1 + 2 * i], s = plan[2 + 2 * i];
    if (s < 0) return;
    const long long begin = (long long)blockIdx.x * CC_CHUNK;
    const long long end = begin + CC_CHUNK < record ? begin + CC_CHUNK : record;
    const uint4* from = reinterpret_cast<const uint4*>(src + (long long)e * record);
    uint4* to = reinterpret_cast<uint4*>(slab + (long long)s * record);
    for (long long o = begin / 16 + threadIdx.x; o < end / 16; o += 256) to[o] = from[o];
}

void launch_cache_plan(int32_t* idx, int n, int E, int slots, void* state, int32_t* idx_slot, int32_t* plan,
                       long long record, const int32_t* flags, int32_t* slot_flags, const double* logits, int K,
                       int renorm, float* w, hipStream_t s)
{
    hipLaunchKernelGGL(k_cache_plan, dim3(1), dim3(CP_THREADS), 0, s, idx, n, E, slots, state, idx_slot, plan,
                       (unsigned long long)record, flags, slot_flags, logits, K, renorm, w);
}

void launch_cache_copy(const int32_t* plan, int max_copies, const void* src, void* slab, long long record,
                       hipStream_t s)
{
    const unsigned chunks = (unsigned)((record + CC_CHUNK - 1) / CC_CHUNK);
    hipLaunchKernelGGL(k_cache_copy, dim3(chunks, max_copies), dim3(256), 0, s, plan, (const uint8_t*)src,
                       (uint8_t*)slab, record);
}

}  // namespace moe
