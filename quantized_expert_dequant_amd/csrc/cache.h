// cache.h - host-side interface of the HBM expert cache (cache.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// bytes of the cache state for E routed experts and `slots` HBM slots
size_t cache_state_bytes(int E, int slots);
// every slot empty, counters zero
void launch_cache_reset(void* state, int E, int slots, hipStream_t s);
// the call's plan from the selected ids idx [n]: slot ids idx_slot [n] (-1 for ids
// outside [0, E)) and the copy list plan = [count, (expert, slot) x count]
// flags (nullable): per expert range flags [E + 1]; then slot_flags [slots + 1] receives
// them by slot (slot `slots`: the shared expert's)
// logits (nullable): [n / K][E] fp64; the plan first selects each token's top-K itself
// and writes idx [n] and the weights w [n] (needs n / K <= CP_ROUTE_MAX_B); without
// them idx is the caller's selection and w is not touched
constexpr int CP_ROUTE_MAX_B = 16;
void launch_cache_plan(int32_t* idx, int n, int E, int slots, void* state, int32_t* idx_slot, int32_t* plan,
                       long long record, const int32_t* flags, int32_t* slot_flags, const double* logits, int K,
                       int renorm, float* w, hipStream_t s);
// copy the planned records (at most max_copies) from src (device-accessible) into slab
void launch_cache_copy(const int32_t* plan, int max_copies, const void* src, void* slab, long long record,
                       hipStream_t s);

}  // namespace moe
