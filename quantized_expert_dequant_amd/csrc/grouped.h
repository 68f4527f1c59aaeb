// grouped.h - host-side interface of the batched decode path (grouped.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"
#include "common.h"
#include "launch.h"

namespace moe {

// Output of the grouping kernel.  offsets / tokens / slots: the assignments of
// expert e are positions [offsets[e], offsets[e+1]) of tokens (token id) and
// slots (slot b*K + k), in slot order.  The rest is the work list and may be
// null together.  The entries (0 .. B-1: the shared expert's, one per token;
// B + p: position p of the sort) of an expert with fewer than gv_t tokens form
// one GEMV group; a larger expert's are cut into MFMA groups of at most 32
// entries.  Each list holds the shared expert first (if it falls in it), then
// the routed experts by id.  MFMA group v (v < grp_u[0]) is expert
// act_expert[v] with entries act_off[v] .. act_off[v] + act_n[v] - 1, GEMV
// group v (v < grp_u[1]) likewise with gv_expert / gv_off / gv_n; the entries'
// tokens are ent_token[]; slot_pos[b*K + k] = entry of that slot (-1: invalid id).
struct GroupOut {
    int32_t* offsets;     // [E + 1]
    int32_t* tokens;      // [B*K]
    int32_t* slots;       // [B*K]
    int32_t* grp_u;       // [2]: MFMA groups, GEMV groups
    int32_t* act_expert;  // [V]
    int32_t* act_off;     // [V]
    int32_t* act_n;       // [V]
    int32_t* gv_expert;   // [V]
    int32_t* gv_off;      // [V]
    int32_t* gv_n;        // [V]
    int32_t* ent_token;   // [B + B*K]
    int32_t* slot_pos;    // [B*K]
};

// Workspace of the batched path, carved from the caller's buffer.
struct GroupedWork {
    double* partial;  // router partial logits [splits][B][E]
    GroupOut g;
    uint4* xh;        // MFMA token operands: x * 2^-e minus its chunk mean, as fp16 in chunk order [B][2 G_h][4] uint4
    uint2* xsum;      // per chunk: 2^-5 * sum as fp16 (hi, lo), and the fp16 pair (2m, 2m) of the
                      // chunk mean m the operands are deviations from [B][2 G_h]
    float* xscale;    // [B]
    float* hb;        // h in fp32, pair-layout order [B + B*K][8][G_i][8]
    uint4* hb16;      // h * 2^-e(entry) as fp16 pairs in chunk order [B + B*K][2 G_i][4]:
                      // uint4 (c, d) holds pairs 4(4(c / G_i) + d) .. +3 of group c % G_i
    float* hscale;    // 2^e(entry) [B + B*K]
    float4* hstats;   // per group of hb16: (C, S, scale, 0) for the dot2 GEMV [B + B*K][G_i]
    float* part;      // down outputs [B + B*K][H]
    float* split;     // partial gate/up sums of tiles split between blocks
};

bool grouped_supported(const Layout& L, int B, int K);
// blocks of the batched launches on the current device (each as many as stay resident)
struct GroupedBlocks {
    int gateup, down, gemv_gateup, gemv_down;
    int gateup2, down2;  // the 2-bit matrix-core launches
    int gateup3, down3;  // the 3-bit matrix-core launches
};
GroupedBlocks grouped_blocks();
// MFMA tiles of one work-list group (128 output rows) in the gate/up and the down phase
int grouped_tiles(const Layout& L, int down);
// K chunks a gate/up tile is cut into when the tiles outnumber the gate/up blocks
int grouped_gateup_chunks();
// most tokens of one matrix-core work-list group
int grouped_group_tokens();
size_t grouped_workspace_bytes(const Layout& L, int B, int K, int E);
GroupedWork carve_grouped(void* base, const Layout& L, int B, int K, int E);
int router_splits(int H);
// Token operands the batched top-K kernel writes beside the selection (xh
// nullptr: none; xq nullptr: no dot2 operand).  x and H are filled in by
// launch_route_batched.
struct TokenPrep {
    const float* x;
    int H;
    uint4* xh;
    uint2* xsum;
    float* xscale;
    uint4* xq;
    float4* xst;
};
void launch_route_batched(const float* x, int B, const float* W, const float* bias, int H, int E, int K, int renorm,
                          double* partial, int32_t* idx, float* w, const TokenPrep& P, hipStream_t s, Timing t);
// experts with fewer tokens than this run as GEMV groups (1: none)
int gemv_tokens(const Layout& L);
// flags (nullable): per expert (index E: the shared one), nonzero = run it as GEMV groups
void launch_group(const int32_t* idx, int B, int K, int E, int gv_tokens, const int32_t* flags, const GroupOut& O,
                  hipStream_t s);
// flags[e] of records [0, n): 1 if a scale or bias lies outside the matrix-core path's range
void launch_expert_ranges(const Layout& L, const void* slab, int n, int32_t* flags, hipStream_t s);
// xq / xst: room for the B tokens' dot2 operands (fp16 pairs + group stats)
// prepped: the token operands are already written (by the batched top-K kernel)
void launch_ffn_grouped(const Layout& L, const void* slab, const GroupedWork& W, const float* x, const float* w,
                        float shared_w, int B, int K, int E, uint4* xq, float4* xst, bool prepped, float* y,
                        hipStream_t s, Timing tg, Timing td);

}  // namespace moe
