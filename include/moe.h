/*
 * moe.h - C ABI of libmoe.so: per-token decode of one quantized
 * Mixture-of-Experts layer on an AMD Instinct MI355X (gfx950).
 *
 * Pages that define the operation (titles as published):
 *   [LLMAPIS] llmapis.com, "Flash-MoE：把 397B MoE 真正跑进消费级笔记本，意味着
 *             '大模型本地化'开始从演示走向系统工程"
 *   [MFFB]    f.mffb.com.cn, Flash-MoE article ("HN上281票 ... 8200行纯C代码 ...")
 *   [CLAUDAY] clauday.com, "Flash-MoE: Running a 397B Parameter Model on a
 *             MacBook with Pure C and Metal"
 *
 * The layer ([LLMAPIS] section 深度分析): a router picks K of E experts per
 * token (E = 512, K = 4, plus one always-on shared expert), the active experts'
 * quantized weights are read and dequantized, each expert's FFN is computed,
 * and the results are combined with the routing weights.  Expert weights are
 * 4-bit or 2-bit codes (3-bit also built) with a per-group scale and bias ([LLMAPIS] sections
 * 为什么值得关注 and 深度分析); the router stays at full precision
 * ([CLAUDAY]).  Readings this library fixes where the pages are silent:
 * w = s*q + b with unsigned q, bf16 s and b per group of 64 (or 128, 256)
 * consecutive weights along each row's input dimension; SwiGLU experts h = silu(Wg x) * (Wu x),
 * y_e = Wd h; softmax over all E, keep the top K (ties to the lower id,
 * output in rank order), renormalize; y = sum_k w_k y_{idx_k} +
 * shared_weight * y_shared.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are device pointers to caller-owned memory (e.g. torch
 *     tensors' data_ptr()), unless stated otherwise.  Pointers must be 16-byte
 *     aligned, except routing buffers (idx, w) and logit_bias, which need 4
 *     bytes.  The library keeps no pointer after a call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously; no call synchronizes the host and none
 *     allocates device or pinned memory.
 *   - Scratch memory is a caller-provided workspace `ws` of at least the
 *     size the matching *_workspace_bytes query returns; its contents need no
 *     initialization.  Calls that share a workspace must be ordered on one
 *     stream.
 *   - Return value: MOE_OK, or a negative MOE_E* code.  On an error return
 *     nothing has been enqueued and no output has been written;
 *     moe_last_error() describes the failure (thread-local).  Faults inside
 *     kernels surface at the caller's next synchronization.
 *   - Expert ids handed to moe_expert_ffn_* that are outside [0, E) make that
 *     token's output NaN (they are never dereferenced).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_EINVAL (-1)        /* null / misaligned pointer, bad shape, workspace too small */
#define MOE_EUNSUPPORTED (-2)  /* bits not 2, 3 or 4, group not 64/128/256, K > 32, E > 1024, B > 256, H > 65536, I > 8192 */
#define MOE_EHIP (-3)          /* the HIP runtime refused a launch */

#define MOE_MAX_K 32
#define MOE_MAX_E 1024
#define MOE_MAX_B 256

/*
 * One MoE layer.  All pointers are device memory owned by the caller.
 *   H: hidden size, I: expert intermediate size (both multiples of the group).
 *   E: routed experts, K: experts kept per token, bits: 4, 3 or 2 (3-bit: I a
 *   multiple of 128), group: weights per
 *   scale/bias group along each row, 64, 128 or 256 (the pages give per-group
 *   scales and biases, [LLMAPIS] section 深度分析, without a size).
 *   experts: packed slab of E + 1 records written by moe_pack_experts, the
 *            shared expert at index E; record stride moe_expert_record_bytes().
 *   w_router: fp32 [E][H] row-major.  logit_bias: fp32 [E] added to the
 *            logits before selection (e.g. a prior over expert ids), or NULL.
 *   shared_weight: factor of the shared expert in the combine (1.0 = plain sum).
 *   renormalize: 1 = routing weights renormalized over the kept K; 0 = raw
 *            softmax probabilities over all E.
 *   expert_flags: int32 [E + 1] as written by moe_expert_ranges, or NULL.  With
 *            it, batches route experts flagged as holding scales or biases beyond
 *            the matrix cores' range to the fp32-scaled GEMV path; without it the
 *            range limit of moe_layer_decode applies.
 */
typedef struct moe_layer_desc {
    int32_t H, I, E, K, bits, group;
    const void* experts;
    const float* w_router;
    const float* logit_bias;
    float shared_weight;
    int32_t renormalize;
    const int32_t* expert_flags;
} moe_layer_desc;

/*
 * Bytes of one packed expert record: gate and up [I][H] plus down [H][I]
 * codes at `bits` per weight, plus a bf16 scale and bias per group of `group`
 * weights.  Equal to the canonical size of one expert, e.g. 7,077,888 B
 * (6.75 MiB) at H = 4096, I = 1024, 4-bit, group 64 ([LLMAPIS] section 深度分析
 * gives about 6.75MB per expert).  Returns 0 for unsupported arguments.
 */
size_t moe_expert_record_bytes(int bits, int H, int I, int group);

/*
 * Workspace bytes needed by moe_layer_decode / moe_expert_ffn_* for B tokens
 * (and by moe_stack_decode, which needs the same).  The workspace holds what
 * passes between the steps of the layer ([LLMAPIS] section 深度分析: routing,
 * reading, dequantization, local compute, combine): the logits and routing, the
 * token's dequant operand (scale*x / bias*x folded per group), h of every
 * active expert and, for batches, the grouping and per-expert partial outputs.
 * 0 on an invalid desc or B (moe_last_error says why).
 */
size_t moe_workspace_bytes(const moe_layer_desc* desc, int B);

/* Workspace bytes needed by moe_route_topk: the fp64 logits of B tokens over E
 * experts ([LLMAPIS] section 深度分析, the routing step).  0 on invalid arguments. */
size_t moe_route_workspace_bytes(int B, int E, int K);

/*
 * Pack n_experts experts from the canonical format into records
 * [first_expert, first_expert + n_experts) of `slab_out`.
 * Canonical inputs (device, stacked over the n experts):
 *   gate_codes, up_codes: uint8 [n][I][H*bits/8]; down_codes: uint8 [n][H][I*bits/8]
 *     (4-bit: element 2j is the low nibble of byte j; 2-bit: element 4j+t sits
 *     at bits 2t..2t+1 of byte j; 3-bit: each row is one little-endian bit
 *     string with element c at bits 3c..3c+2);
 *   scales_bf16, biases_bf16: uint16 bf16 bit patterns [n][ng], per expert
 *     concatenated gate [I][H/group] | up [I][H/group] | down [H][I/group].
 * The record layout is private to the library ([LLMAPIS] section 深度分析:
 * each expert is fetched as one unit; here one contiguous record).
 * slab_out must hold at least (first_expert + n_experts) records.
 */
int moe_pack_experts(int bits, int H, int I, int group, int n_experts, const uint8_t* gate_codes,
                     const uint8_t* up_codes, const uint8_t* down_codes,
                     const uint16_t* scales_bf16, const uint16_t* biases_bf16, void* slab_out,
                     int first_expert, void* stream);

/*
 * Offline requantization of n_experts canonical 4-bit experts to canonical 2-bit
 * experts of the same shape ([CLAUDAY] and [LLMAPIS] section 数据和技术细节: the
 * experts were requantized from 4-bit to 2-bit, 209 GB -> 120 GB; the pages give no
 * procedure).  Per group of `group` weights w_c = s4 q4_c + b4: b2 = bf16(min w),
 * s2 = bf16((max w - min w) / 3), q2_c = clamp(rint((w_c - b2) / s2), 0, 3) (0 when
 * s2 = 0 or the quotient is not a number), every operation in IEEE double and bf16() the nearest bf16, ties to even.
 * Inputs: the canonical 4-bit tensors as for moe_pack_experts (device, stacked
 * over the n experts); outputs: gate2, up2 uint8 [n][I][H/4], down2 [n][H][I/4],
 * scales2, biases2 uint16 [n][ng] in the same order as the inputs' scales.  The
 * result is packed with moe_pack_experts(bits = 2).  MOE_EINVAL / MOE_EUNSUPPORTED
 * as for moe_pack_experts.
 */
int moe_requant_4to2(int H, int I, int group, int n_experts, const uint8_t* gate4, const uint8_t* up4,
                     const uint8_t* down4, const uint16_t* scales4, const uint16_t* biases4, uint8_t* gate2,
                     uint8_t* up2, uint8_t* down2, uint16_t* scales2, uint16_t* biases2, void* stream);

/*
 * The attention half of a decode step.  The pages name the model's attention
 * layers, 45 GatedDeltaNet (linear attention) and 15 full-attention layers, and say
 * the linear attention ran on the CPU with BLAS ([LLMAPIS] section 深度分析; [MFFB]
 * section 有效的优化), without formulas; the readings below are the library's.
 *
 * moe_gdn_step: one step of the gated delta rule per head h (as published by Yang,
 * Kautz and Hatamizadeh, 2024): S_h <- alpha_h S_h (I - beta_h k_h k_h^T) +
 * beta_h v_h k_h^T, then o_h = S_h q_h.
 *   state: fp32 [n_heads][dv][dk], updated in place; q, k: fp32 [n_heads][dk];
 *   v: fp32 [n_heads][dv]; alpha, beta: fp32 [n_heads]; o_out: fp32 [n_heads][dv].
 *   dk must be 64, 128 or 256 (MOE_EUNSUPPORTED otherwise); 4-byte alignment.
 */
int moe_gdn_step(int n_heads, int dk, int dv, float* state, const float* q, const float* k, const float* v,
                 const float* alpha, const float* beta, float* o_out, void* stream);

/*
 * moe_attn_decode: one decode step of grouped-query attention over T cached
 * positions: query head h reads KV head g = h / (n_q / n_kv),
 * o_h = sum_t softmax_t(q_h . K_g[t] / sqrt(d)) V_g[t].
 *   q: fp32 [n_q][d]; K, V: bf16 bit patterns [n_kv][T][d]; o_out: fp32 [n_q][d];
 *   ws: moe_attn_workspace_bytes bytes (per-block partial results over the cached
 *   positions); q, K, V and ws 16-byte aligned.  d must be 64, 128 or 256 and
 *   n_q / n_kv at most 16 (MOE_EUNSUPPORTED otherwise).  The products run on the
 *   matrix cores in bf16 with q and the softmax weights split into two bf16 terms
 *   each (relative residual about 2^-17), accumulating in fp32.
 */
size_t moe_attn_workspace_bytes(int n_q, int n_kv, int d, int T);
int moe_attn_decode(int n_q, int n_kv, int d, int T, const float* q, const uint16_t* K, const uint16_t* V,
                    float* o_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Dequantize one packed record back to dense fp32, reading it exactly as the
 * compute kernels do: W_out = [Wg (I x H) | Wu (I x H) | Wd (H x I)] row-major,
 * each element fmaf(s, q, b).  A check of the packed layout, not a hot path.
 */
int moe_dequant_expert(int bits, int H, int I, int group, const void* record, float* W_out,
                       void* stream);

/*
 * Range flags of records [0, n_experts) of a packed slab, for
 * moe_layer_desc.expert_flags: flags_out[e] = 1 if record e holds a group whose
 * scale or bias the batched matrix-core path cannot take (|s| >= 256,
 * |b| >= 2048 or not finite), else 0.  Reads only the records' scales and biases
 * (1/9 of a 4-bit record).  flags_out: device int32 [n_experts].
 */
int moe_expert_ranges(int bits, int H, int I, int group, const void* slab, int n_experts, int32_t* flags_out,
                      void* stream);

/*
 * Router ([LLMAPIS] section 深度分析; [CLAUDAY]): logits = W_r x (+ bias),
 * each fp32 product accumulated in fp64; keep the K largest (ties to the
 * lower id), in rank order; w = softmax weights (renormalized over the K if
 * renormalize != 0).
 *   x: fp32 [B][H]; idx_out: int32 [B][K]; w_out: fp32 [B][K].
 */
int moe_route_topk(const float* x, int B, const float* w_router, const float* logit_bias, int H,
                   int E, int K, int renormalize, int32_t* idx_out, float* w_out, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * Expert FFNs and combine for given routing ([LLMAPIS] section 深度分析: read the
 * selected experts, dequantize, compute, combine with the routing weights, the
 * dequant folding precomputed scale*x and bias*x into fused multiply-adds; 4-bit
 * or 2-bit experts, [LLMAPIS] section 为什么值得关注; one always-on shared expert,
 * [LLMAPIS] section 数据和技术细节):
 * y[b] = sum_k w[b][k] * FFN_{idx[b][k]}(x[b]) + shared_weight * FFN_shared(x[b]).
 *   x: fp32 [B][H]; idx: int32 [B][K]; w: fp32 [B][K]; y_out: fp32 [B][H].
 * _q4 requires desc->bits == 4, _q2 requires desc->bits == 2.
 * With B > 1 the tokens are grouped by expert (as moe_group_tokens) so each
 * active expert's weights are read once per call and multiplied against all of
 * its tokens on the matrix cores (value range as for moe_layer_decode); a batch
 * whose desc->expert_flags is set runs token by token instead unless its codes
 * are 4-bit with H, I <= 4096.
 */
int moe_expert_ffn_q4(const moe_layer_desc* desc, const float* x, int B, const int32_t* idx,
                      const float* w, float* y_out, void* ws, size_t ws_bytes, void* stream);
int moe_expert_ffn_q2(const moe_layer_desc* desc, const float* x, int B, const int32_t* idx,
                      const float* w, float* y_out, void* ws, size_t ws_bytes, void* stream);
/* 3-bit experts (desc->bits == 3; batches grouped on the matrix cores as at 2 bits). */
int moe_expert_ffn_q3(const moe_layer_desc* desc, const float* x, int B, const int32_t* idx,
                      const float* w, float* y_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Whole layer ([LLMAPIS] section 深度分析: routing + reading + dequantization +
 * local compute + result combine; [CLAUDAY]: K of 512 experts active, router at
 * full precision): route, then expert FFNs and combine, as above.
 *   x: fp32 [B][H]; y_out: fp32 [B][H]; idx_out: int32 [B][K] or NULL;
 *   w_out: fp32 [B][K] or NULL.
 * Value range: with B >= 2 the experts that several tokens share run on the
 * matrix cores, which take each group's scale s as fp16 and (b + 8 s) through
 * fp16 operands 2^5 b and 2^8 s: there |s| < 256 and |b| < 2048 per group
 * (larger values overflow to inf in y) unless desc->expert_flags
 * (moe_expert_ranges) marks such experts: with 4-bit codes and H, I <= 4096 these
 * then run on the GEMV path; any other batch with flags (2-bit codes, or H or I
 * above 4096) runs token by token.  The other paths apply scale and bias in fp32.
 */
int moe_layer_decode(const moe_layer_desc* desc, const float* x, int B, float* y_out,
                     int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_layer_decode without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory during a call (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments, results and kernels as moe_layer_decode; its scratch is a
 * library-owned array of MOE_NOALLOC_SCRATCH_BYTES in each GPU's memory, held
 * until the process ends.  A batch whose grouped-path workspace
 * (moe_workspace_bytes) would exceed it runs the token-by-token kernels instead
 * (same results within the same bounds); calls whose token-by-token workspace
 * exceeds it too return MOE_EUNSUPPORTED: at H = 4096, I = 1024, E = 512, K = 4
 * batches up to about 240 tokens fit.  Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (different streams or
 * threads without ordering) race and must not be issued.  The array's contents
 * need no initialization.  MOE_EHIP if the array's device address cannot be
 * obtained.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (8 << 20)
int moe_layer_decode_noalloc(const moe_layer_desc* desc, const float* x, int B, float* y_out,
                             int32_t* idx_out, float* w_out, void* stream);

/*
 * Tiered expert residency ([LLMAPIS] section 深度分析: only the K selected
 * experts of a layer are brought near the processor, and the OS page cache decides
 * what stays; [ACGFAV] section 到底做了什么).  Here the layer's packed records live
 * in a backing store, normally pinned host memory (allocated with hipHostMalloc,
 * e.g. torch's pin_memory=True), and `slots` of them plus the shared expert in an
 * HBM cache.  Each cached decode routes on the GPU, maps the selected experts onto
 * slots (a hit refreshes its slot; each miss evicts the least recently used slot
 * that the call does not use, ties to the lowest slot, misses taken in ascending
 * expert id), brings the missing records in from the store with GPU code that reads
 * the host memory directly (for one token, or per-token batches of at most 64
 * (token, expert) pairs, inside the gate/up launch, whose blocks of a missed expert
 * read its rows from the store; otherwise a copy launch first), and runs the expert
 * FFNs on the cache.  Nothing waits
 * on the host, so a call can be captured in a HIP graph.
 *   slab:  device, (slots + 1) records of moe_expert_record_bytes; the last holds
 *          the shared expert.
 *   state: device, moe_cache_state_bytes(E, slots) bytes, set up by moe_cache_init
 *          and updated by every cached decode (calls on one cache must be ordered
 *          on one stream).  Its first 32 bytes are uint64 counters: hits, misses,
 *          bytes copied from the store, calls.
 * With the cache the results are those of moe_layer_decode on the same records.
 */
#define MOE_MAX_CACHE_SLOTS 65536
typedef struct moe_expert_cache {
    int32_t slots;
    void* slab;
    void* state;
} moe_expert_cache;

/* Bytes of the cache state for E routed experts and `slots` slots (0 if invalid). */
size_t moe_cache_state_bytes(int E, int slots);

/* Empties every slot, zeroes the counters and copies the shared expert (record E of
 * desc->experts, the store) into its slot.  MOE_EINVAL for a bad desc or cache, or a
 * store that is neither device memory nor pinned host memory. */
int moe_cache_init(const moe_layer_desc* desc, const moe_expert_cache* cache, void* stream);

/* Workspace bytes of moe_layer_decode_cached for B tokens (0 if invalid). */
size_t moe_cache_workspace_bytes(const moe_layer_desc* desc, int slots, int B);

/*
 * moe_layer_decode with desc->experts a store of E + 1 packed records (pinned host
 * memory or device memory) and the experts computed from `cache`.  idx_out / w_out
 * (nullable) receive the routing in expert ids.  MOE_EINVAL if slots < min(E, B*K)
 * (a call's distinct experts must fit) or the workspace is too small.
 */
int moe_layer_decode_cached(const moe_layer_desc* desc, const moe_expert_cache* cache, const float* x, int B,
                            float* y_out, int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes,
                            void* stream);

/*
 * Token -> expert grouping of a batch's routing ([LLMAPIS] section 深度分析: only
 * the selected experts are read; with B tokens each selected expert is read
 * once for all the tokens that chose it).  A stable counting sort of the B*K
 * slots (slot i = b*K + k names expert idx[i]) by expert id:
 *   offsets_out: int32 [E + 1]; the slots of expert e are positions
 *     offsets_out[e] .. offsets_out[e+1]-1 of
 *   tokens_out: int32 [B*K] (token b of the slot) and
 *   slots_out:  int32 [B*K] (the slot index b*K + k), in increasing slot order.
 * Slots whose id is outside [0, E) are left out (offsets_out[E] is the number
 * placed).  All arrays are device memory owned by the caller; no workspace.
 */
int moe_group_tokens(const int32_t* idx, int B, int K, int E, int32_t* offsets_out,
                     int32_t* tokens_out, int32_t* slots_out, void* stream);

/*
 * x_out[b] = y[b] / sqrt(mean(y[b]^2) + eps), no gain, no residual: the
 * normalization between stacked MoE layers ([LLMAPIS] section 数据和技术细节 gives
 * the 60-layer stack; the pages do not print the normalization, this RMS form
 * without gain or residual is the reading the library fixes).
 * y, x_out: fp32 [B][H]; may alias.  MOE_EINVAL for B outside [1, 256], H <= 0,
 * eps < 0 or a NULL / misaligned pointer.
 */
int moe_rmsnorm(const float* y, int B, int H, float eps, float* x_out, void* stream);

/*
 * n_layers layers in sequence ([LLMAPIS] section 数据和技术细节: a stack of 60
 * MoE layers): x_0 = x; y_l = layer_l(x_l); x_{l+1} = rmsnorm(y_l, eps).
 * y_out receives y of the last layer.  idx_out / w_out: [n_layers][B][K] or
 * NULL.  Every layer must have the same H, I, E and K; code widths and group
 * sizes may differ from layer to layer (ws sized by moe_workspace_bytes of any
 * of them, plus moe_stack_extra_bytes).
 */
size_t moe_stack_extra_bytes(int B, int H);
int moe_stack_decode(const moe_layer_desc* layers, int n_layers, const float* x, int B, float eps,
                     float* y_out, int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * Timing hook.  While set, every launch of `kernel` issued from the calling
 * thread records start_event just before it and stop_event just after it on
 * the launch stream (hipEvent_t handles created by the caller, passed as
 * void*), so the caller can read the kernel's own duration with
 * hipEventElapsedTime.  NULL, NULL clears the hook.  Kernels:
 *   MOE_KERNEL_ROUTER  router logits (+ the token's dequant operand)
 *   MOE_KERNEL_GATEUP  top-K + fused gate/up dequant-GEMV + SwiGLU over the active
 *                      experts (the dominant kernel: 2/3 of the expert bytes)
 *   MOE_KERNEL_DOWN    down dequant-GEMV + router-weighted combine
 */
#define MOE_KERNEL_ROUTER 1
#define MOE_KERNEL_GATEUP 2
#define MOE_KERNEL_DOWN 3
int moe_set_timing_events(int kernel, void* start_event, void* stop_event);

/*
 * Launch shape of the batched path for B tokens of this layer on the calling
 * thread's current device, for inspection (no device work, no synchronization).
 * info_out: host int32 [8]:
 *   [0] 1 if B tokens take the grouped path (each active expert read once per
 *       call, [LLMAPIS] section 深度分析), else 0 (token by token)
 *   [1] blocks of the gate/up matrix-core launch (its work units are cut into
 *       that many equal ranges)
 *   [2] matrix-core tiles per work-list group in the gate/up phase
 *   [3] K chunks per gate/up tile when tiles outnumber the blocks of [1] (the
 *       partial sums of a tile shared by two blocks are added in K order)
 *   [4] blocks of the down matrix-core launch   [5] tiles per group, down
 *   [6] experts with fewer tokens than this run as GEMV groups (not on the matrix cores)
 *   [7] most tokens of one matrix-core work-list group
 */
int moe_grouped_launch_info(const moe_layer_desc* desc, int B, int32_t* info_out);

/* Text of the last error on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
