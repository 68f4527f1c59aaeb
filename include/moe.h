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
 * 4-bit or 2-bit codes with a per-group scale and bias ([LLMAPIS] sections
 * 为什么值得关注 and 深度分析); the router stays at full precision
 * ([CLAUDAY]).  Readings this library fixes where the pages are silent:
 * w = s*q + b with unsigned q, bf16 s and b per 64 consecutive weights along
 * each row's input dimension; SwiGLU experts h = silu(Wg x) * (Wu x),
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
#define MOE_EUNSUPPORTED (-2)  /* bits not 2 or 4, group not 64, K > 32, E > 1024, B > 256, H > 65536, I > 8192 */
#define MOE_EHIP (-3)          /* the HIP runtime refused a launch */

#define MOE_MAX_K 32
#define MOE_MAX_E 1024
#define MOE_MAX_B 256

/*
 * One MoE layer.  All pointers are device memory owned by the caller.
 *   H: hidden size, I: expert intermediate size (both multiples of 64).
 *   E: routed experts, K: experts kept per token, bits: 4 or 2, group: 64.
 *   experts: packed slab of E + 1 records written by moe_pack_experts, the
 *            shared expert at index E; record stride moe_expert_record_bytes().
 *   w_router: fp32 [E][H] row-major.  logit_bias: fp32 [E] added to the
 *            logits before selection (e.g. a prior over expert ids), or NULL.
 *   shared_weight: factor of the shared expert in the combine (1.0 = plain sum).
 *   renormalize: 1 = routing weights renormalized over the kept K; 0 = raw
 *            softmax probabilities over all E.
 */
typedef struct moe_layer_desc {
    int32_t H, I, E, K, bits, group;
    const void* experts;
    const float* w_router;
    const float* logit_bias;
    float shared_weight;
    int32_t renormalize;
} moe_layer_desc;

/*
 * Bytes of one packed expert record: gate and up [I][H] plus down [H][I]
 * codes at `bits` per weight, plus a bf16 scale and bias per group of 64.
 * Equal to the canonical size of one expert, e.g. 7,077,888 B (6.75 MiB) at
 * H = 4096, I = 1024, 4-bit ([LLMAPIS] section 深度分析 gives about 6.75MB
 * per expert).  Returns 0 for unsupported arguments.
 */
size_t moe_expert_record_bytes(int bits, int H, int I, int group);

/* Workspace bytes needed by moe_layer_decode / moe_expert_ffn_* for B tokens
 * (and by moe_stack_decode, which needs the same).  0 on invalid desc/B. */
size_t moe_workspace_bytes(const moe_layer_desc* desc, int B);

/* Workspace bytes needed by moe_route_topk. 0 on invalid arguments. */
size_t moe_route_workspace_bytes(int B, int E, int K);

/*
 * Pack n_experts experts from the canonical format into records
 * [first_expert, first_expert + n_experts) of `slab_out`.
 * Canonical inputs (device, stacked over the n experts):
 *   gate_codes, up_codes: uint8 [n][I][H*bits/8]; down_codes: uint8 [n][H][I*bits/8]
 *     (4-bit: element 2j is the low nibble of byte j; 2-bit: element 4j+t sits
 *     at bits 2t..2t+1 of byte j);
 *   scales_bf16, biases_bf16: uint16 bf16 bit patterns [n][ng], per expert
 *     concatenated gate [I][H/64] | up [I][H/64] | down [H][I/64].
 * The record layout is private to the library ([LLMAPIS] section 深度分析:
 * each expert is fetched as one unit; here one contiguous record).
 * slab_out must hold at least (first_expert + n_experts) records.
 */
int moe_pack_experts(int bits, int H, int I, int group, int n_experts, const uint8_t* gate_codes,
                     const uint8_t* up_codes, const uint8_t* down_codes,
                     const uint16_t* scales_bf16, const uint16_t* biases_bf16, void* slab_out,
                     int first_expert, void* stream);

/*
 * Dequantize one packed record back to dense fp32, reading it exactly as the
 * compute kernels do: W_out = [Wg (I x H) | Wu (I x H) | Wd (H x I)] row-major,
 * each element fmaf(s, q, b).  A check of the packed layout, not a hot path.
 */
int moe_dequant_expert(int bits, int H, int I, int group, const void* record, float* W_out,
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
 * Expert FFNs and combine for given routing: y[b] = sum_k w[b][k] *
 * FFN_{idx[b][k]}(x[b]) + shared_weight * FFN_shared(x[b]).
 *   x: fp32 [B][H]; idx: int32 [B][K]; w: fp32 [B][K]; y_out: fp32 [B][H].
 * _q4 requires desc->bits == 4, _q2 requires desc->bits == 2.
 * With 4-bit codes and B > 1 the tokens are grouped by expert (as
 * moe_group_tokens) so each active expert's weights are read once per call and
 * multiplied against all of its tokens on the matrix cores (value range as
 * for moe_layer_decode); 2-bit batches run token by token.
 */
int moe_expert_ffn_q4(const moe_layer_desc* desc, const float* x, int B, const int32_t* idx,
                      const float* w, float* y_out, void* ws, size_t ws_bytes, void* stream);
int moe_expert_ffn_q2(const moe_layer_desc* desc, const float* x, int B, const int32_t* idx,
                      const float* w, float* y_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Whole layer: route, then expert FFNs and combine, as above.
 *   x: fp32 [B][H]; y_out: fp32 [B][H]; idx_out: int32 [B][K] or NULL;
 *   w_out: fp32 [B][K] or NULL.
 * Value range: with 4-bit codes and B >= 2 the experts that several tokens
 * share run on the matrix cores, which take each group's scale s as fp16 and
 * (b + 8 s) through fp16 operands 2^5 b and 2^8 s: there |s| < 256 and
 * |b| < 2048 per group (larger values overflow to inf in y).  The other paths
 * apply scale and bias in fp32.
 */
int moe_layer_decode(const moe_layer_desc* desc, const float* x, int B, float* y_out,
                     int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes, void* stream);

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
 * normalization between stacked layers.  y, x_out: fp32 [B][H]; may alias.
 */
int moe_rmsnorm(const float* y, int B, int H, float eps, float* x_out, void* stream);

/*
 * n_layers layers in sequence ([LLMAPIS] section 数据和技术细节: a stack of 60
 * MoE layers): x_0 = x; y_l = layer_l(x_l); x_{l+1} = rmsnorm(y_l, eps).
 * y_out receives y of the last layer.  idx_out / w_out: [n_layers][B][K] or
 * NULL.  Every layer must have the same H, I, K, bits (ws sized by
 * moe_workspace_bytes of any of them, plus moe_stack_extra_bytes).
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

/* Text of the last error on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
