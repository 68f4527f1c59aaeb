/*
 * oracle.c - plain, slow, float64 CPU oracle of one quantized MoE layer's
 * per-token decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the GPU library; the two agree only on the canonical input
 * format, which each side implements on its own.
 *
 * Pages cited (titles as published):
 *   [LLMAPIS] llmapis.com, "Flash-MoE：把 397B MoE 真正跑进消费级笔记本，意味着
 *             '大模型本地化'开始从演示走向系统工程"
 *   [MFFB]    f.mffb.com.cn, "HN上281票 ... 8200行纯C代码 ..." (Flash-MoE article)
 *   [ACGFAV]  acgfav.com, "iPhone 17 Pro也能跑近400B大模型？Flash-MoE把端侧AI推到新极限"
 *   [CLAUDAY] clauday.com, "Flash-MoE: Running a 397B Parameter Model on a MacBook
 *             with Pure C and Metal"
 *
 * What the layer computes, in the order the pages give it ([LLMAPIS]
 * section 深度分析: routing, reading, dequantization, local compute, result
 * combine):
 *   1. router logits l[e] = sum_h Wr[e][h] x[h] (+ optional prior[e]); the router
 *      stays at full precision ([CLAUDAY]: routing matrices kept at original
 *      precision).
 *   2. keep the K largest logits, K = 4 of 512 experts plus one always-on
 *      shared expert ([LLMAPIS] section 深度分析 and 数据和技术细节; [CLAUDAY]:
 *      active experts cut from 10 to 4).  Softmax over all E, renormalized over
 *      the kept K (the full-E denominator cancels).
 *   3. dequantize the active experts: each weight is an unsigned 4- or 2-bit
 *      code q with a per-group scale s and bias b, w = s*q + b ([LLMAPIS]
 *      section 深度分析: the dequant kernel folds precomputed scale*x and
 *      bias*x into FMAs, which presumes an additive bias per group; section
 *      为什么值得关注: 4-bit / 2-bit expert quantization).
 *   4. each expert is a SwiGLU FFN: h = silu(Wg x) * (Wu x), y_e = Wd h.
 *   5. y = sum_k w_k y_{idx_k} + shared_weight * y_shared.
 * Readings where the pages are silent (group 64 along the input dimension,
 * bf16 scale/bias, SwiGLU, shared weight 1, tie-break to the lower id,
 * RMS renorm with eps between stacked layers) are the workload's contract and
 * are listed with the rest of the design notes.
 *
 * Every floating-point step is done in double.  fp32 inputs and bf16 scale /
 * bias widen to double exactly.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 * (OpenMP is used only by oracle_layer_decode_mt, the timed baseline, and by
 * oracle_layer_decode_par, which runs the serial per-token decode on many
 * tokens at once.)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- canonical format ---------------------------------------------------- */

/* Element c of a canonically packed row: 4-bit: element 2j is the low nibble
 * of byte j and 2j+1 the high nibble; 2-bit: element 4j+t sits at bits
 * 2t..2t+1 of byte j; 3-bit: the row is one little-endian bit string and
 * element c holds its bits 3c..3c+2, lowest bit first (a code may straddle two
 * bytes). */
int oracle_code_at(const uint8_t* row, int bits, long c)
{
    if (bits == 4) {
        uint8_t byte = row[c / 2];
        return (c % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
    }
    if (bits == 2) {
        uint8_t byte = row[c / 4];
        return (byte >> (2 * (c % 4))) & 0x03;
    }
    if (bits == 3) {
        int q = 0;
        for (int t = 0; t < 3; ++t) {  /* bit 3c + t of the string */
            long bit = 3 * c + t;
            q |= ((row[bit / 8] >> (bit % 8)) & 1) << t;
        }
        return q;
    }
    return -1;
}

/* bf16 bit pattern -> double (exact: bf16 is the top half of an fp32). */
double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Dequantize one [rows][cols] matrix: W[r][c] = s[r][c/group] * q[r][c] + b[r][c/group]. */
void oracle_dequant_matrix(int bits, int rows, int cols, int group, const uint8_t* codes,
                           const uint16_t* scales, const uint16_t* biases, double* W)
{
    long row_bytes = (long)cols * bits / 8;
    int gpr = cols / group;
    for (int r = 0; r < rows; ++r) {
        const uint8_t* row = codes + (long)r * row_bytes;
        for (int c = 0; c < cols; ++c) {
            double s = oracle_bf16_to_double(scales[(long)r * gpr + c / group]);
            double b = oracle_bf16_to_double(biases[(long)r * gpr + c / group]);
            int q = oracle_code_at(row, bits, c);
            W[(long)r * cols + c] = s * (double)q + b;
        }
    }
}

/* ---- router --------------------------------------------------------------- */

/* logits[b][e] = sum_h Wr[e][h] * x[b][h] (+ prior[e]), summed in double in h order. */
void oracle_router_logits(int B, int H, int E, const float* x, const float* Wr, const float* prior,
                          double* logits)
{
    for (int b = 0; b < B; ++b)
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h) acc += (double)Wr[(long)e * H + h] * (double)x[(long)b * H + h];
            if (prior) acc += (double)prior[e];
            logits[(long)b * E + e] = acc;
        }
}

/* "a ranks before b": larger logit first, equal logits -> lower id first. */
static int ranks_before(double la, int a, double lb, int b)
{
    if (la != lb) return la > lb;
    return a < b;
}

/*
 * Top-K of one token's logits plus its routing weights.
 * idx: the K best ids in rank order.  w: softmax over all E, then (if
 * renormalize) divided by the sum over the kept K.  margin: l_(K) - l_(K+1)
 * (+inf when K == E).  Selection is a plain repeated scan for the best
 * remaining expert.  Returns 0, or -1 on bad arguments.
 */
int oracle_topk(int E, int K, const double* logits, int renormalize, int32_t* idx, double* w,
                double* margin)
{
    if (K < 1 || K > E) return -1;
    char* taken = (char*)calloc((size_t)E, 1);
    if (!taken) return -1;
    for (int k = 0; k < K; ++k) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || ranks_before(logits[e], e, logits[best], best)) best = e;
        }
        taken[best] = 1;
        idx[k] = best;
    }
    if (margin) {
        int next = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (next < 0 || ranks_before(logits[e], e, logits[next], next)) next = e;
        }
        *margin = next < 0 ? INFINITY : logits[idx[K - 1]] - logits[next];
    }
    free(taken);

    double lmax = logits[0];
    for (int e = 1; e < E; ++e) if (logits[e] > lmax) lmax = logits[e];
    double z = 0.0;
    for (int e = 0; e < E; ++e) z += exp(logits[e] - lmax);
    double kept = 0.0;
    for (int k = 0; k < K; ++k) {
        w[k] = exp(logits[idx[k]] - lmax) / z;
        kept += w[k];
    }
    if (renormalize)
        for (int k = 0; k < K; ++k) w[k] /= kept;
    return 0;
}

/* ---- expert FFN ------------------------------------------------------------ */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * One SwiGLU expert on one token, dense in double:
 *   g = Wg x, u = Wu x, h = silu(g) * u, y = Wd h.
 * scales/biases: gate [I][H/group] | up [I][H/group] | down [H][I/group].
 * h may be NULL.  Returns 0, or -1 if out of memory.
 */
int oracle_expert_ffn(int bits, int H, int I, int group, const uint8_t* gate_codes,
                      const uint8_t* up_codes, const uint8_t* down_codes, const uint16_t* scales,
                      const uint16_t* biases, const double* x, double* h_out, double* y)
{
    long ngu = (long)I * (H / group);
    double* Wg = (double*)malloc(sizeof(double) * (size_t)I * H);
    double* Wu = (double*)malloc(sizeof(double) * (size_t)I * H);
    double* Wd = (double*)malloc(sizeof(double) * (size_t)H * I);
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    if (!Wg || !Wu || !Wd || !h) {
        free(Wg); free(Wu); free(Wd); free(h);
        return -1;
    }
    oracle_dequant_matrix(bits, I, H, group, gate_codes, scales, biases, Wg);
    oracle_dequant_matrix(bits, I, H, group, up_codes, scales + ngu, biases + ngu, Wu);
    oracle_dequant_matrix(bits, H, I, group, down_codes, scales + 2 * ngu, biases + 2 * ngu, Wd);
    for (int r = 0; r < I; ++r) {
        double g = 0.0, u = 0.0;
        for (int c = 0; c < H; ++c) {
            g += Wg[(long)r * H + c] * x[c];
            u += Wu[(long)r * H + c] * x[c];
        }
        h[r] = silu(g) * u;
    }
    for (int r = 0; r < H; ++r) {
        double acc = 0.0;
        for (int j = 0; j < I; ++j) acc += Wd[(long)r * I + j] * h[j];
        y[r] = acc;
    }
    if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)I);
    free(Wg); free(Wu); free(Wd); free(h);
    return 0;
}

/* ---- one layer ------------------------------------------------------------- */

/*
 * Expert tables: entry e (0 <= e < E) is routed expert e, entry E is the
 * shared expert; each entry points at that expert's canonical tensors.  An
 * entry may be NULL if the expert is never selected (the call then fails with
 * -2 if it is needed).
 */
typedef struct {
    const uint8_t* const* gate;
    const uint8_t* const* up;
    const uint8_t* const* down;
    const uint16_t* const* scales;
    const uint16_t* const* biases;
} oracle_expert_table;

static int ffn_of(const oracle_expert_table* t, int e, int bits, int H, int I, int group,
                  const double* x, double* y)
{
    if (!t->gate[e] || !t->up[e] || !t->down[e] || !t->scales[e] || !t->biases[e]) return -2;
    return oracle_expert_ffn(bits, H, I, group, t->gate[e], t->up[e], t->down[e], t->scales[e],
                             t->biases[e], x, NULL, y);
}

/*
 * Decode B tokens through one layer; each token is independent.
 * Outputs: y [B][H] double, idx [B][K], w [B][K] double, margin [B].
 */
int oracle_layer_decode(int bits, int H, int I, int E, int K, int group, int renormalize,
                        double shared_weight, const float* x, int B, const float* Wr,
                        const float* prior, const uint8_t* const* gate, const uint8_t* const* up,
                        const uint8_t* const* down, const uint16_t* const* scales,
                        const uint16_t* const* biases, double* y, int32_t* idx, double* w,
                        double* margin)
{
    oracle_expert_table t = {gate, up, down, scales, biases};
    double* logits = (double*)malloc(sizeof(double) * (size_t)E);
    double* xd = (double*)malloc(sizeof(double) * (size_t)H);
    double* ye = (double*)malloc(sizeof(double) * (size_t)H);
    int rc = 0;
    if (!logits || !xd || !ye) rc = -1;
    for (int b = 0; b < B && rc == 0; ++b) {
        const float* xb = x + (long)b * H;
        oracle_router_logits(1, H, E, xb, Wr, prior, logits);
        rc = oracle_topk(E, K, logits, renormalize, idx + (long)b * K, w + (long)b * K,
                         margin ? margin + b : NULL);
        if (rc) break;
        for (int c = 0; c < H; ++c) xd[c] = (double)xb[c];
        double* yb = y + (long)b * H;
        for (int c = 0; c < H; ++c) yb[c] = 0.0;
        for (int k = 0; k < K && rc == 0; ++k) {
            rc = ffn_of(&t, idx[(long)b * K + k], bits, H, I, group, xd, ye);
            for (int c = 0; c < H && rc == 0; ++c) yb[c] += w[(long)b * K + k] * ye[c];
        }
        if (rc == 0) rc = ffn_of(&t, E, bits, H, I, group, xd, ye);
        for (int c = 0; c < H && rc == 0; ++c) yb[c] += shared_weight * ye[c];
    }
    free(logits); free(xd); free(ye);
    return rc;
}

/*
 * Same computation as oracle_layer_decode for one token, with the active
 * experts' FFNs spread over OpenMP threads.  Only the CPU baseline timing uses
 * it; each expert's FFN is the same serial oracle_expert_ffn.
 */
int oracle_layer_decode_mt(int bits, int H, int I, int E, int K, int group, int renormalize,
                           double shared_weight, const float* x, const float* Wr, const float* prior,
                           const uint8_t* const* gate, const uint8_t* const* up,
                           const uint8_t* const* down, const uint16_t* const* scales,
                           const uint16_t* const* biases, double* y, int32_t* idx, double* w)
{
    oracle_expert_table t = {gate, up, down, scales, biases};
    double* logits = (double*)malloc(sizeof(double) * (size_t)E);
    double* xd = (double*)malloc(sizeof(double) * (size_t)H);
    double* ys = (double*)malloc(sizeof(double) * (size_t)H * (K + 1));
    int rc = (!logits || !xd || !ys) ? -1 : 0;
    if (rc == 0) {
        #pragma omp parallel for schedule(static)
        for (int e = 0; e < E; ++e) oracle_router_logits(1, H, 1, x, Wr + (long)e * H, NULL, logits + e);
        if (prior)
            for (int e = 0; e < E; ++e) logits[e] += (double)prior[e];
        rc = oracle_topk(E, K, logits, renormalize, idx, w, NULL);
    }
    if (rc == 0) {
        for (int c = 0; c < H; ++c) xd[c] = (double)x[c];
        int err = 0;
        #pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
        for (int k = 0; k <= K; ++k) {
            int e = (k < K) ? idx[k] : E;
            err |= ffn_of(&t, e, bits, H, I, group, xd, ys + (long)k * H) ? 1 : 0;
        }
        if (err) rc = -2;
    }
    if (rc == 0)
        for (int c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) acc += w[k] * ys[(long)k * H + c];
            y[c] = acc + shared_weight * ys[(long)K * H + c];
        }
    free(logits); free(xd); free(ys);
    return rc;
}

/*
 * oracle_layer_decode over B tokens with the tokens spread over OpenMP
 * threads: each token is decoded by oracle_layer_decode on its own, so every
 * token's result is the serial one bit for bit.  Used where many tokens of a
 * full-size batch are checked.  Same outputs and return codes as
 * oracle_layer_decode (the first failing token's code).
 */
int oracle_layer_decode_par(int bits, int H, int I, int E, int K, int group, int renormalize,
                            double shared_weight, const float* x, int B, const float* Wr,
                            const float* prior, const uint8_t* const* gate, const uint8_t* const* up,
                            const uint8_t* const* down, const uint16_t* const* scales,
                            const uint16_t* const* biases, double* y, int32_t* idx, double* w,
                            double* margin)
{
    int rc = 0;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        int r = oracle_layer_decode(bits, H, I, E, K, group, renormalize, shared_weight,
                                    x + (long)b * H, 1, Wr, prior, gate, up, down, scales, biases,
                                    y + (long)b * H, idx + (long)b * K, w + (long)b * K,
                                    margin ? margin + b : NULL);
        if (r) {
            #pragma omp critical
            if (rc == 0) rc = r;
        }
    }
    return rc;
}

/* ---- batched decode: token -> expert grouping ------------------------------- */

/*
 * Group the B*K (token, slot) assignments by expert id, stable in token order:
 * offsets[e]..offsets[e+1] index the tokens routed to expert e; tokens[] holds
 * the token id and slots[] the position b*K + k of that assignment.
 * Returns the number U of distinct routed experts.  offsets has E+1 entries.
 */
int oracle_group_by_expert(int B, int K, int E, const int32_t* idx, int32_t* offsets,
                           int32_t* tokens, int32_t* slots)
{
    int U = 0;
    int pos = 0;
    for (int e = 0; e < E; ++e) {
        offsets[e] = pos;
        for (int b = 0; b < B; ++b)
            for (int k = 0; k < K; ++k)
                if (idx[(long)b * K + k] == e) {
                    tokens[pos] = b;
                    slots[pos] = b * K + k;
                    ++pos;
                }
        if (pos > offsets[e]) ++U;
    }
    offsets[E] = pos;
    return U;
}

/* ---- stacked layers ------------------------------------------------------------ */

/* x = y / sqrt(mean(y^2) + eps), no gain, no residual. */
void oracle_rms_renorm(int H, const double* y, double eps, double* x)
{
    double ss = 0.0;
    for (int c = 0; c < H; ++c) ss += y[c] * y[c];
    double inv = 1.0 / sqrt(ss / H + eps);
    for (int c = 0; c < H; ++c) x[c] = y[c] * inv;
}

/* ---- offline 4-bit -> 2-bit requantization ------------------------------------- */

/*
 * The pages report that the experts were requantized from 4-bit to 2-bit,
 * shrinking the expert files from 209 GB to 120 GB ([CLAUDAY]; [LLMAPIS]
 * section 数据和技术细节), without giving the procedure.  The reading used here is
 * a per-group min/max affine refit of the dequantized 4-bit weights:
 *   w_c = s4 * q4_c + b4 for the 64 weights c of a group (exact in double),
 *   b2  = bf16(min_c w_c), s2 = bf16((max_c w_c - min_c w_c) / 3),
 *   q2_c = clamp(rint((w_c - b2) / s2), 0, 3)   (q2_c = 0 when s2 == 0, and when the
 *   quotient is not a number, as with a scale or bias beyond the bf16 range),
 * every step in IEEE double (rint: to nearest, ties to even) and bf16() a single
 * rounding of the double to the nearest bf16 value, ties to even.
 */

/* Nearest bf16 value of a finite double, ties to even, as a bit pattern: one
 * rounding of the 53-bit mantissa to bf16's 8 bits, with fp32's exponent range
 * (subnormals in steps of 2^-133); magnitudes that round past the largest bf16
 * become infinity. */
uint16_t oracle_bf16_round(double v)
{
    if (v != v) return 0x7FC0;
    uint16_t sign = (v < 0 || (v == 0 && 1.0 / v < 0)) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                      /* a = m * 2^e, 0.5 <= m < 1 */
    int q = e - 8;                     /* a normal bf16 keeps 8 significant bits: quantum 2^(e-8) */
    if (q < -133) q = -133;            /* below 2^-126: the subnormal quantum */
    double r = nearbyint(ldexp(a, -q));   /* multiple of the quantum, ties to even */
    double rv = ldexp(r, q);
    if (rv > 3.3895313892515355e38) return (uint16_t)(sign | 0x7F80);   /* past the largest bf16 */
    float f = (float)rv;               /* exact: rv is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

/* One group of n weights given as 4-bit codes q4[c] with bf16 s4, b4 -> 2-bit codes q2[c]
 * and bf16 s2, b2 (bit patterns), as defined above. */
void oracle_requant_group(int n, const int* q4, uint16_t s4, uint16_t b4, int* q2, uint16_t* s2_out,
                          uint16_t* b2_out)
{
    double s = oracle_bf16_to_double(s4), b = oracle_bf16_to_double(b4);
    double lo = s * q4[0] + b, hi = lo;
    for (int c = 1; c < n; ++c) {
        double w = s * q4[c] + b;
        if (w < lo) lo = w;
        if (w > hi) hi = w;
    }
    uint16_t b2 = oracle_bf16_round(lo);
    uint16_t s2 = oracle_bf16_round((hi - lo) / 3.0);
    double bd = oracle_bf16_to_double(b2), sd = oracle_bf16_to_double(s2);
    for (int c = 0; c < n; ++c) {
        if (sd == 0.0) {
            q2[c] = 0;
            continue;
        }
        double t = nearbyint((s * q4[c] + b - bd) / sd);
        q2[c] = t >= 3.0 ? 3 : (t > 0.0 ? (int)t : 0);   /* a quotient that is not a number gives 0 */
    }
    *s2_out = s2;
    *b2_out = b2;
}

/* A [rows][cols] matrix of canonical 4-bit codes with per-group bf16 scales and
 * biases -> canonical 2-bit codes [rows][cols/4 bytes] and new scales / biases. */
static void requant_matrix(int rows, int cols, int group, const uint8_t* codes4, const uint16_t* s4,
                           const uint16_t* b4, uint8_t* codes2, uint16_t* s2, uint16_t* b2)
{
    int gpr = cols / group;
    int* q4 = (int*)malloc(sizeof(int) * (size_t)group);
    int* q2 = (int*)malloc(sizeof(int) * (size_t)group);
    if (!q4 || !q2) {
        free(q4);
        free(q2);
        return;
    }
    memset(codes2, 0, (size_t)rows * cols / 4);
    for (int r = 0; r < rows; ++r)
        for (int g = 0; g < gpr; ++g) {
            const uint8_t* row = codes4 + (long)r * cols / 2;
            for (int c = 0; c < group; ++c) q4[c] = oracle_code_at(row, 4, (long)g * group + c);
            long gi = (long)r * gpr + g;
            oracle_requant_group(group, q4, s4[gi], b4[gi], q2, s2 + gi, b2 + gi);
            for (int c = 0; c < group; ++c) {
                long col = (long)g * group + c;
                codes2[(long)r * cols / 4 + col / 4] |= (uint8_t)(q2[c] << (2 * (col % 4)));
            }
        }
    free(q4);
    free(q2);
}

/* One canonical 4-bit expert -> the canonical 2-bit expert (same H, I, group). */
void oracle_requant_expert(int H, int I, int group, const uint8_t* gate4, const uint8_t* up4,
                           const uint8_t* down4, const uint16_t* scales4, const uint16_t* biases4,
                           uint8_t* gate2, uint8_t* up2, uint8_t* down2, uint16_t* scales2,
                           uint16_t* biases2)
{
    long ngu = (long)I * (H / group);
    requant_matrix(I, H, group, gate4, scales4, biases4, gate2, scales2, biases2);
    requant_matrix(I, H, group, up4, scales4 + ngu, biases4 + ngu, up2, scales2 + ngu, biases2 + ngu);
    requant_matrix(H, I, group, down4, scales4 + 2 * ngu, biases4 + 2 * ngu, down2, scales2 + 2 * ngu,
                   biases2 + 2 * ngu);
}

/* ---- the attention half of a decode step ----------------------------------------- */

/*
 * The pages name the two kinds of attention layer of the model, 45 GatedDeltaNet
 * (linear attention) layers and 15 full-attention layers, and say the linear
 * attention ran on the CPU with BLAS ([LLMAPIS] section 深度分析; [MFFB] section
 * 有效的优化), without formulas.  The readings used here:
 *
 * GatedDeltaNet, one decode step of the gated delta rule per head h (state S_h,
 * dv x dk, row-major; the rule as published by Yang, Kautz and Hatamizadeh, 2024):
 *   S_h <- alpha_h * S_h (I - beta_h k_h k_h^T) + beta_h v_h k_h^T,   o_h = S_h q_h
 * with q_h, k_h in R^dk, v_h in R^dv, a decay alpha_h and a write strength beta_h,
 * all given (the projections that make them are plain GEMVs and not part of this
 * step).
 *
 * Full attention, one decode step of grouped-query attention: query head h reads
 * key/value head g = h / (n_q / n_kv) over T cached positions,
 *   o_h = sum_t softmax_t(q_h . K_g[t] / sqrt(d)) V_g[t],
 * with K and V as bf16 bit patterns [n_kv][T][d].
 */

/* One step of the gated delta rule for n_heads heads; S [n][dv][dk] is updated in place. */
void oracle_gdn_step(int n_heads, int dk, int dv, double* S, const double* q, const double* k,
                     const double* v, const double* alpha, const double* beta, double* o)
{
    double* Sk = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!Sk) return;
    for (int h = 0; h < n_heads; ++h) {
        double* Sh = S + (long)h * dv * dk;
        const double* kh = k + (long)h * dk;
        const double* qh = q + (long)h * dk;
        const double* vh = v + (long)h * dv;
        /* S (I - beta k k^T) = S - beta (S k) k^T */
        for (int r = 0; r < dv; ++r) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += Sh[(long)r * dk + c] * kh[c];
            Sk[r] = acc;
        }
        for (int r = 0; r < dv; ++r)
            for (int c = 0; c < dk; ++c) {
                double m = Sh[(long)r * dk + c] - beta[h] * Sk[r] * kh[c];
                Sh[(long)r * dk + c] = alpha[h] * m + beta[h] * vh[r] * kh[c];
            }
        for (int r = 0; r < dv; ++r) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += Sh[(long)r * dk + c] * qh[c];
            o[(long)h * dv + r] = acc;
        }
    }
    free(Sk);
}

/* One decode step of grouped-query attention over T cached positions (n_q % n_kv == 0). */
int oracle_attn_decode(int n_q, int n_kv, int d, int T, const double* q, const uint16_t* K,
                       const uint16_t* V, double* o)
{
    if (n_kv < 1 || n_q % n_kv != 0 || T < 1) return -1;
    double* sc = (double*)malloc(sizeof(double) * (size_t)T);
    if (!sc) return -1;
    int per = n_q / n_kv;
    double scale = 1.0 / sqrt((double)d);
    for (int h = 0; h < n_q; ++h) {
        int g = h / per;
        const uint16_t* Kg = K + (long)g * T * d;
        const uint16_t* Vg = V + (long)g * T * d;
        double mx = -INFINITY;
        for (int t = 0; t < T; ++t) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c) acc += q[(long)h * d + c] * oracle_bf16_to_double(Kg[(long)t * d + c]);
            sc[t] = acc * scale;
            if (sc[t] > mx) mx = sc[t];
        }
        double z = 0.0;
        for (int t = 0; t < T; ++t) {
            sc[t] = exp(sc[t] - mx);
            z += sc[t];
        }
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int t = 0; t < T; ++t) acc += sc[t] * oracle_bf16_to_double(Vg[(long)t * d + c]);
            o[(long)h * d + c] = acc / z;
        }
    }
    free(sc);
    return 0;
}
