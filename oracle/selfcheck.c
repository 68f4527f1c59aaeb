/*
 * selfcheck.c - drives every function of the float64 oracle (oracle.c) and of
 * the seeded input generator (synth.c) on small inputs, so that both can be run
 * under AddressSanitizer and UndefinedBehaviorSanitizer on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY (built and run by the CPU test suite):
 *   gcc -g -O1 -fsanitize=address,undefined -fno-sanitize-recover=all -fopenmp \
 *       selfcheck.c oracle.c ../synth/synth.c -lm
 * Besides memory and UB errors, which the sanitizers report, it checks facts that
 * hold by construction: the unpack of hand-built bytes, that the dequantized
 * weight is s*q + b element by element, that the threaded and the token-parallel
 * decodes equal the serial one bit for bit, that K = E keeps every expert with
 * an infinite margin, that the grouping places every valid slot once, and that a
 * renormalized vector has the closed-form RMS.  Exit status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* oracle.c */
int oracle_code_at(const uint8_t* row, int bits, long c);
double oracle_bf16_to_double(uint16_t b);
void oracle_dequant_matrix(int bits, int rows, int cols, int group, const uint8_t* codes,
                           const uint16_t* scales, const uint16_t* biases, double* W);
void oracle_router_logits(int B, int H, int E, const float* x, const float* Wr, const float* prior,
                          double* logits);
int oracle_topk(int E, int K, const double* logits, int renormalize, int32_t* idx, double* w, double* margin);
int oracle_expert_ffn(int bits, int H, int I, int group, const uint8_t* gate_codes, const uint8_t* up_codes,
                      const uint8_t* down_codes, const uint16_t* scales, const uint16_t* biases, const double* x,
                      double* h_out, double* y);
int oracle_layer_decode(int bits, int H, int I, int E, int K, int group, int renormalize, double shared_weight,
                        const float* x, int B, const float* Wr, const float* prior, const uint8_t* const* gate,
                        const uint8_t* const* up, const uint8_t* const* down, const uint16_t* const* scales,
                        const uint16_t* const* biases, double* y, int32_t* idx, double* w, double* margin);
int oracle_layer_decode_par(int bits, int H, int I, int E, int K, int group, int renormalize, double shared_weight,
                            const float* x, int B, const float* Wr, const float* prior, const uint8_t* const* gate,
                            const uint8_t* const* up, const uint8_t* const* down, const uint16_t* const* scales,
                            const uint16_t* const* biases, double* y, int32_t* idx, double* w, double* margin);
int oracle_layer_decode_mt(int bits, int H, int I, int E, int K, int group, int renormalize, double shared_weight,
                           const float* x, const float* Wr, const float* prior, const uint8_t* const* gate,
                           const uint8_t* const* up, const uint8_t* const* down, const uint16_t* const* scales,
                           const uint16_t* const* biases, double* y, int32_t* idx, double* w);
int oracle_group_by_expert(int B, int K, int E, const int32_t* idx, int32_t* offsets, int32_t* tokens,
                           int32_t* slots);
void oracle_rms_renorm(int H, const double* y, double eps, double* x);
uint16_t oracle_bf16_round(double v);
void oracle_requant_expert(int H, int I, int group, const uint8_t* gate4, const uint8_t* up4, const uint8_t* down4,
                           const uint16_t* scales4, const uint16_t* biases4, uint8_t* gate2, uint8_t* up2,
                           uint8_t* down2, uint16_t* scales2, uint16_t* biases2);

void oracle_gdn_step(int n_heads, int dk, int dv, double* S, const double* q, const double* k, const double* v,
                     const double* alpha, const double* beta, double* o);
int oracle_attn_decode(int n_q, int n_kv, int d, int T, const double* q, const uint16_t* K, const uint16_t* V,
                       double* o);

/* synth.c */
size_t synth_codes_bytes(int bits, int rows, int cols);
void synth_experts(uint64_t seed, int64_t layer, int64_t first, int n, int bits, int H, int I, int group,
                   double scale_std, double bias_std, uint8_t* gate_codes, uint8_t* up_codes, uint8_t* down_codes,
                   uint16_t* scales, uint16_t* biases);
void synth_router(uint64_t seed, int64_t layer, int E, int H, float* w);
void synth_tokens(uint64_t seed, int64_t step, int B, int H, float* x);
void synth_zipf_bias(int E, double s, float* bias);

static int failures = 0;
#define EXPECT(cond, ...)                                   \
    do {                                                    \
        if (!(cond)) {                                      \
            fprintf(stderr, "FAIL line %d: ", __LINE__);    \
            fprintf(stderr, __VA_ARGS__);                   \
            fprintf(stderr, "\n");                          \
            ++failures;                                     \
        }                                                   \
    } while (0)

static void* xmalloc(size_t n)
{
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static int run_layer(int bits, int H, int I, int E, int K, int B, int with_prior)
{
    const int group = 64, n = E + 1;
    const size_t cb = synth_codes_bytes(bits, I, H), db = synth_codes_bytes(bits, H, I);
    const size_t ng = (size_t)2 * I * (H / group) + (size_t)H * (I / group);
    uint8_t* g = xmalloc(cb * n);
    uint8_t* u = xmalloc(cb * n);
    uint8_t* d = xmalloc(db * n);
    uint16_t* s = xmalloc(ng * n * 2);
    uint16_t* bb = xmalloc(ng * n * 2);
    synth_experts(77, 0, 0, n, bits, H, I, group, 0.02, 0.01, g, u, d, s, bb);
    const uint8_t** pg = xmalloc(sizeof(void*) * n);
    const uint8_t** pu = xmalloc(sizeof(void*) * n);
    const uint8_t** pd = xmalloc(sizeof(void*) * n);
    const uint16_t** ps = xmalloc(sizeof(void*) * n);
    const uint16_t** pb = xmalloc(sizeof(void*) * n);
    for (int e = 0; e < n; ++e) {
        pg[e] = g + cb * e;
        pu[e] = u + cb * e;
        pd[e] = d + db * e;
        ps[e] = s + ng * e;
        pb[e] = bb + ng * e;
    }
    float* Wr = xmalloc(sizeof(float) * (size_t)E * H);
    float* x = xmalloc(sizeof(float) * (size_t)B * H);
    float* prior = with_prior ? xmalloc(sizeof(float) * E) : NULL;
    synth_router(77, 0, E, H, Wr);
    synth_tokens(77, 3, B, H, x);
    if (prior) synth_zipf_bias(E, 1.1, prior);

    /* dequant: every element equals s * q + b of its group */
    double* W = xmalloc(sizeof(double) * (size_t)I * H);
    oracle_dequant_matrix(bits, I, H, group, pg[1], ps[1], pb[1], W);
    for (int r = 0; r < I; r += 7)
        for (int c = 0; c < H; c += 13) {
            const long gi = (long)r * (H / group) + c / group;
            const double want = oracle_bf16_to_double(ps[1][gi]) * oracle_code_at(pg[1] + (size_t)r * H * bits / 8, bits, c) +
                                oracle_bf16_to_double(pb[1][gi]);
            EXPECT(W[(long)r * H + c] == want, "dequant r=%d c=%d", r, c);
        }
    free(W);

    /* 4-bit -> 2-bit requantization of expert 1: every requantized weight lies within
     * the refit's range [b2, b2 + 3 s2] and every code is one of the four levels */
    if (bits == 4) {
        uint8_t* g2 = xmalloc(cb / 2);
        uint8_t* u2 = xmalloc(cb / 2);
        uint8_t* d2 = xmalloc(db / 2);
        uint16_t* s2 = xmalloc(ng * 2);
        uint16_t* b2 = xmalloc(ng * 2);
        oracle_requant_expert(H, I, group, pg[1], pu[1], pd[1], ps[1], pb[1], g2, u2, d2, s2, b2);
        double* W2 = xmalloc(sizeof(double) * (size_t)I * H);
        oracle_dequant_matrix(2, I, H, group, g2, s2, b2, W2);
        for (int r = 0; r < I; r += 5)
            for (int c = 0; c < H; c += 3) {
                const long gi = (long)r * (H / group) + c / group;
                const double lo = oracle_bf16_to_double(b2[gi]), st = oracle_bf16_to_double(s2[gi]);
                EXPECT(W2[(long)r * H + c] >= lo && W2[(long)r * H + c] <= lo + 3 * st, "requant r=%d c=%d", r, c);
            }
        free(W2); free(g2); free(u2); free(d2); free(s2); free(b2);
    }

    /* one expert's FFN, h returned */
    double* xd = xmalloc(sizeof(double) * H);
    double* h = xmalloc(sizeof(double) * I);
    double* ye = xmalloc(sizeof(double) * H);
    for (int c = 0; c < H; ++c) xd[c] = x[c];
    EXPECT(oracle_expert_ffn(bits, H, I, group, pg[0], pu[0], pd[0], ps[0], pb[0], xd, h, ye) == 0, "ffn");
    free(xd);
    free(h);
    free(ye);

    /* serial, token-parallel and expert-threaded decodes agree bit for bit */
    double* y1 = xmalloc(sizeof(double) * (size_t)B * H);
    double* y2 = xmalloc(sizeof(double) * (size_t)B * H);
    double* y3 = xmalloc(sizeof(double) * H);
    int32_t* i1 = xmalloc(sizeof(int32_t) * (size_t)B * K);
    int32_t* i2 = xmalloc(sizeof(int32_t) * (size_t)B * K);
    int32_t* i3 = xmalloc(sizeof(int32_t) * K);
    double* w1 = xmalloc(sizeof(double) * (size_t)B * K);
    double* w2 = xmalloc(sizeof(double) * (size_t)B * K);
    double* w3 = xmalloc(sizeof(double) * K);
    double* m1 = xmalloc(sizeof(double) * B);
    double* m2 = xmalloc(sizeof(double) * B);
    EXPECT(oracle_layer_decode(bits, H, I, E, K, group, 1, 1.0, x, B, Wr, prior, pg, pu, pd, ps, pb, y1, i1, w1, m1) == 0,
           "serial decode");
    EXPECT(oracle_layer_decode_par(bits, H, I, E, K, group, 1, 1.0, x, B, Wr, prior, pg, pu, pd, ps, pb, y2, i2, w2, m2) == 0,
           "parallel decode");
    EXPECT(memcmp(y1, y2, sizeof(double) * (size_t)B * H) == 0, "par y");
    EXPECT(memcmp(i1, i2, sizeof(int32_t) * (size_t)B * K) == 0, "par idx");
    EXPECT(memcmp(w1, w2, sizeof(double) * (size_t)B * K) == 0, "par w");
    EXPECT(memcmp(m1, m2, sizeof(double) * B) == 0, "par margin");
    for (int b = 0; b < B; ++b) {
        EXPECT(oracle_layer_decode_mt(bits, H, I, E, K, group, 1, 1.0, x + (size_t)b * H, Wr, prior, pg, pu, pd, ps, pb,
                                      y3, i3, w3) == 0,
               "mt decode");
        EXPECT(memcmp(y3, y1 + (size_t)b * H, sizeof(double) * H) == 0, "mt y token %d", b);
        EXPECT(memcmp(i3, i1 + (size_t)b * K, sizeof(int32_t) * K) == 0, "mt idx token %d", b);
        EXPECT(memcmp(w3, w1 + (size_t)b * K, sizeof(double) * K) == 0, "mt w token %d", b);
    }

    /* K = E keeps every expert; the margin past the last one is infinite */
    double* lg = xmalloc(sizeof(double) * E);
    int32_t* ia = xmalloc(sizeof(int32_t) * E);
    double* wa = xmalloc(sizeof(double) * E);
    double mg = 0.0;
    oracle_router_logits(1, H, E, x, Wr, prior, lg);
    EXPECT(oracle_topk(E, E, lg, 1, ia, wa, &mg) == 0 && isinf(mg), "K=E margin");
    int seen = 0;
    for (int e = 0; e < E; ++e) seen += (ia[e] >= 0 && ia[e] < E);
    EXPECT(seen == E, "K=E ids");
    EXPECT(oracle_topk(E, 0, lg, 1, ia, wa, &mg) == -1, "K=0 rejected");

    /* grouping: every valid slot placed once, invalid ids left out */
    int32_t* off = xmalloc(sizeof(int32_t) * (E + 1));
    int32_t* tok = xmalloc(sizeof(int32_t) * (size_t)B * K);
    int32_t* sl = xmalloc(sizeof(int32_t) * (size_t)B * K);
    i1[0] = -1;
    oracle_group_by_expert(B, K, E, i1, off, tok, sl);
    EXPECT(off[E] == B * K - 1, "grouping count %d", off[E]);
    for (int p = 0; p < off[E]; ++p) EXPECT(i1[sl[p]] >= 0 && sl[p] / K == tok[p], "grouping slot %d", p);

    /* RMS renorm of y: mean square 1 / (1 + eps / mean(y^2)) */
    double* xr = xmalloc(sizeof(double) * H);
    oracle_rms_renorm(H, y1, 1e-6, xr);
    double ms = 0.0, my = 0.0;
    for (int c = 0; c < H; ++c) {
        ms += xr[c] * xr[c];
        my += y1[c] * y1[c];
    }
    ms /= H;
    my /= H;
    EXPECT(fabs(ms - 1.0 / (1.0 + 1e-6 / my)) < 1e-12, "rms %.17g", ms);

    free(xr); free(off); free(tok); free(sl); free(lg); free(ia); free(wa);
    free(y1); free(y2); free(y3); free(i1); free(i2); free(i3); free(w1); free(w2); free(w3); free(m1); free(m2);
    free(Wr); free(x); free(prior);
    free(pg); free(pu); free(pd); free(ps); free(pb);
    free(g); free(u); free(d); free(s); free(bb);
    return 0;
}

int main(void)
{
    const uint8_t b21 = 0x21, be4 = 0xE4;
    EXPECT(oracle_code_at(&b21, 4, 0) == 1 && oracle_code_at(&b21, 4, 1) == 2, "nibbles of 0x21");
    for (int t = 0; t < 4; ++t) EXPECT(oracle_code_at(&be4, 2, t) == t, "crumb %d of 0xE4", t);
    {   /* 3-bit: one bit string, codes straddling bytes (codes 0..7 in three bytes) */
        const uint8_t r3[3] = {0x88, 0xC6, 0xFA};
        for (int c = 0; c < 8; ++c) EXPECT(oracle_code_at(r3, 3, c) == c, "3-bit code %d", c);
    }
    EXPECT(oracle_code_at(&b21, 5, 0) == -1, "bits=5 rejected");
    EXPECT(oracle_bf16_to_double(0x3F00) == 0.5 && oracle_bf16_to_double(0xBF80) == -1.0, "bf16 widening");
    EXPECT(oracle_bf16_round(1.0 + 1.0 / 256) == 0x3F80 && oracle_bf16_round(1.0 + 3.0 / 256) == 0x3F82,
           "bf16 rounding ties to even");
    EXPECT(oracle_bf16_round(3.4e38) == 0x7F80 && oracle_bf16_round(-0.0) == 0x8000, "bf16 rounding edges");
    {   /* the attention half: a gated-delta step with beta = 0 only decays the state; one cached
           position makes attention return that position's value */
        enum { NH = 3, DK = 8, DV = 6, T = 5, D = 8 };
        double S[NH * DV * DK], S0[NH * DV * DK], q[NH * DK], k[NH * DK], v[NH * DV], a[NH], b[NH], o[NH * DV];
        for (int i = 0; i < NH * DV * DK; ++i) S[i] = S0[i] = (double)((i * 37) % 11) - 5.0;
        for (int i = 0; i < NH * DK; ++i) q[i] = k[i] = (double)((i * 13) % 7) - 3.0;
        for (int i = 0; i < NH * DV; ++i) v[i] = (double)(i % 5);
        for (int h = 0; h < NH; ++h) { a[h] = 0.5; b[h] = 0.0; }
        oracle_gdn_step(NH, DK, DV, S, q, k, v, a, b, o);
        for (int i = 0; i < NH * DV * DK; ++i) EXPECT(S[i] == 0.5 * S0[i], "gdn decay %d", i);
        uint16_t K[2 * T * D], V[2 * T * D];
        double qa[4 * D], oa[4 * D];
        for (int i = 0; i < 2 * T * D; ++i) { K[i] = 0x3F80; V[i] = (uint16_t)(0x3F80 + (i % 3)); }
        for (int i = 0; i < 4 * D; ++i) qa[i] = 0.25 * (i % 4);
        EXPECT(oracle_attn_decode(4, 2, D, 1, qa, K, V, oa) == 0, "attention T=1");
        for (int h = 0; h < 4; ++h)
            for (int c = 0; c < D; ++c)
                EXPECT(oa[h * D + c] == oracle_bf16_to_double(V[(h / 2) * 1 * D + c]), "attention h=%d c=%d", h, c);
        EXPECT(oracle_attn_decode(4, 3, D, T, qa, K, V, oa) == -1, "attention n_q %% n_kv rejected");
    }
    run_layer(4, 128, 64, 16, 4, 3, 0);
    run_layer(2, 128, 64, 16, 4, 3, 1);
    run_layer(4, 192, 128, 37, 5, 4, 1);
    if (failures) {
        fprintf(stderr, "%d failure(s)\n", failures);
        return 1;
    }
    printf("selfcheck ok\n");
    return 0;
}
