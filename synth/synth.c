/*
 * synth.c - seeded, counter-based generator of the synthetic workload.
 *
 * This module produces inputs only: expert weights in the canonical
 * quantized format, router weights, token activations and the Zipf logit
 * prior.  It holds none of the method's arithmetic (no dequantization, no
 * routing, no FFN) and is shared by the GPU path's tests/bench and by the
 * oracle, which must both see the same bytes.
 *
 * Every value is a pure function of (seed, layer, expert, tensor, index), so
 * any single expert of any layer can be regenerated on demand without
 * generating the rest of the layer.
 *
 * Hash: the SplitMix64 output function (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014).  Element i of a
 * stream with key k is mix64(k + (i + 1) * GOLDEN_GAMMA).
 * Normals: the Box-Muller transform in double, using two hashed uniforms in
 * (0, 1] per element (only the cosine branch is used, so each element is an
 * independent function of its own index).
 *
 * Distributions (the synthetic workload of the Flash-MoE layer):
 *   codes  : uniform bytes, hence every 4-bit nibble uniform in [0,15] and
 *            every 2-bit field uniform in [0,3]
 *   scale  : |N(0, 0.02)| rounded once from double to bf16 (round to nearest even)
 *   bias   : N(0, 0.01)   rounded once from double to bf16
 *   router : N(0, 1/sqrt(H)) rounded to fp32
 *   tokens : N(0, 1) rounded to fp32
 *   zipf   : prior[e] = -s * ln(e + 1) rounded to fp32
 * (the second argument of N is a standard deviation).
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC synth.c -o libsynth.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

/* tensor ids inside one (seed, layer, expert) */
enum {
    SYN_T_GATE_CODES = 1,
    SYN_T_UP_CODES = 2,
    SYN_T_DOWN_CODES = 3,
    SYN_T_SCALES = 4,
    SYN_T_BIASES = 5,
    SYN_T_ROUTER = 6,
    SYN_T_TOKENS = 7
};

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_stream_key(uint64_t seed, int64_t layer, int64_t expert, int64_t tensor)
{
    uint64_t k = mix64(seed + GOLDEN_GAMMA);
    k = mix64(k ^ ((uint64_t)layer * 0xD1B54A32D192ED03ULL + 0x632BE59BD9B4E019ULL));
    k = mix64(k ^ ((uint64_t)expert * 0xAEF17502108EF2D9ULL + 0x8CB92BA72F3D8DD7ULL));
    k = mix64(k ^ ((uint64_t)tensor * 0xDB4F0B9175AE2165ULL + 0x4F1BBCDCBFA53E0BULL));
    return k;
}

static inline uint64_t stream_at(uint64_t key, uint64_t i)
{
    return mix64(key + (i + 1) * GOLDEN_GAMMA);
}

/* uniform in (0, 1]: 53 random bits */
static inline double unit_open0(uint64_t h)
{
    return (double)((h >> 11) + 1) * 0x1.0p-53;
}

static inline double normal_at(uint64_t key, uint64_t i)
{
    const double two_pi = 6.283185307179586476925286766559;
    double u1 = unit_open0(stream_at(key, 2 * i));
    double u2 = unit_open0(stream_at(key, 2 * i + 1));
    return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

/* Round a double to the nearest bf16 (ties to even), in one step. */
uint16_t synth_bf16_from_double(double d)
{
    if (isnan(d)) return 0x7FC0;
    uint16_t sign = signbit(d) ? 0x8000 : 0;
    double a = fabs(d);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int e;
    (void)frexp(a, &e);            /* a in [2^(e-1), 2^e) */
    int q = e - 8;                 /* spacing of bf16 values in that binade */
    if (q < -133) q = -133;        /* subnormal spacing of bf16 */
    double r = nearbyint(ldexp(a, -q)); /* default rounding mode: nearest-even */
    double v = ldexp(r, q);
    if (v > 0x1.FEp127) return sign | 0x7F80;
    float f = (float)v;            /* exact: v has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (u >> 16));
}

void synth_bytes(uint64_t key, size_t n, uint8_t* out)
{
    size_t nw = n / 8;
    #pragma omp parallel for schedule(static) if (nw > (1u << 16))
    for (size_t w = 0; w < nw; ++w) {
        uint64_t h = stream_at(key, w);
        memcpy(out + 8 * w, &h, 8);
    }
    if (n % 8) {
        uint64_t h = stream_at(key, nw);
        memcpy(out + 8 * nw, &h, n % 8);
    }
}

void synth_normal_f64(uint64_t key, size_t n, double mean, double std, double* out)
{
    #pragma omp parallel for schedule(static) if (n > (1u << 14))
    for (size_t i = 0; i < n; ++i) out[i] = mean + std * normal_at(key, i);
}

void synth_normal_f32(uint64_t key, size_t n, double mean, double std, float* out)
{
    #pragma omp parallel for schedule(static) if (n > (1u << 14))
    for (size_t i = 0; i < n; ++i) out[i] = (float)(mean + std * normal_at(key, i));
}

void synth_normal_bf16(uint64_t key, size_t n, double mean, double std, int absval, uint16_t* out)
{
    #pragma omp parallel for schedule(static) if (n > (1u << 14))
    for (size_t i = 0; i < n; ++i) {
        double v = mean + std * normal_at(key, i);
        if (absval) v = fabs(v);
        out[i] = synth_bf16_from_double(v);
    }
}

/* Byte sizes of one expert in the canonical format. */
size_t synth_codes_bytes(int bits, int rows, int cols) { return (size_t)rows * cols * bits / 8; }

/*
 * One expert in the canonical format:
 *   gate_codes [I][H*bits/8], up_codes [I][H*bits/8], down_codes [H][I*bits/8]
 *   scales, biases: bf16 bit patterns, per expert concatenated
 *     gate [I][H/group] | up [I][H/group] | down [H][I/group]
 * Any output pointer may be NULL to skip that tensor.
 */
void synth_expert(uint64_t seed, int64_t layer, int64_t expert, int bits, int H, int I, int group,
                  double scale_std, double bias_std,
                  uint8_t* gate_codes, uint8_t* up_codes, uint8_t* down_codes,
                  uint16_t* scales, uint16_t* biases)
{
    size_t cb = synth_codes_bytes(bits, I, H);
    size_t ng = (size_t)I * (H / group) * 2 + (size_t)H * (I / group);
    if (gate_codes) synth_bytes(synth_stream_key(seed, layer, expert, SYN_T_GATE_CODES), cb, gate_codes);
    if (up_codes) synth_bytes(synth_stream_key(seed, layer, expert, SYN_T_UP_CODES), cb, up_codes);
    if (down_codes) synth_bytes(synth_stream_key(seed, layer, expert, SYN_T_DOWN_CODES), cb, down_codes);
    if (scales) synth_normal_bf16(synth_stream_key(seed, layer, expert, SYN_T_SCALES), ng, 0.0, scale_std, 1, scales);
    if (biases) synth_normal_bf16(synth_stream_key(seed, layer, expert, SYN_T_BIASES), ng, 0.0, bias_std, 0, biases);
}

/* n_experts consecutive experts [first, first + n) into stacked arrays, parallel over experts. */
void synth_experts(uint64_t seed, int64_t layer, int64_t first, int n, int bits, int H, int I, int group,
                   double scale_std, double bias_std,
                   uint8_t* gate_codes, uint8_t* up_codes, uint8_t* down_codes,
                   uint16_t* scales, uint16_t* biases)
{
    size_t cb = synth_codes_bytes(bits, I, H);
    size_t ng = (size_t)I * (H / group) * 2 + (size_t)H * (I / group);
    #pragma omp parallel for schedule(dynamic, 1)
    for (int j = 0; j < n; ++j) {
        synth_expert(seed, layer, first + j, bits, H, I, group, scale_std, bias_std,
                     gate_codes ? gate_codes + j * cb : NULL, up_codes ? up_codes + j * cb : NULL,
                     down_codes ? down_codes + j * cb : NULL, scales ? scales + j * ng : NULL,
                     biases ? biases + j * ng : NULL);
    }
}

/* Router weights [E][H], N(0, 1/sqrt(H)). */
void synth_router(uint64_t seed, int64_t layer, int E, int H, float* w)
{
    synth_normal_f32(synth_stream_key(seed, layer, -1, SYN_T_ROUTER), (size_t)E * H, 0.0, 1.0 / sqrt((double)H), w);
}

/* Token activations [B][H], N(0,1); step selects the decode step. */
void synth_tokens(uint64_t seed, int64_t step, int B, int H, float* x)
{
    synth_normal_f32(synth_stream_key(seed, -1, step, SYN_T_TOKENS), (size_t)B * H, 0.0, 1.0, x);
}

/* Zipf(s) prior over expert ids, as additive logit bias: -s * ln(e + 1). */
void synth_zipf_bias(int E, double s, float* bias)
{
    for (int e = 0; e < E; ++e) bias[e] = (float)(-s * log((double)e + 1.0));
}
