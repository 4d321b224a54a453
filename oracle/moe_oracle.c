/*
 * CPU oracle for the routed MoE SwiGLU FFN forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library. It shares no code,
 * header, table or helper with the HIP library, and the HIP library never
 * calls it.
 *
 * What it computes follows "Prime Flash MoE - Faster MoE Kernels optimized
 * for Blackwell", section 1 "The computation": for each routed
 * (token, expert) pair, gate|up = W1[e] x_t with W1 stored output-major and
 * gate rows first, act = silu(gate) * up, y = W2[e] act, and the token's
 * output is the routing-weighted sum of its experts' y. The page's naive
 * per-expert loop (same section) fixes the gate-first split of W1's rows
 * and that the routing weight multiplies the expert output. Accumulation
 * is fp32 (the page's accumulators are fp32, section 5 "The two
 * epilogues"), summing over the contraction index in ascending order; the
 * result is rounded once to bf16, round-to-nearest-even.
 *
 * The MX-fp8 variant (same page, section 7 "The MXFP8 variant") takes e4m3
 * codes with one e8m0 scale per 32 contiguous K elements, dequantizes them
 * exactly, and requantizes the SwiGLU output per 32 along H before the
 * down projection (section 7, "The epilogue also quantizes"). The scale
 * rule (MXQ) is the plain reading of "Porting Block-Scaled GEMM Kernels
 * from Blackwell to Rubin", section 6.2 (scale byte by a round-up
 * conversion, then scale and convert to e4m3 with saturation):
 *   amax = max |v| over the 32 values;
 *   amax == 0      -> s = -127;
 *   otherwise      -> s = the smallest integer with amax <= 448 * 2^s,
 *                     clamped to [-127, 127];
 *   scale byte     =  s + 127;
 *   code_i         =  e4m3fn(v_i * 2^-s), round to nearest even, values
 *                     beyond 448 in magnitude saturate to +-448.
 *
 * MXFP4 weights ("GC-MoE on SM120", section on scale formats: 4-bit E2M1
 * codes in blocks of 32 along K, each block with one UE8M0 power-of-two
 * scale; activations stay MX-fp8): e2m1 has 1 sign bit, 2 exponent bits (bias 1) and 1
 * mantissa bit, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6, no infinities or
 * NaN. Two codes share a byte, the even K index in the low nibble. The
 * pages give no scale rule for fp4; MXQ4 reads MXQ with 6 in place of 448:
 * s = the smallest integer with amax <= 6 * 2^s (clamped to [-127, 127],
 * amax == 0 -> -127), codes e2m1(v_i * 2^-s) rounded to nearest, ties to
 * an even code, saturating at 6.
 *
 * Route maps: a stable counting sort of the pairs p = t*k + j by expert
 * (ascending p inside each expert). Ids outside [0, E) are dropped routes:
 * they are not counted and contribute nothing.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------- scalar formats ---------- */

float oracle_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

uint16_t oracle_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u); /* quiet NaN */
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; largest finite magnitude 1.75 * 2^8 = 448. */
float oracle_e4m3_decode(uint8_t c) {
    int sign = c >> 7, ex = (c >> 3) & 15, man = c & 7;
    float mag;
    if (ex == 15 && man == 7) return NAN;
    if (ex == 0)
        mag = ldexpf((float)man, -9);                 /* subnormal: man/8 * 2^-6 */
    else
        mag = ldexpf(1.0f + (float)man / 8.0f, ex - 7);
    return sign ? -mag : mag;
}

/* Round v (finite fp32) to the nearest e4m3fn value, ties to an even
 * mantissa, saturating to +-448; returns the code. */
uint8_t oracle_e4m3_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 448.0) return sign | 0x7e;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                        /* a = m * 2^e, m in [0.5, 1) */
    int unb = e - 1;                     /* a in [2^unb, 2^(unb+1)) */
    if (unb < -6) unb = -6;              /* subnormal range shares 2^-6's quantum */
    double quantum = ldexp(1.0, unb - 3);
    double q = nearbyint(a / quantum);   /* default rounding: nearest, ties to even */
    double r = q * quantum;
    if (r >= 448.0) return sign | 0x7e;  /* can only reach 448 exactly here */
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -6)) return sign | (uint8_t)(r / ldexp(1.0, -9));
    frexp(r, &e);
    int ex = e - 1;                      /* r in [2^ex, 2^(ex+1)) */
    int man = (int)((r / ldexp(1.0, ex) - 1.0) * 8.0);
    return sign | (uint8_t)(((ex + 7) << 3) | man);
}

/* MXQ scale exponent s for one block (see the header comment). */
int oracle_mx_scale_exp(const float* v, int n) {
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) return -127;
    int e;
    double m = frexp((double)amax, &e);  /* amax = m * 2^e; 448 = 0.875 * 2^9 */
    int s = e - 9;                       /* 448 * 2^s = 0.875 * 2^e */
    if (m > 0.875) s += 1;
    if (s < -127) s = -127;
    if (s > 127) s = 127;
    return s;
}

/* Quantize rows x K (K a multiple of 32) of fp32 to e4m3 codes + e8m0 bytes
 * [rows, K/32], scale blocks of 32 contiguous values along K. */
void oracle_mx_quantize(const float* src, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < K / 32; ++b) {
            const float* v = src + r * K + b * 32;
            int s = oracle_mx_scale_exp(v, 32);
            scales[r * (K / 32) + b] = (uint8_t)(s + 127);
            for (int i = 0; i < 32; ++i)
                codes[r * K + b * 32 + i] = oracle_e4m3_encode(ldexpf(v[i], -s));
        }
    }
}

float oracle_mx_value(uint8_t code, uint8_t scale) {
    return ldexpf(oracle_e4m3_decode(code), (int)scale - 127);
}

/* e2m1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa; exponent 0
 * is subnormal (mantissa * 0.5). */
float oracle_e2m1_decode(uint8_t c) {
    int sign = (c >> 3) & 1, ex = (c >> 1) & 3, man = c & 1;
    float mag = ex == 0 ? 0.5f * (float)man : ldexpf(1.0f + 0.5f * (float)man, ex - 1);
    return sign ? -mag : mag;
}

/* Nearest e2m1 value to v (finite), ties to the even code (mantissa bit 0),
 * saturating to +-6; returns the 4-bit code. A search over the 8 codes. */
uint8_t oracle_e2m1_encode(float v) {
    uint8_t sign = signbit(v) ? 8 : 0;
    double a = fabs((double)v);
    if (a >= 6.0) return sign | 7;
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c < 8; ++c) {
        double d = fabs(a - (double)oracle_e2m1_decode((uint8_t)c));
        if (d < best_d || (d == best_d && (best & 1) == 1)) {
            best = c;
            best_d = d;
        }
    }
    return sign | (uint8_t)best;
}

/* MXQ4 scale exponent s for one block (see the header comment). */
int oracle_mx4_scale_exp(const float* v, int n) {
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) return -127;
    int e;
    double m = frexp((double)amax, &e);  /* amax = m * 2^e; 6 = 0.75 * 2^3 */
    int s = e - 3;                       /* 6 * 2^s = 0.75 * 2^e */
    if (m > 0.75) s += 1;
    if (s < -127) s = -127;
    if (s > 127) s = 127;
    return s;
}

/* Quantize rows x K (K a multiple of 32) of fp32 to packed e2m1 codes
 * [rows, K/2] (even index in the low nibble) + e8m0 bytes [rows, K/32]. */
void oracle_mx4_quantize(const float* src, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < K / 32; ++b) {
            const float* v = src + r * K + b * 32;
            int s = oracle_mx4_scale_exp(v, 32);
            scales[r * (K / 32) + b] = (uint8_t)(s + 127);
            for (int i = 0; i < 32; i += 2) {
                uint8_t lo = oracle_e2m1_encode(ldexpf(v[i], -s));
                uint8_t hi = oracle_e2m1_encode(ldexpf(v[i + 1], -s));
                codes[r * (K / 2) + (b * 32 + i) / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
}

/* ---------- route maps ---------- */

/* counts[E], offsets[E+1] (exclusive prefix sum of counts), sorted_to_pair[P]
 * (entries past offsets[E] are -1), pair_to_sorted[P] (-1 for dropped routes). */
void oracle_route(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t* counts,
                  int32_t* offsets, int32_t* sorted_to_pair, int32_t* pair_to_sorted) {
    int64_t P = T * (int64_t)k;
    for (int32_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t p = 0; p < P; ++p)
        if (ids[p] >= 0 && ids[p] < E) counts[ids[p]]++;
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int32_t e = 0; e < E; ++e) next[e] = offsets[e];
    for (int64_t i = 0; i < P; ++i) sorted_to_pair[i] = -1;
    for (int64_t p = 0; p < P; ++p) {
        int32_t e = ids[p];
        if (e < 0 || e >= E) {
            pair_to_sorted[p] = -1;
            continue;
        }
        int32_t i = next[e]++;
        sorted_to_pair[i] = (int32_t)p;
        pair_to_sorted[p] = i;
    }
    free(next);
}

/* ---------- router ---------- */

/* The router the pass starts from ("Prime Flash MoE", section 1 "The
 * computation": each token arrives with its top-k experts and normalized
 * routing weights): probabilities p = softmax(logits) over the E experts;
 * the k most probable experts, most probable first, ties to the lower
 * expert id; their probabilities renormalized to sum to 1.
 *
 * Softmax is strictly increasing in the logit, so "most probable" is
 * "largest logit": the order is taken on the fp32 logits themselves, which
 * fixes the ids exactly (two distinct logits never tie, whatever the
 * rounding of their probabilities). The weights are the picks'
 * probabilities divided by their sum; the softmax normalizer cancels in
 * that ratio, so they are evaluated in double as exp(l_j - max l) over the
 * sum of the picks' exp(l_i - max l), each rounded once to fp32.
 * Inputs the definition leaves open: -0 and +0 are equal logits; a NaN
 * logit ranks below every other logit (-inf included), NaNs among
 * themselves by id, and a NaN among the picks makes the token's weights
 * NaN. */
typedef struct {
    float v;
    int32_t id;
} oracle_scored;

static int oracle_scored_cmp(const void* a, const void* b) {
    const oracle_scored* x = (const oracle_scored*)a;
    const oracle_scored* y = (const oracle_scored*)b;
    const int xn = isnan(x->v), yn = isnan(y->v);
    if (xn != yn) return xn - yn;
    if (xn) return (x->id > y->id) - (x->id < y->id);
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->id > y->id) - (x->id < y->id);
}

void oracle_router(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids, float* wts) {
#pragma omp parallel
    {
        oracle_scored* s = (oracle_scored*)malloc(sizeof(oracle_scored) * (size_t)E);
        double* p = (double*)malloc(sizeof(double) * (size_t)E);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const float* l = logits + t * E;
            float m = -INFINITY;
            for (int32_t e = 0; e < E; ++e)
                if (l[e] > m) m = l[e];
            for (int32_t e = 0; e < E; ++e) {
                p[e] = exp((double)l[e] - (double)m);
                s[e].v = l[e];
                s[e].id = e;
            }
            qsort(s, (size_t)E, sizeof(oracle_scored), oracle_scored_cmp);
            double sel = 0.0;
            for (int32_t j = 0; j < k; ++j) sel += p[s[j].id];
            for (int32_t j = 0; j < k; ++j) {
                ids[t * k + j] = s[j].id;
                wts[t * k + j] = (float)(p[s[j].id] / sel);
            }
        }
        free(s);
        free(p);
    }
}

/* ---------- forward ---------- */

static float silu(float z) { return z / (1.0f + expf(-z)); }

/* One expert on one token, accumulated into acc: gate|up = W1 x (W1
 * [2H, D], gate rows first), act = silu(gate) * up, acc += w * (W2 act)
 * (W2 [D, H]). gu holds 2H floats, act H. */
static void expert_ffn(const float* xv, const uint16_t* W1, const uint16_t* W2, int32_t D, int32_t H, float w,
                       float* gu, float* act, float* acc) {
    for (int32_t n = 0; n < 2 * H; ++n) {
        float s = 0.0f;
        for (int32_t d = 0; d < D; ++d) s += oracle_bf16_to_f32(W1[(int64_t)n * D + d]) * xv[d];
        gu[n] = s;
    }
    for (int32_t h = 0; h < H; ++h) act[h] = silu(gu[h]) * gu[H + h];
    for (int32_t d = 0; d < D; ++d) {
        float s = 0.0f;
        for (int32_t h = 0; h < H; ++h) s += oracle_bf16_to_f32(W2[(int64_t)d * H + h]) * act[h];
        acc[d] += w * s;
    }
}

/* The activation variant ("Porting Block-Scaled GEMM Kernels from Blackwell
 * to Rubin", section 5.3, and "GC-MoE on SM120", sections 4.8 and 5.4):
 * gate and up are first scaled by the expert's global scale alpha[e] (1
 * when alpha is NULL) and, with weight_before_act, by the pair's routing
 * weight, which then no longer scales the expert's output. kind 0 is the
 * plain SwiGLU; kind 1 clamps in the gpt-oss style, the gate from above
 * only and up on both sides, at `limit`, and computes up * silu(gate):
 *   s   = alpha[e] * (weight_before_act ? w : 1)
 *   g'  = s * g,  u' = s * u
 *   act = silu(min(g', limit)) * max(min(u', limit), -limit)   (kind 1)
 *   acc += (weight_before_act ? 1 : w) * (W2 act). */
static void expert_ffn_act(const float* xv, const uint16_t* W1, const uint16_t* W2, int32_t D, int32_t H, float w,
                           int32_t kind, float limit, float alpha_e, int32_t wba, float* gu, float* act,
                           float* acc) {
    for (int32_t n = 0; n < 2 * H; ++n) {
        float s = 0.0f;
        for (int32_t d = 0; d < D; ++d) s += oracle_bf16_to_f32(W1[(int64_t)n * D + d]) * xv[d];
        gu[n] = s;
    }
    const float s_in = wba ? alpha_e * w : alpha_e;
    const float s_out = wba ? 1.0f : w;
    for (int32_t h = 0; h < H; ++h) {
        float g = s_in * gu[h], u = s_in * gu[H + h];
        if (kind == 1) {
            g = fminf(g, limit);
            u = fmaxf(fminf(u, limit), -limit);
        }
        act[h] = silu(g) * u;
    }
    for (int32_t d = 0; d < D; ++d) {
        float s = 0.0f;
        for (int32_t h = 0; h < H; ++h) s += oracle_bf16_to_f32(W2[(int64_t)d * H + h]) * act[h];
        acc[d] += s_out * s;
    }
}

void oracle_forward_bf16_act(int64_t T, int32_t D, int32_t H, int32_t E, int32_t k, const uint16_t* x,
                             const uint16_t* w1, const uint16_t* w2, const int32_t* ids, const float* wts,
                             int32_t kind, float limit, const float* alpha, int32_t wba, uint16_t* out,
                             const int64_t* tokens, int64_t n_tok) {
    if (!tokens) n_tok = T;
#pragma omp parallel
    {
        float* xv = (float*)malloc(sizeof(float) * (size_t)D);
        float* gu = (float*)malloc(sizeof(float) * 2 * (size_t)H);
        float* act = (float*)malloc(sizeof(float) * (size_t)H);
        float* acc = (float*)malloc(sizeof(float) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < n_tok; ++it) {
            int64_t t = tokens ? tokens[it] : it;
            for (int32_t d = 0; d < D; ++d) {
                xv[d] = oracle_bf16_to_f32(x[t * D + d]);
                acc[d] = 0.0f;
            }
            for (int32_t j = 0; j < k; ++j) {
                int32_t e = ids[t * k + j];
                if (e < 0 || e >= E) continue;
                expert_ffn_act(xv, w1 + (int64_t)e * 2 * H * D, w2 + (int64_t)e * D * H, D, H, wts[t * k + j], kind,
                               limit, alpha ? alpha[e] : 1.0f, wba, gu, act, acc);
            }
            for (int32_t d = 0; d < D; ++d) out[t * D + d] = oracle_f32_to_bf16(acc[d]);
        }
        free(xv);
        free(gu);
        free(act);
        free(acc);
    }
}

/* bf16 forward for the tokens listed in `tokens` (n_tok of them; NULL means
 * all T tokens in order). out rows are written at the token's own row.
 * With ws1 != NULL, one shared expert (ws1 [2Hs, D], ws2 [D, Hs]) runs on
 * every token and its output joins the token's sum with weight 1 after the
 * k routed slots ("GC-MoE on SM120", section 4.7: a shared expert is
 * applied to every token, and its output is added into the same fp32 sum
 * that folds the k routed slots). */
void oracle_forward_bf16_shared(int64_t T, int32_t D, int32_t H, int32_t E, int32_t k, const uint16_t* x,
                                const uint16_t* w1, const uint16_t* w2, const int32_t* ids, const float* wts,
                                const uint16_t* ws1, const uint16_t* ws2, int32_t Hs, uint16_t* out,
                                const int64_t* tokens, int64_t n_tok) {
    if (!tokens) n_tok = T;
    const int32_t Hm = ws1 && Hs > H ? Hs : H;
#pragma omp parallel
    {
        float* xv = (float*)malloc(sizeof(float) * (size_t)D);
        float* gu = (float*)malloc(sizeof(float) * 2 * (size_t)Hm);
        float* act = (float*)malloc(sizeof(float) * (size_t)Hm);
        float* acc = (float*)malloc(sizeof(float) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < n_tok; ++it) {
            int64_t t = tokens ? tokens[it] : it;
            for (int32_t d = 0; d < D; ++d) {
                xv[d] = oracle_bf16_to_f32(x[t * D + d]);
                acc[d] = 0.0f;
            }
            for (int32_t j = 0; j < k; ++j) {
                int32_t e = ids[t * k + j];
                if (e < 0 || e >= E) continue;
                expert_ffn(xv, w1 + (int64_t)e * 2 * H * D, w2 + (int64_t)e * D * H, D, H, wts[t * k + j], gu, act,
                           acc);
            }
            if (ws1) expert_ffn(xv, ws1, ws2, D, Hs, 1.0f, gu, act, acc);
            for (int32_t d = 0; d < D; ++d) out[t * D + d] = oracle_f32_to_bf16(acc[d]);
        }
        free(xv);
        free(gu);
        free(act);
        free(acc);
    }
}

void oracle_forward_bf16(int64_t T, int32_t D, int32_t H, int32_t E, int32_t k, const uint16_t* x,
                         const uint16_t* w1, const uint16_t* w2, const int32_t* ids,
                         const float* wts, uint16_t* out, const int64_t* tokens, int64_t n_tok) {
    oracle_forward_bf16_shared(T, D, H, E, k, x, w1, w2, ids, wts, NULL, NULL, 0, out, tokens, n_tok);
}

/* MX forward. x codes [T, D] + scales [T, D/32]; w1 codes [E, 2H, D] +
 * scales [E, 2H, D/32]; w2 codes [E, D, H] + scales [E, D, H/32] (w4: the
 * weight codes packed e2m1, half the bytes per row). The SwiGLU output is
 * requantized with MXQ (e4m3) per 32 along H when requant != 0 (the
 * method's behaviour); requant == 0 keeps it in fp32 (used by a pin). */
/* Weight element idx of a row of K: e4m3 codes [.., K] (w4 == 0) or packed
 * e2m1 codes [.., K/2] (w4 != 0), without its scale. */
static float weight_code_value(const uint8_t* codes, int64_t row, int32_t K, int32_t idx, int32_t w4,
                               const float* lut8, const float* lut4) {
    if (!w4) return lut8[codes[row * K + idx]];
    uint8_t byte = codes[row * (K / 2) + idx / 2];
    return lut4[(idx & 1) ? (byte >> 4) : (byte & 15)];
}

static void forward_mx_any(int64_t T, int32_t D, int32_t H, int32_t E, int32_t k, const uint8_t* xc,
                           const uint8_t* xs, const uint8_t* w1c, const uint8_t* w1s, const uint8_t* w2c,
                           const uint8_t* w2s, const int32_t* ids, const float* wts, uint16_t* out,
                           const int64_t* tokens, int64_t n_tok, int32_t requant, int32_t w4) {
    if (!tokens) n_tok = T;
    /* The tables are exact: e4m3 and e2m1 values carry at most 4 significant
     * bits and 2^(b-127) >= 2^-127, so every product lut * pow2 is an fp32
     * number (smallest magnitude 2^-9 * 2^-127 = 2^-136 > 2^-149). */
    float lut[256], lut4[16], pow2[256];
    for (int c = 0; c < 256; ++c) {
        lut[c] = oracle_e4m3_decode((uint8_t)c);
        pow2[c] = ldexpf(1.0f, c - 127);
    }
    for (int c = 0; c < 16; ++c) lut4[c] = oracle_e2m1_decode((uint8_t)c);
    const int32_t DB = D / 32, HB = H / 32;
#pragma omp parallel
    {
        float* xv = (float*)malloc(sizeof(float) * (size_t)D);
        float* gu = (float*)malloc(sizeof(float) * 2 * (size_t)H);
        float* act = (float*)malloc(sizeof(float) * (size_t)H);
        float* acc = (float*)malloc(sizeof(float) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < n_tok; ++it) {
            int64_t t = tokens ? tokens[it] : it;
            for (int32_t d = 0; d < D; ++d) {
                xv[d] = lut[xc[t * D + d]] * pow2[xs[t * DB + d / 32]];
                acc[d] = 0.0f;
            }
            for (int32_t j = 0; j < k; ++j) {
                int32_t e = ids[t * k + j];
                if (e < 0 || e >= E) continue;
                for (int32_t n = 0; n < 2 * H; ++n) {
                    int64_t row = (int64_t)e * 2 * H + n;
                    float s = 0.0f;
                    for (int32_t d = 0; d < D; ++d)
                        s += weight_code_value(w1c, row, D, d, w4, lut, lut4) * pow2[w1s[row * DB + d / 32]] * xv[d];
                    gu[n] = s;
                }
                for (int32_t h = 0; h < H; ++h) act[h] = silu(gu[h]) * gu[H + h];
                if (requant) {
                    for (int32_t b = 0; b < HB; ++b) {
                        float* v = act + b * 32;
                        int sc = oracle_mx_scale_exp(v, 32);
                        for (int i = 0; i < 32; ++i)
                            v[i] = lut[oracle_e4m3_encode(ldexpf(v[i], -sc))] * pow2[sc + 127];
                    }
                }
                float w = wts[t * k + j];
                for (int32_t d = 0; d < D; ++d) {
                    int64_t row = (int64_t)e * D + d;
                    float s = 0.0f;
                    for (int32_t h = 0; h < H; ++h)
                        s += weight_code_value(w2c, row, H, h, w4, lut, lut4) * pow2[w2s[row * HB + h / 32]] * act[h];
                    acc[d] += w * s;
                }
            }
            for (int32_t d = 0; d < D; ++d) out[t * D + d] = oracle_f32_to_bf16(acc[d]);
        }
        free(xv);
        free(gu);
        free(act);
        free(acc);
    }
}

void oracle_forward_mx(int64_t T, int32_t D, int32_t H, int32_t E, int32_t k, const uint8_t* xc,
                       const uint8_t* xs, const uint8_t* w1c, const uint8_t* w1s, const uint8_t* w2c,
                       const uint8_t* w2s, const int32_t* ids, const float* wts, uint16_t* out,
                       const int64_t* tokens, int64_t n_tok, int32_t requant) {
    forward_mx_any(T, D, H, E, k, xc, xs, w1c, w1s, w2c, w2s, ids, wts, out, tokens, n_tok, requant, 0);
}

/* MXFP4-weight forward: as oracle_forward_mx, with w1 packed e2m1 codes
 * [E, 2H, D/2] and w2 [E, D, H/2] (scales as for MX-fp8); x and the
 * requantized act stay e4m3. */
void oracle_forward_mx4(int64_t T, int32_t D, int32_t H, int32_t E, int32_t k, const uint8_t* xc,
                        const uint8_t* xs, const uint8_t* w1c, const uint8_t* w1s, const uint8_t* w2c,
                        const uint8_t* w2s, const int32_t* ids, const float* wts, uint16_t* out,
                        const int64_t* tokens, int64_t n_tok, int32_t requant) {
    forward_mx_any(T, D, H, E, k, xc, xs, w1c, w1s, w2c, w2s, ids, wts, out, tokens, n_tok, requant, 1);
}

int oracle_num_threads(void) {
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}

/* Threads for the OpenMP loops that follow (the CPU-baseline timing runs the
 * oracle on one thread as well as on all of them). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n < 1 ? 1 : n);
#else
    (void)n;
#endif
}
