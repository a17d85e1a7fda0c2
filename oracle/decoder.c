/*
 * decoder.c -- oracle for one serial decoding step of a small random-init
 * decoder, the model behind the end-to-end verify step.  TEST INFRASTRUCTURE
 * ONLY, like oracle.c (whose number formats, W4 linear, MLP and sampler it
 * uses); nothing in the product path may include, link or call it.
 *
 * What it follows:
 *   [README] TensorFold README, exactness paragraph: drafted decoding writes the
 *            same bytes as serial decoding, one token a round; a verify row gets
 *            the bits of a one-row step.  This file is that one-row step.
 *   [650G]   "Faster, provably the same model", section "TensorFold: the
 *            contract is what it does not change": a draft survives exactly when
 *            it equals the serially sampled token.
 * The layer itself is the standard pre-norm decoder block the pages' models
 * share (RMSNorm, grouped-query attention with rotary positions, SiLU-gated
 * MLP); its details, which the pages leave open, are fixed as follows:
 *   * RMSNorm(x)_i = x_i / sqrt(mean(x^2) + eps) * gain_i, then bf16 (RNE);
 *   * rotary positions, "rotate half": within each head, pair (i, i + d/2) is
 *     turned by the angle p * base^(-2i/d); cos and sin in double, rounded to
 *     fp32, the rotated values rounded to fp32;
 *   * query head h reads key/value head h / (heads / kv_heads);
 *   * keys and values are stored in fp16 (RNE, saturating: a value beyond the
 *     largest finite fp16, 65504, is stored as +-65504, never as infinity) at
 *     slot p of the cache, and the token at slot p attends to slots 0..p;
 *   * scores q.k / sqrt(d), softmax, output sum_j pi_j v_j, all in double; the
 *     output is rounded to bf16 as the o projection's input;
 *   * the residual stream is fp32: each linear output is rounded to fp32, then
 *     the sum.
 * Every operation is an IEEE double operation; roundings happen only at the
 * listed tensor boundaries.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

double ov_bf16_to_f64(uint16_t b);
double ov_f16_to_f64(uint16_t h);
uint16_t ov_f64_to_bf16(double v);
uint16_t ov_f64_to_f16(double v);
void ov_w4_linear_f32(const uint16_t* x, int R, int K, const uint8_t* q,
                      const uint16_t* s, const uint16_t* b, int N, int G, float* y);
void ov_mlp(const uint16_t* x, int R, int H, int I, int G,
            const uint8_t* gq, const uint16_t* gs, const uint16_t* gb,
            const uint8_t* uq, const uint16_t* us, const uint16_t* ub,
            const uint8_t* dq, const uint16_t* ds, const uint16_t* db,
            float* y, float* g_out, float* u_out, uint16_t* h_out);

typedef struct {
    int32_t token;
    double gap;
    int32_t n_cand;
    int32_t n_kept;
    int32_t topp_edge;
} ov_sample_out;
void ov_sample_row(const float* l, int V, int64_t pos, double T, int top_k,
                   double top_p, uint64_t seed, ov_sample_out* out);

/* A cache entry: fp16 by round-to-nearest-even, clamped to the finite range
 * first, so that a large key or value stays finite. */
static uint16_t f16_saturating(double v)
{
    if (v > 65504.0) v = 65504.0;
    if (v < -65504.0) v = -65504.0;
    return ov_f64_to_f16(v);
}

/* RMSNorm of an fp32 vector with fp32 gains, rounded to bf16. */
void ov_rmsnorm_bf16(const float* x, int H, const float* gain, double eps, uint16_t* out)
{
    double ss = 0.0;
    for (int i = 0; i < H; i++)
        ss += (double)x[i] * (double)x[i];
    double r = 1.0 / sqrt(ss / H + eps);
    for (int i = 0; i < H; i++)
        out[i] = ov_f64_to_bf16((double)x[i] * r * (double)gain[i]);
}

/* Rotary position of one head vector v[d] (fp32, in place) at position p. */
void ov_rope(float* v, int d, int64_t p, double base)
{
    int half = d / 2;
    for (int i = 0; i < half; i++) {
        double ang = (double)p * pow(base, -2.0 * i / d);
        double c = (double)(float)cos(ang), s = (double)(float)sin(ang);
        double a = v[i], b = v[i + half];
        v[i] = (float)(a * c - b * s);
        v[i + half] = (float)(b * c + a * s);
    }
}

/* Every fp16 pattern's value, filled once from ov_f16_to_f64 (the same exact
 * conversion, looked up instead of recomputed for each cache entry read). */
static double f16_value[65536];
static int f16_value_ready;

static void f16_table_init(void)
{
    if (f16_value_ready) return;
    for (int h = 0; h < 65536; h++) f16_value[h] = ov_f16_to_f64((uint16_t)h);
    f16_value_ready = 1;
}

/* Attention of one query q[d] (fp32) over n cached slots K/V [n][d] (fp16):
 * o = sum_j softmax_j(q.k_j / sqrt(d)) v_j, in double. */
void ov_attend(const float* q, const uint16_t* K, const uint16_t* V, int n, int d, double* o)
{
    f16_table_init();
    double* s = (double*)malloc(sizeof(double) * (size_t)n);
    double m = -INFINITY;
    for (int j = 0; j < n; j++) {
        double acc = 0.0;
        for (int i = 0; i < d; i++)
            acc += (double)q[i] * f16_value[K[(size_t)j * d + i]];
        s[j] = acc / sqrt((double)d);
        if (s[j] > m) m = s[j];
    }
    double Z = 0.0;
    for (int j = 0; j < n; j++) {
        s[j] = exp(s[j] - m);
        Z += s[j];
    }
    for (int i = 0; i < d; i++) o[i] = 0.0;
    for (int j = 0; j < n; j++) {
        double pj = s[j] / Z;
        for (int i = 0; i < d; i++)
            o[i] += pj * f16_value[V[(size_t)j * d + i]];
    }
    free(s);
}

/* Configuration: ci = {layers, hidden, heads, kv_heads, head_dim, inter,
 * vocab, group}; cd = {rope_base, rms_eps}.
 * Weights w[] (host arrays, standard layouts, per-layer matrices stacked):
 *   0 embed [V][H] bf16           1 attn_norm [L][H] f32   2 mlp_norm [L][H] f32
 *   3 final_norm [H] f32
 *   4-6   qkv  q/s/b  [L][(heads + 2 kv_heads) d][H/2 | H/G]  (q rows, k rows, v rows)
 *   7-9   o    q/s/b  [L][H][heads d / 2 | heads d / G]
 *   10-12 gate q/s/b  [L][I][H/2 | H/G]     13-15 up (same)
 *   16-18 down q/s/b  [L][H][I/2 | I/G]     19-21 lm q/s/b [V][H/2 | H/G]
 * KV caches kc, vc: [L][kv_heads][C][d] fp16, slot p written by this step.
 * One step: token at position p (slot p) -> logits of position p + 1 and the
 * token sampled there. */
enum { CI_L, CI_H, CI_NH, CI_NKV, CI_D, CI_I, CI_V, CI_G };

void ov_decoder_step_h(const int32_t* ci, const double* cd, const void* const* w,
                       uint16_t* kc, uint16_t* vc, int C, int32_t token, int64_t p,
                       double T, int top_k, double top_p, uint64_t seed,
                       float* logits, int32_t* token_out, double* gap_out, uint16_t* hidden_out)
{
    const int L = ci[CI_L], H = ci[CI_H], NH = ci[CI_NH], NKV = ci[CI_NKV], D = ci[CI_D];
    const int I = ci[CI_I], V = ci[CI_V], G = ci[CI_G];
    const double base = cd[0], eps = cd[1];
    const int DQ = NH * D, NQKV = (NH + 2 * NKV) * D;
    const uint16_t* embed = (const uint16_t*)w[0];
    const float* an = (const float*)w[1];
    const float* mn = (const float*)w[2];
    const float* fn = (const float*)w[3];

    float* x = (float*)malloc(sizeof(float) * (size_t)H);
    float* t = (float*)malloc(sizeof(float) * (size_t)(H > NQKV ? H : NQKV));
    uint16_t* nb = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(H > DQ ? H : DQ));
    double* o = (double*)malloc(sizeof(double) * (size_t)NH * D); /* one output per head */

    for (int i = 0; i < H; i++)
        x[i] = (float)ov_bf16_to_f64(embed[(size_t)token * H + i]);

    for (int l = 0; l < L; l++) {
        /* attention block */
        ov_rmsnorm_bf16(x, H, an + (size_t)l * H, eps, nb);
        ov_w4_linear_f32(nb, 1, H,
                         (const uint8_t*)w[4] + (size_t)l * NQKV * (H / 2),
                         (const uint16_t*)w[5] + (size_t)l * NQKV * (H / G),
                         (const uint16_t*)w[6] + (size_t)l * NQKV * (H / G), NQKV, G, t);
        for (int h = 0; h < NH; h++) ov_rope(t + (size_t)h * D, D, p, base);
        for (int g = 0; g < NKV; g++) {
            float* k = t + (size_t)DQ + (size_t)g * D;
            const float* v = t + (size_t)DQ + (size_t)NKV * D + (size_t)g * D;
            ov_rope(k, D, p, base);
            size_t slot = (((size_t)l * NKV + g) * C + (size_t)p) * D;
            for (int i = 0; i < D; i++) {
                kc[slot + i] = f16_saturating(k[i]);
                vc[slot + i] = f16_saturating(v[i]);
            }
        }
        f16_table_init(); /* before the heads run in parallel */
#pragma omp parallel for schedule(static)
        for (int h = 0; h < NH; h++) { /* heads are independent outputs */
            int g = h / (NH / NKV);
            size_t head = ((size_t)l * NKV + g) * C * D;
            double* oh = o + (size_t)h * D;
            ov_attend(t + (size_t)h * D, kc + head, vc + head, (int)(p + 1), D, oh);
            for (int i = 0; i < D; i++) nb[(size_t)h * D + i] = ov_f64_to_bf16(oh[i]);
        }
        ov_w4_linear_f32(nb, 1, DQ,
                         (const uint8_t*)w[7] + (size_t)l * H * (DQ / 2),
                         (const uint16_t*)w[8] + (size_t)l * H * (DQ / G),
                         (const uint16_t*)w[9] + (size_t)l * H * (DQ / G), H, G, t);
        for (int i = 0; i < H; i++) x[i] = (float)((double)x[i] + (double)t[i]);

        /* MLP block */
        ov_rmsnorm_bf16(x, H, mn + (size_t)l * H, eps, nb);
        size_t gi = (size_t)l * I * (H / 2), gs = (size_t)l * I * (H / G);
        size_t di = (size_t)l * H * (I / 2), ds = (size_t)l * H * (I / G);
        ov_mlp(nb, 1, H, I, G,
               (const uint8_t*)w[10] + gi, (const uint16_t*)w[11] + gs, (const uint16_t*)w[12] + gs,
               (const uint8_t*)w[13] + gi, (const uint16_t*)w[14] + gs, (const uint16_t*)w[15] + gs,
               (const uint8_t*)w[16] + di, (const uint16_t*)w[17] + ds, (const uint16_t*)w[18] + ds,
               t, NULL, NULL, NULL);
        for (int i = 0; i < H; i++) x[i] = (float)((double)x[i] + (double)t[i]);
    }

    ov_rmsnorm_bf16(x, H, fn, eps, nb);
    if (hidden_out) memcpy(hidden_out, nb, sizeof(uint16_t) * (size_t)H); /* the LM head's input */
    ov_w4_linear_f32(nb, 1, H, (const uint8_t*)w[19], (const uint16_t*)w[20],
                     (const uint16_t*)w[21], V, G, logits);
    ov_sample_out so;
    ov_sample_row(logits, V, p + 1, T, top_k, top_p, seed, &so);
    if (token_out) *token_out = so.token;
    if (gap_out) *gap_out = so.gap;

    free(x);
    free(t);
    free(nb);
    free(o);
}

/* The step without the hidden row. */
void ov_decoder_step(const int32_t* ci, const double* cd, const void* const* w,
                     uint16_t* kc, uint16_t* vc, int C, int32_t token, int64_t p,
                     double T, int top_k, double top_p, uint64_t seed,
                     float* logits, int32_t* token_out, double* gap_out)
{
    ov_decoder_step_h(ci, cd, w, kc, vc, C, token, p, T, top_k, top_p, seed, logits, token_out, gap_out, NULL);
}

