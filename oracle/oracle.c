/*
 * oracle.c -- plain, slow, serial CPU oracle for the exact drafted-decoding
 * verify pass.  TEST INFRASTRUCTURE ONLY: nothing in the product path may
 * include, link or call this file.  It shares no code, header, table or
 * constant generator with the HIP library; it decodes every number format
 * itself and implements the keyed hash itself.
 *
 * Sources (the pages this follows):
 *   [README]  TensorFold project README (mirror at git.imzlh.top/EugeneClaw/
 *             TensorFold), the paragraph that states the two exactness
 *             guarantees (keyed Gumbel-max token, row-exact verify rows) and the
 *             options table (temperature 0 is greedy, --no-drafts is the serial
 *             reference).
 *   [BLOG]    "TensorFold: The engine that makes local LLMs 2-3x faster -- without
 *             a single token changing" (contextstudios.ai), sections "The
 *             differentiator: byte-exact drafted decoding" and "FAQ".
 *   [650G]    650 Group, "Faster, provably the same model" (marketintelligence
 *             research.com), section "TensorFold: the contract is what it does
 *             not change".
 *   [NEVIZ]   "TensorFold v0.6 ..." (nevizhai.com), section "How exact
 *             speculative decoding works".
 *
 * Arithmetic: every value is computed in IEEE double.  The only roundings are
 * the data-type boundaries the method fixes for its tensors: linear inputs are
 * bf16, linear outputs / logits / the residual stream are fp32, the KV cache is
 * fp16.  Each such rounding is round-to-nearest-even, written out below.
 * Compile with -O2 -fno-fast-math -ffp-contract=off.  OpenMP is used only over
 * independent output columns, which cannot change any value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Number formats.                                                           */
/* ------------------------------------------------------------------------- */

/* bf16 is the top half of an IEEE binary32: value = the float whose bits are
 * (b << 16).  Exact. */
double ov_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.  Exact. */
double ov_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Round a double to the nearest value of a binary format with p significand
 * bits, minimum normal exponent emin and largest finite value maxfin; ties go
 * to the even significand.  Overflow gives +-inf. */
static double round_to_format(double v, int p, int emin, double maxfin)
{
    if (v == 0.0 || !isfinite(v))
        return v;
    int e;
    frexp(v, &e);        /* |v| = f * 2^e, 0.5 <= f < 1 */
    int lead = e - 1;    /* exponent of the leading bit */
    if (lead < emin)
        lead = emin;     /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, lead - (p - 1));
    double r = nearbyint(v / quantum) * quantum; /* default mode: nearest-even */
    if (fabs(r) > maxfin)
        return v > 0 ? INFINITY : -INFINITY;
    return r;
}

uint16_t ov_f64_to_bf16(double v)
{
    if (isnan(v))
        return 0x7FC0;
    double r = round_to_format(v, 8, -126, ldexp(255.0, 120)); /* (2-2^-7)*2^127 */
    float f = (float)r; /* exact: r is a bf16 value, hence a binary32 value */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

uint16_t ov_f64_to_f16(double v)
{
    if (isnan(v))
        return 0x7E00;
    double r = round_to_format(v, 11, -14, 65504.0);
    uint16_t sign = signbit(r) ? 0x8000 : 0;
    double a = fabs(r);
    if (isinf(a))
        return sign | 0x7C00;
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);
    int lead = e - 1;
    if (lead < -14) /* subnormal: a = m * 2^-24 */
        return sign | (uint16_t)ldexp(a, 24);
    uint16_t m = (uint16_t)(ldexp(a, 10 - lead) - 1024.0);
    return sign | (uint16_t)((lead + 15) << 10) | m;
}

float ov_f64_to_f32(double v) { return (float)v; } /* C conversion: nearest-even */

/* ------------------------------------------------------------------------- */
/* Keyed noise: a hash of (seed, position, token id) [README exactness        */
/* paragraph; 650G].  The hash is SplitMix64 (Steele, Lea & Flood, OOPSLA     */
/* 2014): its output function mix64 and its increment gamma.                  */
/* ------------------------------------------------------------------------- */

#define OV_GAMMA 0x9E3779B97F4A7C15ULL

uint64_t ov_mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Row key: the (pos+1)-th output of a SplitMix64 stream whose state starts at
 * mix64(seed).  Token hash: the (tok+1)-th output of the stream that starts at
 * the row key. */
uint64_t ov_noise_hash(uint64_t seed, int64_t pos, int32_t tok)
{
    uint64_t row = ov_mix64(ov_mix64(seed) + (uint64_t)(pos + 1) * OV_GAMMA);
    return ov_mix64(row + (uint64_t)((int64_t)tok + 1) * OV_GAMMA);
}

/* Uniform in (0,1): the top 52 bits plus one half, over 2^52, so u is never 0
 * or 1.  Gumbel(0,1) by inversion: g = -log(-log(u)). */
double ov_uniform(uint64_t h) { return ((double)(h >> 12) + 0.5) * 0x1p-52; }
double ov_gumbel(uint64_t h) { return -log(-log(ov_uniform(h))); }

/* ------------------------------------------------------------------------- */
/* W4 linear: y[r][n] = sum_k x[r][k] * w[n][k], with the affine group        */
/* dequantisation w[n][k] = s[n][k/G] * q[n][k] + b[n][k/G].  4-bit weights in */
/* groups of 32 or 64 ([BLOG] "The numbers": same 4-bit checkpoints; [README] */
/* checkpoint list: groups of 64 / of 32).  q is packed two per byte, the low */
/* nibble holding the even k:  q[n][k] = (byte[n][k/2] >> (4*(k%2))) & 15.    */
/* Each row r is computed alone, in order.                                   */
/* ------------------------------------------------------------------------- */

static int q_at(const uint8_t* q, int K, int n, int k)
{
    uint8_t byte = q[(size_t)n * (size_t)(K / 2) + (size_t)(k / 2)];
    return (k % 2 == 0) ? (byte & 15) : (byte >> 4);
}

void ov_w4_linear(const uint16_t* x, int R, int K, const uint8_t* q,
                  const uint16_t* s, const uint16_t* b, int N, int G, double* y)
{
    int ng = K / G;
    double* xd = (double*)malloc(sizeof(double) * (size_t)K);
    for (int r = 0; r < R; r++) {
        for (int k = 0; k < K; k++)
            xd[k] = ov_bf16_to_f64(x[(size_t)r * K + k]);
#pragma omp parallel for schedule(static)
        for (int n = 0; n < N; n++) {
            double acc = 0.0;
            double sc = 0.0, bi = 0.0; /* the current group's scale and bias */
            for (int k = 0; k < K; k++) {
                if (k % G == 0) {
                    sc = ov_f16_to_f64(s[(size_t)n * ng + k / G]);
                    bi = ov_f16_to_f64(b[(size_t)n * ng + k / G]);
                }
                double w = sc * (double)q_at(q, K, n, k) + bi;
                acc += w * xd[k];
            }
            y[(size_t)r * N + n] = acc;
        }
    }
    free(xd);
}

/* The same linear with its output rounded to the method's output type, fp32. */
void ov_w4_linear_f32(const uint16_t* x, int R, int K, const uint8_t* q,
                      const uint16_t* s, const uint16_t* b, int N, int G, float* y)
{
    double* t = (double*)malloc(sizeof(double) * (size_t)R * N);
    ov_w4_linear(x, R, K, q, s, b, N, G, t);
    for (size_t i = 0; i < (size_t)R * N; i++)
        y[i] = (float)t[i];
    free(t);
}

/* The same linear evaluated in fp32, in the two-level order of its groups:  */
/* w = fl(fl(s * q) + b); per group g, p_g = the fp32 sum of fl(w * x) over   */
/* the group's k in ascending order, from 0; y = the fp32 sum of the p_g in   */
/* ascending g.  Every operation is one binary32 operation (no contraction). */
/* This is the fp32 form of the definition; ov_w4_linear (fp64, one rounding */
/* at the output) decides when it and another fp32 evaluation disagree.      */
void ov_w4_linear_fp32(const uint16_t* x, int R, int K, const uint8_t* q,
                       const uint16_t* s, const uint16_t* b, int N, int G, float* y)
{
    int ng = K / G;
    float* xf = (float*)malloc(sizeof(float) * (size_t)K);
    for (int r = 0; r < R; r++) {
        for (int k = 0; k < K; k++)
            xf[k] = (float)ov_bf16_to_f64(x[(size_t)r * K + k]);
#pragma omp parallel for schedule(static)
        for (int n = 0; n < N; n++) {
            float total = 0.0f;
            for (int g = 0; g < ng; g++) {
                float sc = (float)ov_f16_to_f64(s[(size_t)n * ng + g]);
                float bi = (float)ov_f16_to_f64(b[(size_t)n * ng + g]);
                float part = 0.0f;
                for (int k = g * G; k < (g + 1) * G; k++) {
                    float sq = sc * (float)q_at(q, K, n, k);
                    float w = sq + bi;
                    float wx = w * xf[k];
                    part = part + wx;
                }
                total = total + part;
            }
            y[(size_t)r * N + n] = total;
        }
    }
    free(xf);
}

/* ------------------------------------------------------------------------- */
/* A second 4-bit format: NVFP4-style block scales [blog "The honest limits": */
/* NVFP4 checkpoints].  w[n][k] = e2m1(q[n][k]) * e4m3(s[n][k/16]) * s_t:     */
/*   q  [N][K/2] bytes, two FP4 E2M1 codes per byte, low nibble = even k;     */
/*   s  [N][K/16] FP8 E4M3 block scales (one per 16 k);                       */
/*   s_t one fp32 scale for the whole tensor.                                 */
/* E2M1 (the OCP microscaling formats' FP4): sign, 2 exponent bits (bias 1),  */
/* 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives.            */
/* E4M3 (OCP, "FN": no infinities): sign, 4 exponent bits (bias 7), 3         */
/* mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN.    */
/* ------------------------------------------------------------------------- */

double ov_e2m1_to_f64(int code)
{
    int sign = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -v : v;
}

double ov_e4m3_to_f64(uint8_t b)
{
    int sign = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* y[r][n] = sum_k x[r][k] * w[n][k] in fp64, rows one at a time, rounded to fp32. */
void ov_nvfp4_linear_f32(const uint16_t* x, int R, int K, const uint8_t* q, const uint8_t* s,
                         float s_t, int N, float* y)
{
    double* xd = (double*)malloc(sizeof(double) * (size_t)K);
    for (int r = 0; r < R; r++) {
        for (int k = 0; k < K; k++)
            xd[k] = ov_bf16_to_f64(x[(size_t)r * K + k]);
#pragma omp parallel for schedule(static)
        for (int n = 0; n < N; n++) {
            double acc = 0.0;
            for (int k = 0; k < K; k++) {
                double w = ov_e2m1_to_f64(q_at(q, K, n, k)) *
                           ov_e4m3_to_f64(s[(size_t)n * (K / 16) + k / 16]) * (double)s_t;
                acc += w * xd[k];
            }
            y[(size_t)r * N + n] = (float)acc;
        }
    }
    free(xd);
}

/* ------------------------------------------------------------------------- */
/* SiLU-gated MLP glue: h = bf16(silu(g) * u), silu(v) = v / (1 + e^-v).      */
/* ------------------------------------------------------------------------- */

double ov_silu(double v) { return v / (1.0 + exp(-v)); }

void ov_silu_mul_bf16(const float* g, const float* u, size_t n, uint16_t* h)
{
    for (size_t i = 0; i < n; i++)
        h[i] = ov_f64_to_bf16(ov_silu((double)g[i]) * (double)u[i]);
}

/* Dense MLP slice: gate and up W4 linears H->I, the glue, down W4 linear I->H.
 * Optional intermediates (g, u as fp32, h as bf16) are returned when non-NULL. */
void ov_mlp(const uint16_t* x, int R, int H, int I, int G,
            const uint8_t* gq, const uint16_t* gs, const uint16_t* gb,
            const uint8_t* uq, const uint16_t* us, const uint16_t* ub,
            const uint8_t* dq, const uint16_t* ds, const uint16_t* db,
            float* y, float* g_out, float* u_out, uint16_t* h_out)
{
    size_t ri = (size_t)R * I;
    float* g = (float*)malloc(sizeof(float) * ri);
    float* u = (float*)malloc(sizeof(float) * ri);
    uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * ri);
    ov_w4_linear_f32(x, R, H, gq, gs, gb, I, G, g);
    ov_w4_linear_f32(x, R, H, uq, us, ub, I, G, u);
    ov_silu_mul_bf16(g, u, ri, h);
    ov_w4_linear_f32(h, R, I, dq, ds, db, H, G, y);
    if (g_out) memcpy(g_out, g, sizeof(float) * ri);
    if (u_out) memcpy(u_out, u, sizeof(float) * ri);
    if (h_out) memcpy(h_out, h, sizeof(uint16_t) * ri);
    free(g);
    free(u);
    free(h);
}

/* ------------------------------------------------------------------------- */
/* Keyed sampler [README exactness paragraph; 650G]: the token at position p  */
/* is the argmax, over the top-k / top-p candidates, of l/T + g(seed, p, id). */
/* Temperature 0 is greedy [README options table].                            */
/* Order used for every selection and tie: larger logit first, then the lower */
/* token id.                                                                  */
/* ------------------------------------------------------------------------- */

static int ranks_before(const float* l, int a, int b) /* a before b? */
{
    return l[a] > l[b] || (l[a] == l[b] && a < b);
}

/* The k first token ids under (logit desc, id asc), by k scans of the row. */
int ov_topk(const float* l, int V, int k, int32_t* ids)
{
    if (k > V) k = V;
    char* taken = (char*)calloc((size_t)V, 1);
    for (int j = 0; j < k; j++) {
        int best = -1;
        for (int i = 0; i < V; i++)
            if (!taken[i] && (best < 0 || ranks_before(l, i, best)))
                best = i;
        taken[best] = 1;
        ids[j] = best;
    }
    free(taken);
    return k;
}

typedef struct {
    int32_t token;    /* sampled token id */
    double gap;       /* best minus second-best perturbed score (+inf if one) */
    int32_t n_cand;   /* candidates after top-k */
    int32_t n_kept;   /* candidates after top-p */
    int32_t topp_edge;/* 1 if the nucleus cut lies within 1e-9*Z of top_p*Z */
} ov_sample_out;

/* Second stage: top-p over the n ordered candidates, then the keyed argmax.
 * cand[] must be ordered (logit desc, id asc). */
void ov_sample_from_candidates(const float* l, const int32_t* cand, int n,
                               int64_t pos, double T, double top_p,
                               uint64_t seed, ov_sample_out* out)
{
    double* e = (double*)malloc(sizeof(double) * (size_t)n);
    double m = (double)l[cand[0]];
    double Z = 0.0;
    for (int j = 0; j < n; j++) {
        e[j] = exp(((double)l[cand[j]] - m) / T);
        Z += e[j];
    }
    /* nucleus: candidate j stays while the mass strictly before it is below
     * top_p * Z; candidate 0 always stays. */
    int kept = 0;
    double before = 0.0;
    int edge = 0;
    for (int j = 0; j < n; j++) {
        if (j > 0 && !(before < top_p * Z))
            break;
        kept = j + 1;
        before += e[j];
    }
    /* flag a cut whose decision lies within 1e-9 Z of the threshold */
    {
        double acc = 0.0;
        for (int j = 0; j < n; j++) {
            if (j > 0 && fabs(acc - top_p * Z) < 1e-9 * Z)
                edge = 1;
            acc += e[j];
        }
    }
    int best = -1;
    double zb = -INFINITY, z2 = -INFINITY;
    for (int j = 0; j < kept; j++) {
        int t = cand[j];
        double z = (double)l[t] / T + ov_gumbel(ov_noise_hash(seed, pos, t));
        if (best < 0 || z > zb || (z == zb && t < best)) {
            z2 = zb;
            zb = z;
            best = t;
        } else if (z > z2) {
            z2 = z;
        }
    }
    out->token = best;
    out->gap = (kept > 1) ? zb - z2 : INFINITY;
    out->n_cand = n;
    out->n_kept = kept;
    out->topp_edge = edge;
    free(e);
}

/* Top-p over the whole vocabulary (top_k == 0).  The nucleus cut reads the  */
/* masses in fixed point so that they can be added in any order to the same  */
/* total: with the tokens ordered (logit desc, id asc) and m the largest      */
/* logit, token j's mass is the integer e_j = nearest(exp((l_j - m) / T) *    */
/* 2^40) (the largest token's is 2^40), Z = sum of all e_j (< 2^58), and the  */
/* threshold thr = max(1, trunc(fl(top_p * fl(Z)))) in fp64.  Token j is     */
/* kept iff the mass of the tokens before it is below thr (token 0 always).   */
/* Then the keyed argmax over the kept tokens, as for the candidates above.   */
/* topp_edge flags a cut within Z / 2^30 of thr.                              */
#define OV_FX_SCALE 1099511627776.0 /* 2^40 */

static const float* g_sort_l; /* qsort's view of the row */
static int cmp_rank(const void* a, const void* b)
{
    int i = *(const int32_t*)a, j = *(const int32_t*)b;
    if (ranks_before(g_sort_l, i, j)) return -1;
    if (ranks_before(g_sort_l, j, i)) return 1;
    return 0;
}

void ov_sample_topp_full(const float* l, int V, int64_t pos, double T, double top_p,
                         uint64_t seed, ov_sample_out* out)
{
    int32_t* ord = (int32_t*)malloc(sizeof(int32_t) * (size_t)V);
    uint64_t* e = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)V);
    for (int i = 0; i < V; i++) ord[i] = i;
    g_sort_l = l;
    qsort(ord, (size_t)V, sizeof(int32_t), cmp_rank);
    double m = (double)l[ord[0]];
    uint64_t Z = 0;
    for (int j = 0; j < V; j++) {
        e[j] = (uint64_t)nearbyint(exp(((double)l[ord[j]] - m) / T) * OV_FX_SCALE);
        Z += e[j];
    }
    uint64_t thr = (uint64_t)(top_p * (double)Z);
    if (thr < 1) thr = 1;
    int kept = 0, edge = 0;
    uint64_t before = 0;
    for (int j = 0; j < V; j++) {
        if (j > 0 && !(before < thr)) break;
        kept = j + 1;
        before += e[j];
    }
    {
        uint64_t acc = 0;
        double tol = (double)Z / 1073741824.0; /* Z / 2^30 */
        for (int j = 0; j < V; j++) {
            if (j > 0 && fabs((double)acc - (double)thr) < tol) edge = 1;
            acc += e[j];
        }
    }
    int best = -1;
    double zb = -INFINITY, z2 = -INFINITY;
    for (int j = 0; j < kept; j++) {
        int t = ord[j];
        double z = (double)l[t] / T + ov_gumbel(ov_noise_hash(seed, pos, t));
        if (best < 0 || z > zb || (z == zb && t < best)) {
            z2 = zb;
            zb = z;
            best = t;
        } else if (z > z2) {
            z2 = z;
        }
    }
    out->token = best;
    out->gap = (kept > 1) ? zb - z2 : INFINITY;
    out->n_cand = V;
    out->n_kept = kept;
    out->topp_edge = edge;
    free(ord);
    free(e);
}

/* One row: greedy when T == 0, else top-k (none when top_k == 0), top-p and  */
/* the keyed argmax. */
void ov_sample_row(const float* l, int V, int64_t pos, double T, int top_k,
                   double top_p, uint64_t seed, ov_sample_out* out)
{
    if (T == 0.0) {
        int best = 0;
        for (int i = 1; i < V; i++)
            if (ranks_before(l, i, best))
                best = i;
        int second = -1;
        for (int i = 0; i < V; i++)
            if (i != best && (second < 0 || ranks_before(l, i, second)))
                second = i;
        out->token = best;
        out->gap = (second < 0) ? INFINITY : (double)l[best] - (double)l[second];
        out->n_cand = V;
        out->n_kept = 1;
        out->topp_edge = 0;
        return;
    }
    if (top_k == 0) { /* no top-k: top-p over the whole vocabulary */
        ov_sample_topp_full(l, V, pos, T, top_p, seed, out);
        return;
    }
    int k = top_k < V ? top_k : V;
    int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    ov_topk(l, V, k, cand);
    ov_sample_from_candidates(l, cand, k, pos, T, top_p, seed, out);
    free(cand);
}

/* Serial sampling of R rows, one at a time. */
void ov_sample_rows(const float* logits, int R, int V, const int64_t* pos,
                    double T, int top_k, double top_p, uint64_t seed,
                    int32_t* tokens, double* gaps, int32_t* n_kept, int32_t* edge)
{
    for (int r = 0; r < R; r++) {
        ov_sample_out o;
        ov_sample_row(logits + (size_t)r * V, V, pos[r], T, top_k, top_p, seed, &o);
        tokens[r] = o.token;
        if (gaps) gaps[r] = o.gap;
        if (n_kept) n_kept[r] = o.n_kept;
        if (edge) edge[r] = o.topp_edge;
    }
}

/* ------------------------------------------------------------------------- */
/* Accept rule [README; BLOG FAQ; 650G]: a draft is accepted exactly when it  */
/* equals the token serial decoding samples there.  Row i's sample is         */
/* compared with draft i; the leading run of equal pairs is accepted, and the */
/* next row's sample is committed with it (capped at the R rows sampled).     */
/* ------------------------------------------------------------------------- */

void ov_accept(const int32_t* sampled, int R, const int32_t* draft, int D,
               int32_t* n_accept, int32_t* n_commit)
{
    int a = 0;
    while (a < D && draft[a] == sampled[a])
        a++;
    *n_accept = a;
    *n_commit = (a + 1 < R) ? a + 1 : R;
}

/* ------------------------------------------------------------------------- */
/* MoE verify layer (30B-A3B-like): router softmax, top-E_k experts, weights  */
/* renormalised over the chosen experts, each expert a SwiGLU MLP of W4        */
/* linears, outputs summed in rank order.  Every lane is routed on its own.   */
/* Expert e's matrices sit at offset e in each stacked array.                 */
/* ------------------------------------------------------------------------- */

void ov_moe_route(const float* rho, int E, int top, int32_t* ids, double* w)
{
    /* softmax over all experts */
    double m = -INFINITY;
    for (int e = 0; e < E; e++)
        if ((double)rho[e] > m) m = (double)rho[e];
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    double S = 0.0;
    for (int e = 0; e < E; e++) {
        p[e] = exp((double)rho[e] - m);
        S += p[e];
    }
    for (int e = 0; e < E; e++)
        p[e] /= S;
    /* top experts by router logit (the softmax is increasing), lower id on ties */
    ov_topk(rho, E, top, ids);
    double sel = 0.0;
    for (int j = 0; j < top; j++)
        sel += p[ids[j]];
    for (int j = 0; j < top; j++)
        w[j] = p[ids[j]] / sel;
    free(p);
}

void ov_moe(const uint16_t* x, const float* rho, int R, int H, int I, int E,
            int top, int G,
            const uint8_t* gq, const uint16_t* gs, const uint16_t* gb,
            const uint8_t* uq, const uint16_t* us, const uint16_t* ub,
            const uint8_t* dq, const uint16_t* ds, const uint16_t* db,
            float* y, int32_t* ids_out, double* w_out)
{
    size_t qi = (size_t)I * H / 2, si = (size_t)I * H / G; /* gate/up per expert */
    size_t qd = (size_t)H * I / 2, sd = (size_t)H * I / G; /* down per expert */
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)top);
    double* w = (double*)malloc(sizeof(double) * (size_t)top);
    float* ye = (float*)malloc(sizeof(float) * (size_t)H);
    double* acc = (double*)malloc(sizeof(double) * (size_t)H);
    for (int r = 0; r < R; r++) {
        ov_moe_route(rho + (size_t)r * E, E, top, ids, w);
        for (int i = 0; i < H; i++) acc[i] = 0.0;
        for (int j = 0; j < top; j++) {
            int e = ids[j];
            ov_mlp(x + (size_t)r * H, 1, H, I, G,
                   gq + e * qi, gs + e * si, gb + e * si,
                   uq + e * qi, us + e * si, ub + e * si,
                   dq + e * qd, ds + e * sd, db + e * sd, ye, NULL, NULL, NULL);
            for (int i = 0; i < H; i++)
                acc[i] += w[j] * (double)ye[i];
        }
        for (int i = 0; i < H; i++)
            y[(size_t)r * H + i] = (float)acc[i];
        if (ids_out) memcpy(ids_out + (size_t)r * top, ids, sizeof(int32_t) * top);
        if (w_out) memcpy(w_out + (size_t)r * top, w, sizeof(double) * top);
    }
    free(ids);
    free(w);
    free(ye);
    free(acc);
}

/* Harness loop for statistical tests: n independent calls of ov_sample_row on
 * one logit row, call i with position pos[i] and seed seeds[i]. */
void ov_sample_many(const float* l, int V, int n, const int64_t* pos,
                    const uint64_t* seeds, double T, int top_k, double top_p,
                    int32_t* tokens)
{
    for (int i = 0; i < n; i++) {
        ov_sample_out o;
        ov_sample_row(l, V, pos[i], T, top_k, top_p, seeds[i], &o);
        tokens[i] = o.token;
    }
}

/* Threads OpenMP would use for the column loops (reported with timings), and
 * a way to set them (timings with one thread); neither changes any value. */
#ifdef _OPENMP
#include <omp.h>
int ov_num_threads(void) { return omp_get_max_threads(); }
void ov_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int ov_num_threads(void) { return 1; }
void ov_set_num_threads(int n) { (void)n; }
#endif
