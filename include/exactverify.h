/*
 * exactverify.h -- C ABI of libexactverify.so, the multi-row verify pass of
 * exact ("byte-identical") drafted decoding on AMD Instinct MI355X (gfx950).
 *
 * What the method computes (sources, by page and part):
 *   - TensorFold README (project page mirror), the exactness paragraph: the
 *     token at position p is the argmax over the top-k/top-p candidates of
 *     logit/T + g(seed, p, token), g Gumbel noise from a hash of seed, position
 *     and token id; and a row of a multi-row verify pass gets the same bits as a
 *     one-row step.  Options table: temperature 0 is greedy; --no-drafts (one
 *     token a round) is the serial reference.
 *   - "TensorFold: The engine that makes local LLMs 2-3x faster ...", section
 *     "The differentiator: byte-exact drafted decoding": drafts are verified as
 *     several rows ("lanes") of one forward pass; sampling is keyed.  FAQ: the
 *     target keeps exactly the guessed tokens it would have chosen itself.
 *   - 650 Group, "TensorFold: the contract is what it does not change": the same
 *     two rules, restated.
 *
 * Conventions for every entry point
 *   - Pointers marked (device) are device memory on the current HIP device;
 *     (host) pointers are read before the call returns.  The caller allocates and
 *     owns every buffer; the library allocates device memory in two calls only:
 *     toy_decoder_create (the handle's rotation table) and ev_w4_timing(1).
 *   - bf16 and fp16 values travel as their raw uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue work
 *     and return without synchronising; outputs are valid once the stream has
 *     reached that point.
 *   - Return value: EV_OK, or a negative EV_E* code.  Arguments are validated
 *     before anything is enqueued, so on error no output is written.
 *     ev_last_error() then returns a message (thread-local).
 *   - Row exactness: for any R, row r's outputs are bit-identical to those of a
 *     call with R = 1 on row r alone.  Internal tiling, split counts and
 *     workspace sizes are functions of (N, K, G) or V, never of R.
 */
#ifndef EXACTVERIFY_H
#define EXACTVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EV_OK 0
#define EV_EINVAL (-1)      /* bad pointer, size, alignment or parameter value */
#define EV_EUNSUPPORTED (-2)/* a valid value the library does not handle     */
#define EV_EHIP (-3)        /* the HIP runtime reported an error             */
#define EV_EWORKSPACE (-4)  /* workspace pointer NULL or smaller than needed */

#define EV_MAX_LANES 16     /* R, the rows of one verify pass, is 1..16     */
#define EV_MAX_TOPK 64      /* top_k limit when sampling (T > 0)             */

/* Message for the last error on this thread ("" if none). */
const char* ev_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int32_t ev_version(void);

/* ------------------------------------------------------------------------- */
/* W4 weights: standard layout and the packed layout the kernels stream.     */
/*                                                                            */
/* Four-bit weights in groups of 32 or 64 with an affine dequantisation      */
/* w[n][k] = s[n][k/G] * q[n][k] + b[n][k/G] (the "4-bit checkpoints" of the  */
/* blog's "The numbers" section; the README's checkpoint list gives groups of */
/* 64 and of 32).  Standard layout of an N x K matrix:                        */
/*   q  [N][K/2] bytes: byte k/2 of row n holds q[n][k] in its low nibble     */
/*      when k is even, its high nibble when k is odd;                        */
/*   s, b [N][K/G] fp16.                                                      */
/* w4_pack copies a matrix, once (at load), into the packed layout: tiles of  */
/* 16 rows by chunks of 128 k, each tile-chunk holding its 1 KB of codes in   */
/* the order the kernels' lanes read them, followed by its (scale, bias)      */
/* pairs.  The copy is exact; rows and k beyond N and K are zero padding, so  */
/* for N % 16 == 0 and K % 128 == 0 the packed bytes equal the standard ones. */
/*   q (device, 4-byte aligned), s, b (device, 2-byte aligned): inputs.       */
/*   packed (device, 16-byte aligned) of at least w4_packed_bytes(N, K, G).   */
/* Limits: K > 0, K % G == 0, K % 32 == 0; N > 0; G in {32, 64}; packed size  */
/* below 2^31 bytes.  Errors: EV_EINVAL, EV_EUNSUPPORTED, EV_EHIP.            */
/* ------------------------------------------------------------------------- */
size_t w4_packed_bytes(int32_t N, int32_t K, int32_t G);
int32_t w4_pack(const uint8_t* q, const uint16_t* scale_f16, const uint16_t* bias_f16,
                int32_t N, int32_t K, int32_t G, void* packed, size_t packed_bytes,
                void* stream);

/* ------------------------------------------------------------------------- */
/* W4 verify linear.                                                          */
/*                                                                            */
/* y[r][n] = sum_k x[r][k] * (s[n][k/G] * q[n][k] + b[n][k/G]),  r < R, n < N, */
/* for the R draft rows ("lanes") of one verify pass, which share one read of */
/* the weights (blog, "The differentiator: byte-exact drafted decoding").    */
/*   x_bf16   (device) [R][K] bf16, 16-byte aligned.                          */
/*   w_packed (device) the matrix as written by w4_pack, 16-byte aligned.     */
/*   y        (device) [R][N] fp32, written.                                  */
/*   ws       (device) workspace of at least verify_linear_w4_workspace(K,N,G) */
/*            bytes, 256-byte aligned; contents are scratch.                  */
/* Limits: 1 <= R <= 16 and those of w4_pack.  Errors: EV_EINVAL,             */
/* EV_EUNSUPPORTED, EV_EWORKSPACE, EV_EHIP.                                   */
/* Reduction order: fixed per n by (N, K, G) -- never by R.                   */
/* ------------------------------------------------------------------------- */
size_t verify_linear_w4_workspace(int32_t K, int32_t N, int32_t G);
int32_t verify_linear_w4(const uint16_t* x_bf16, int32_t R, int32_t K, const void* w_packed,
                         int32_t N, int32_t G, float* y, void* ws, size_t ws_bytes,
                         void* stream);

/* The same linear on standard-layout weights (q [N][K/2], scale and bias     */
/* [N][K/G] fp16, as w4_pack takes them), for callers that do not keep a      */
/* packed copy: the call packs the matrix into the front of its workspace     */
/* (w4_pack) and runs verify_linear_w4 on it, so y is bit-identical to        */
/* verify_linear_w4 on the packed matrix; the weights are streamed twice.     */
/*   ws (device) at least verify_linear_w4_standard_workspace(K, N, G) bytes, */
/*   256-byte aligned; contents are scratch.  Pointers and limits: those of   */
/*   w4_pack and verify_linear_w4, all checked before anything is launched.   */
size_t verify_linear_w4_standard_workspace(int32_t K, int32_t N, int32_t G);
int32_t verify_linear_w4_standard(const uint16_t* x_bf16, int32_t R, int32_t K, const uint8_t* q,
                                  const uint16_t* scale_f16, const uint16_t* bias_f16, int32_t N,
                                  int32_t G, float* y, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- */
/* A second 4-bit format: NVFP4-style block scales (the blog's "The honest    */
/* limits" section: NVFP4 checkpoints).                                       */
/*                                                                            */
/* w[n][k] = e2m1(q[n][k]) * e4m3(s[n][k/16]) * tensor_scale, with           */
/*   q [N][K/2] bytes: two FP4 E2M1 codes per byte (sign, 2 exponent bits of  */
/*     bias 1, 1 mantissa bit: 0 .. 6), low nibble = even k;                 */
/*   s [N][K/16] bytes: one FP8 E4M3 scale (OCP, no infinities) per 16 k.     */
/* nvfp4_pack copies a matrix once into the packed layout the kernel streams  */
/* (tiles of 16 rows by chunks of 128 k: 1 KB of codes in the kernel's lane   */
/* order, then the rows' 8 block scales; nvfp4_packed_bytes(N, K) bytes, the  */
/* standard N*K/2 + N*K/16 when N % 16 == 0 and K % 128 == 0).               */
/* verify_linear_nvfp4: y[r][n] = sum_k x[r][k] * w[n][k] for the R <= 16     */
/* rows, arguments as verify_linear_w4 (workspace from                        */
/* verify_linear_nvfp4_workspace), with the same row exactness: the order of  */
/* every reduction is fixed by (N, K).  Limits: K > 0, K % 32 == 0, N > 0,    */
/* tensor_scale finite.  Errors: EV_EINVAL, EV_EUNSUPPORTED, EV_EWORKSPACE,   */
/* EV_EHIP.                                                                   */
/* ------------------------------------------------------------------------- */
size_t nvfp4_packed_bytes(int32_t N, int32_t K);
int32_t nvfp4_pack(const uint8_t* q, const uint8_t* scale_e4m3, int32_t N, int32_t K, void* packed,
                   size_t packed_bytes, void* stream);
size_t verify_linear_nvfp4_workspace(int32_t K, int32_t N);
int32_t verify_linear_nvfp4(const uint16_t* x_bf16, int32_t R, int32_t K, const void* w_packed,
                            int32_t N, float tensor_scale, float* y, void* ws, size_t ws_bytes,
                            void* stream);

/* ------------------------------------------------------------------------- */
/* SiLU-gated MLP verify slice (dense).                                       */
/*                                                                            */
/*   g = W_gate x, u = W_up x          (W4 linears H -> I, fp32 out)          */
/*   h = bf16_rne(silu(g) * u),  silu(v) = v / (1 + e^-v)  (fp32)             */
/*   y = W_down h                      (W4 linear I -> H, fp32 out)           */
/* Each W4 linear is the one defined above; the three matrices are passed     */
/* packed (gate and up I x H, down H x I).  The order in which g and u are    */
/* summed over K is fixed by (H, I, G) -- never by R: two halves of K when    */
/* the pair's columns alone fill the GPU, else fixed K-segments added in      */
/* ascending order.                                                           */
/*   h_bf16  (device, optional, 16-byte aligned) [R][I] bf16: if non-NULL, h  */
/*           is also written there.                                           */
/* Limits as verify_linear_w4 for both shapes.                                */
/* ------------------------------------------------------------------------- */
size_t verify_mlp_w4_workspace(int32_t H, int32_t I, int32_t G);
int32_t verify_mlp_w4(const uint16_t* x_bf16, int32_t R, int32_t H, int32_t I, int32_t G,
                      const void* gate_packed, const void* up_packed, const void* down_packed,
                      float* y, uint16_t* h_bf16, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- */
/* The MLP slice for callers that cannot allocate device memory: code under   */
/* HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.   */
/*                                                                            */
/* verify_mlp_w4 without the workspace arguments: the same launches, results  */
/* bit-identical to verify_mlp_w4's.  The workspace is a device array inside  */
/* the library, EV_MLP_SCRATCH_BYTES long, one per GPU the library runs on,   */
/* held until the process ends.  The call allocates nothing (no hipMalloc, no */
/* allocating library routine); the first call on a device looks the array's */
/* address up once.  Every call on one GPU shares that GPU's array, and the   */
/* array keeps the last call's contents (nothing in it has to start at zero): */
/* calls that overlap on one GPU, on any streams, race and must not be made.  */
/* Limits: those of verify_mlp_w4, and verify_mlp_w4_workspace(H, I, G) <=    */
/* EV_MLP_SCRATCH_BYTES (EV_EWORKSPACE otherwise; the MLP slice 5120 <->      */
/* 17408 needs 24.5 MiB).  Errors: EV_EINVAL, EV_EUNSUPPORTED, EV_EWORKSPACE, */
/* EV_EHIP.                                                                   */
/* ------------------------------------------------------------------------- */
#define EV_MLP_SCRATCH_BYTES (32u << 20)
int32_t verify_mlp_w4_noalloc(const uint16_t* x_bf16, int32_t R, int32_t H, int32_t I, int32_t G,
                              const void* gate_packed, const void* up_packed, const void* down_packed,
                              float* y, uint16_t* h_bf16, void* stream);

/* ------------------------------------------------------------------------- */
/* MoE verify layer (top-`top` routing over E experts, SiLU-gated experts).   */
/*                                                                            */
/* The pages' MoE models (TensorFold README model notes; blog "The numbers":  */
/* Nemotron 30B-A3B) verify their drafted rows through this layer; each lane  */
/* (row) is routed on its own and, by the README's exactness paragraph, its   */
/* output must not depend on the other lanes.  Per lane r:                    */
/*   pi = softmax(router[r]);  ids = the `top` experts by pi (lower id on     */
/*   ties);  w_j = pi[ids_j] / sum_j' pi[ids_j'];                             */
/*   y[r] = sum over j = 0..top-1, in that order, of w_j * MLP_{ids_j}(x[r])  */
/* with MLP_e the SiLU-gated MLP of verify_mlp_w4 on expert e's matrices.     */
/*   x_bf16   (device) [R][H] bf16, 16-byte aligned.                          */
/*   router   (device) [R][E] fp32 router logits (finite), 4-byte aligned.    */
/*   w_gate, w_up (device) E packed I x H matrices, expert e at byte offset   */
/*            e * w4_packed_bytes(I, H, G); w_down: E packed H x I matrices,  */
/*            expert e at e * w4_packed_bytes(H, I, G).  16-byte aligned.     */
/*   y        (device) [R][H] fp32, 16-byte aligned, written.                 */
/*   expert_ids, expert_w (device, optional) [R][top] int32 / fp32: if        */
/*            non-NULL, the routing (ids in rank order, renormalised weights).*/
/*   ws       (device) verify_moe_w4_workspace(H, I, E, top, G) bytes,        */
/*            256-byte aligned (a function of the shapes only, never of R).   */
/* Only the experts some lane selects are read (one grouped pass; each        */
/* expert's weights once for all its lanes).  Limits: 1 <= R <= 16;           */
/* 1 <= E <= 256; 1 <= top <= min(8, E); H and I as for verify_linear_w4.     */
/* Errors: EV_EINVAL, EV_EUNSUPPORTED, EV_EWORKSPACE, EV_EHIP.                */
/* ------------------------------------------------------------------------- */
size_t verify_moe_w4_workspace(int32_t H, int32_t I, int32_t E, int32_t top, int32_t G);
int32_t verify_moe_w4(const uint16_t* x_bf16, const float* router, int32_t R, int32_t H,
                      int32_t I, int32_t E, int32_t top, int32_t G, const void* w_gate,
                      const void* w_up, const void* w_down, float* y, int32_t* expert_ids,
                      float* expert_w, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- */
/* Keyed sampler.                                                             */
/*                                                                            */
/* README exactness paragraph / 650 Group: token at position p = argmax over  */
/* the top-k / top-p candidates of l/T + g(seed, p, id).  Readings used here: */
/*   1. candidates: the top_k largest logits under (logit desc, id asc);      */
/*   2. in fp64, e_j = exp((l_j - l_0)/T), Z = sum of e_j in candidate order; */
/*      candidate j is kept while the mass of the candidates before it is     */
/*      < top_p * Z (candidate 0 always kept);                                */
/*   3. noise key: row = mix64(mix64(seed) + (p+1)*gamma),                    */
/*      h = mix64(row + (id+1)*gamma)  (SplitMix64: gamma 0x9E3779B97F4A7C15, */
/*      mix64 its output function); u = ((h >> 12) + 0.5) * 2^-52;           */
/*      g = -log(-log(u)), all fp64;                                          */
/*   4. z = (double)l / (double)T + g; token = argmax z, lower id on ties;    */
/*      gap = best z - second z (+inf with one kept candidate).               */
/* top_k == 0 (with temperature > 0): no top-k; top-p over the whole         */
/* vocabulary, on fixed-point masses that add to the same total in any order: */
/* with the tokens ordered (l desc, id asc), e_j = nearest(exp((l_j - l_0)/T) */
/* * 2^40) (integers), Z = sum e_j, thr = max(1, trunc(top_p * Z)) (fp64      */
/* product); token j is kept while the mass before it is below thr.           */
/* temperature == 0: greedy, token = argmax l (lower id on ties), gap = l(1) - */
/* l(2) on the raw logits (+inf if V == 1); top_k / top_p are ignored.        */
/*                                                                            */
/*   logits     (device) [R][V] fp32, finite (non-finite values: undefined).  */
/*   positions  (device) [R] int64, the absolute position p each row samples. */
/*   tokens     (device) [R] int32, written.                                  */
/*   gap        (device, optional) [R] fp64, written when non-NULL.           */
/*   ws         (device) at least keyed_sample_workspace(V) bytes.            */
/* Limits: 1 <= R <= 16; 1 <= V <= 262144; temperature >= 0 and finite; when */
/* temperature > 0: 0 <= top_k <= 64 and 0 < top_p <= 1.                      */
/* Errors: EV_EINVAL, EV_EUNSUPPORTED (top_k > 64), EV_EWORKSPACE, EV_EHIP.   */
/* ------------------------------------------------------------------------- */
typedef struct {
    double temperature; /* T; 0 selects greedy */
    int32_t top_k;      /* 1..64 when T > 0; 0: no top-k (whole-vocabulary top-p) */
    double top_p;       /* (0, 1] when T > 0  */
    uint64_t seed;      /* key of the noise    */
} ev_sampling;

size_t keyed_sample_workspace(int32_t V);
int32_t keyed_sample(const float* logits, int32_t R, int32_t V, const int64_t* positions,
                     ev_sampling sampling, int32_t* tokens, double* gap,
                     void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- */
/* Accept prefix.                                                             */
/*                                                                            */
/* A draft is accepted exactly when it equals the token serial decoding       */
/* samples at its position (README exactness paragraph; blog FAQ).  Row i's   */
/* sample is compared with draft i:                                           */
/*   n_accept = number of leading i < D with draft[i] == sampled[i];          */
/*   n_commit = min(n_accept + 1, R)   (the accepted drafts' samples plus the */
/*              sample of the first row whose draft differs).                 */
/*   sampled (device) [R] int32; draft (device) [D] int32 (may be NULL if     */
/*   D == 0); n_accept, n_commit (device) [1] int32, written.                 */
/* Limits: 1 <= R <= 16, 0 <= D <= R.  Errors: EV_EINVAL, EV_EHIP.            */
/* ------------------------------------------------------------------------- */
int32_t accept_prefix(const int32_t* sampled, int32_t R, const int32_t* draft, int32_t D,
                      int32_t* n_accept, int32_t* n_commit, void* stream);

/* ------------------------------------------------------------------------- */
/* Verify step of a small decoder (end to end).                               */
/*                                                                            */
/* One verify pass of drafted decoding (TensorFold README, exactness          */
/* paragraph; 650 Group, "TensorFold: the contract is what it does not        */
/* change"): R rows whose inputs are the last committed token and R-1 drafts  */
/* go through the whole model at once; row r's logits, sample and cache entry */
/* are bit-identical to a one-row (serial) step at its position, so a draft   */
/* is accepted exactly when it equals the serial sample.                      */
/*                                                                            */
/* The model: pre-norm decoder layers, each                                   */
/*   n = bf16(RMSNorm(x) * attn_norm);  q|k|v = W_qkv n  (W4, fp32 out);      */
/*   rotate-half RoPE on q and k at the row's position p, angle               */
/*   p * rope_base^(-2i/head_dim) for pair (i, i + head_dim/2);               */
/*   k, v -> fp16 into cache slot p;  query head h reads kv head              */
/*   h / (heads / kv_heads) over slots 0..p: softmax(q.k / sqrt(head_dim)) v; */
/*   x += W_o bf16(attention);  x += MLP(bf16(RMSNorm(x) * mlp_norm)) with    */
/*   the SiLU-gated MLP of verify_mlp_w4;                                     */
/* then logits = W_lm bf16(RMSNorm(x) * final_norm), x = the fp32 residual    */
/* stream starting from the bf16 embedding row of the input token.            */
/* RMSNorm(x) = x / sqrt(mean(x^2) + rms_eps).                                */
/* ------------------------------------------------------------------------- */
typedef struct {
    int32_t layers;        /* >= 1                                           */
    int32_t hidden;        /* H <= 8192                                      */
    int32_t heads;         /* query heads                                    */
    int32_t kv_heads;      /* key/value heads; heads / kv_heads in {1,2,4}   */
    int32_t head_dim;      /* must be 128                                    */
    int32_t intermediate;  /* MLP width I                                    */
    int32_t vocab;         /* V <= 262144                                    */
    int32_t group;         /* W4 group size, 32 or 64                        */
    double rope_base;      /* > 0                                            */
    double rms_eps;        /* >= 0                                           */
} ev_decoder_config;

/* Device pointers of one layer (packed W4 matrices as written by w4_pack),   */
/* all 16-byte aligned.                                                       */
typedef struct {
    const float* attn_norm; /* [H] fp32 gains                                */
    const void* w_qkv;      /* [(heads + 2 kv_heads) * 128][H]: q, k, v rows  */
    const void* w_o;        /* [H][heads * 128]                              */
    const float* mlp_norm;  /* [H] fp32 gains                                */
    const void* w_gate;     /* [I][H]                                        */
    const void* w_up;       /* [I][H]                                        */
    const void* w_down;     /* [H][I]                                        */
} ev_decoder_layer;

typedef struct {
    const uint16_t* embed;          /* (device) [V][H] bf16, 16-byte aligned  */
    const ev_decoder_layer* layers; /* (host) array of `layers` entries,      */
                                    /* copied by toy_decoder_create           */
    const float* final_norm;        /* (device) [H] fp32 gains, 16-B aligned  */
    const void* w_lm;               /* (device) packed [V][H]                 */
} ev_decoder_weights;

typedef struct ev_decoder ev_decoder;

/* Creates a handle over the caller's weights and caches, 16-byte aligned,    */
/* max_ctx a multiple of 32; the handle owns one device table, the (cos, sin) */
/* of every slot's rotation (max_ctx * 512 bytes):                            */
/*   k_cache (device) [layers][kv_heads][max_ctx][128] fp16;                  */
/*   v_cache (device) [layers][kv_heads][max_ctx/32][128][32] fp16: blocks of */
/*           32 slots, d-major, slot s of a block at position                 */
/*           8*floor((s%16)/4) + 4*floor(s/16) + s%4.                         */
/* The handle keeps non-owning pointers: the weights and caches must outlive  */
/* it.  Errors: EV_EINVAL, EV_EUNSUPPORTED, EV_EHIP.                          */
int32_t toy_decoder_create(const ev_decoder_config* cfg, const ev_decoder_weights* w,
                           uint16_t* k_cache, uint16_t* v_cache, int32_t max_ctx,
                           ev_decoder** out);
/* Synchronises the device if the handle holds captured steps, then frees.   */
void toy_decoder_destroy(ev_decoder* m);

/* Workspace of verify_step: a function of the configuration and max_ctx.     */
size_t verify_step_workspace(const ev_decoder* m);

/* One verify pass.                                                           */
/*   tokens   (device) [R] int32: row r's input token, at cache slot pos0 + r */
/*            (tokens[0] = the last committed token, tokens[1..] the drafts); */
/*            values outside [0, V) are undefined.                            */
/*   pos0     slot of tokens[0]; 0 <= pos0 and pos0 + R <= max_ctx.           */
/*   sampling as keyed_sample; row r samples position pos0 + 1 + r.           */
/*   sampled  (device) [R] int32, written: the token sampled after each row.  */
/*   n_commit (device) [1] int32, written: accept_prefix of sampled against   */
/*            the drafts tokens[1..R-1]; commit sampled[0 .. n_commit-1].     */
/*   logits   (device, optional, 16-byte aligned) [R][V] fp32: if non-NULL,   */
/*            the rows' logits are written there.                             */
/* Writes cache slots pos0 .. pos0+R-1 of every layer; slots at and after     */
/* pos0 + n_commit are stale and are rewritten by the next round, which       */
/* starts at pos0 + n_commit with sampled[n_commit-1].  R = 1 is serial       */
/* decoding.  Limits: 1 <= R <= 16.  Errors: EV_EINVAL, EV_EUNSUPPORTED,      */
/* EV_EWORKSPACE, EV_EHIP; nothing is launched on a validation error.         */
/* Launches: a first kernel takes tokens, pos0 and the sampling parameters   */
/* (copied into ws); the rest of the step reads them from ws.  With graphs on */
/* (the default), logits NULL and the timing hook off, that rest is captured  */
/* as a HIP graph on the first call with a given (R, ws, sampled, n_commit)   */
/* and replayed by later calls with the same four, whatever their tokens,     */
/* position, seed, temperature, top_k or top_p (the handle keeps the 16       */
/* latest; dropping one synchronises the device), so a round costs two        */
/* submissions and a new seed never captures.  Results are identical either  */
/* way.  Calls on one handle must not overlap.                                */
int32_t verify_step(ev_decoder* m, const int32_t* tokens, int32_t R, int64_t pos0,
                    ev_sampling sampling, int32_t* sampled, int32_t* n_commit, float* logits,
                    void* ws, size_t ws_bytes, void* stream);

/* verify_step for a host round loop (TensorFold README, exactness paragraph: */
/* the round's rows are the last committed token and the drafts, and the     */
/* reply commits the accepted prefix plus the verifier's token).             */
/*   tokens   (host) [R] int32, read before the call returns: passed to the   */
/*            step's first kernel as an argument (no copy to the device).     */
/*   sampled  (host) [R] int32, written; n_commit (host) [1] int32, written:  */
/*            as for verify_step.                                             */
/* The step runs on `stream` as verify_step does (graph replay included; its  */
/* results sit in ws); one copy brings sampled and n_commit back into pinned  */
/* memory the handle holds, and the call waits for the stream.  Same limits   */
/* and errors as verify_step (no logits); nothing is launched on a           */
/* validation error.  Calls on one handle must not overlap.                  */
int32_t verify_step_host(ev_decoder* m, const int32_t* tokens, int32_t R, int64_t pos0,
                         ev_sampling sampling, int32_t* sampled, int32_t* n_commit, void* ws,
                         size_t ws_bytes, void* stream);

/* Graph replay of verify_step on (enable != 0, the default) or off (every    */
/* step launched kernel by kernel).  Errors: EV_EINVAL (NULL handle).         */
int32_t toy_decoder_set_graphs(ev_decoder* m, int32_t enable);

/* Grid-aligned chunked prefill (650 Group, "Faster, provably the same       */
/* model", section "The regression it published against itself": a prompt is */
/* processed in chunks aligned to a fixed grid of 2,048 tokens and prompt     */
/* caches are kept only at grid points, so that a chunk's bits do not depend  */
/* on where a conversation resumed).  Writes the cache entries of slots       */
/* pos0 .. pos0+n-1 for the input tokens[0..n) (device, int32, values in      */
/* [0, V)), in passes of at most 16 rows that never cross a multiple of 16 or */
/* of grid (a positive multiple of 16); each pass is a verify step's          */
/* embedding and layers without the LM head or sampling.  Every row is        */
/* row-exact, so the entries are bit-identical to those serial decoding       */
/* writes for the same tokens, and a prefill resumed from a cache copied at   */
/* any slot reproduces a fresh one.  The first decoding step after a prompt   */
/* t_0 .. t_{P-1} prefilled up to slot P-2 is verify_step(t_{P-1}, pos0 =     */
/* P-1).  ws: verify_step_workspace(m) bytes.  Errors: EV_EINVAL (slots       */
/* outside the cache, grid, pointers), EV_EWORKSPACE, EV_EHIP.                */
int32_t toy_decoder_prefill(ev_decoder* m, const int32_t* tokens, int32_t n, int64_t pos0, int32_t grid,
                            void* ws, size_t ws_bytes, void* stream);

/* MTP-style draft chain (TensorFold README options table: --mtp-drafts N    */
/* caps the drafts of a round; on CUDA the chain also stops under 30 %        */
/* confidence).  Run after a verify_step on the same stream, with that step's */
/* workspace (step_ws) and its n_commit and sampled outputs (device): from    */
/* the final-normed hidden row h of row n_commit-1 and its sample t, for i =  */
/* 0 .. max_drafts-1:                                                         */
/*   a = bf16(h + embed[t]);  z = W_draft a  (W4, hidden x hidden);           */
/*   h = bf16(RMSNorm(z) * final_norm);  logits = W_lm h;                     */
/*   t = drafts[i] = argmax logits (lower id on ties), with confidence        */
/*   p = 1 / sum_j exp(l_j - l_max);                                          */
/* n_drafts (device, [1]) = the number of leading drafts with p >= min_conf   */
/* (the chain stops at the first one below it).  The next round verifies     */
/* [sampled[n_commit-1], drafts[0 .. n_drafts-1]].  Drafts change how many    */
/* rows are verified, never the committed tokens.                             */
/*   w_draft  (device) packed hidden x hidden W4 matrix (w4_pack), 16-B       */
/*            aligned, group as the decoder's.                                */
/*   drafts   (device) [max_drafts] int32, written up to the stop.            */
/*   ws       (device) toy_decoder_draft_workspace(m) bytes, 256-B aligned.   */
/* Limits: 1 <= max_drafts <= 15, 0 <= min_conf <= 1.  Errors: EV_EINVAL,     */
/* EV_EWORKSPACE, EV_EHIP.                                                    */
size_t toy_decoder_draft_workspace(const ev_decoder* m);
int32_t toy_decoder_draft(ev_decoder* m, const void* w_draft, const int32_t* n_commit, const int32_t* sampled,
                          int32_t max_drafts, double min_conf, int32_t* drafts, int32_t* n_drafts,
                          const void* step_ws, void* ws, size_t ws_bytes, void* stream);

/* How many steps the handle has captured since it was created (captures,    */
/* host, may be NULL) and how many it holds now (cached, host, may be NULL).  */
/* Errors: EV_EINVAL (NULL handle).                                           */
int32_t toy_decoder_graph_stats(const ev_decoder* m, int64_t* captures, int32_t* cached);

/* ------------------------------------------------------------------------- */
/* Exactness probe.                                                           */
/*                                                                            */
/* The TensorFold README's model notes: a model checks at load that drafted   */
/* rows reproduce one-row decoding on the machine it runs on, and drafts only */
/* when they do (otherwise it decodes one token a round: same output,         */
/* slower).  verify_probe is that check on the handle's live shapes: one      */
/* verify_step of R rows (tokens, pos0, sampling as for verify_step), then    */
/* the same R rows as R one-row steps at slots pos0 + r from the same cache,  */
/* and the number of 32-bit words that differ between the two, over the      */
/* rows' logits, their sampled tokens and the cache entries they wrote, is    */
/* written to mismatch.  0: R-row passes are exact here; otherwise the caller */
/* should decode with R = 1.                                                  */
/*   tokens   (device) [R] int32, values in [0, V).                           */
/*   mismatch (device) [1] int32, written.                                    */
/*   ws       (device) verify_probe_workspace(m) bytes, 256-byte aligned.     */
/* Writes cache slots pos0 .. pos0+R-1 like verify_step (the one-row steps    */
/* last): run it where those slots are free, such as just before the round    */
/* that starts at pos0, which rewrites them.  Limits and errors as            */
/* verify_step.                                                               */
/* ------------------------------------------------------------------------- */
size_t verify_probe_workspace(const ev_decoder* m);
int32_t verify_probe(ev_decoder* m, const int32_t* tokens, int32_t R, int64_t pos0,
                     ev_sampling sampling, int32_t* mismatch, void* ws, size_t ws_bytes,
                     void* stream);

/* ------------------------------------------------------------------------- */
/* Measurement hook for the W4 verify kernel (every entry point that streams  */
/* W4 weights launches it).  ev_w4_timing(1) allocates (once) a 16 MiB device */
/* buffer of timing slots; while on, each workgroup of each W4 launch stores  */
/* the device wall clock at its start and at its end in slots of its own, and */
/* the launch's execution interval is its earliest start to its latest end.   */
/* Each launch also adds its algorithmic bytes                                */
/* nmat * (N*K/2 + 4*N*K/G + 2*R*K + 4*R*N).  ev_w4_timing_read synchronises  */
/* the device, returns the number of launches since the last read, their      */
/* summed intervals (ms) and summed algorithmic bytes, and starts afresh.     */
/* Off by default.  Errors: EV_EHIP; EV_EINVAL past 2^20 recorded workgroups  */
/* without a read (that launch is refused).                                   */
/* ------------------------------------------------------------------------- */
int32_t ev_w4_timing(int32_t enable);
int32_t ev_w4_timing_read(int64_t* launches, double* total_ms, double* total_bytes);
/* The raw stamps behind the next ev_w4_timing_read (which it does not reset):*/
/* stamps (host) receives the (start, end) device wall-clock pairs of every   */
/* recorded workgroup, launch after launch in workgroup order; counts (host)  */
/* each launch's workgroup count; *n_launches the number of launches.         */
/* Errors: EV_EINVAL (NULL pointer, or more launches or workgroups than       */
/* max_launches / max_pairs), EV_EHIP.                                        */
int32_t ev_w4_timing_stamps(uint64_t* stamps, int64_t max_pairs, int32_t* counts, int32_t max_launches,
                            int32_t* n_launches);

/* Measurement aid: the practical ceiling of a streaming read on this part,  */
/* next to the nominal HBM peak.  Reads `bytes` at buf (device, 16-byte       */
/* aligned, a multiple of 16) once with a plain grid-stride kernel (1024      */
/* workgroups of 256 threads, 16-byte loads, the whole grid sweeping the      */
/* buffer in 1 KB wave blocks) and writes nothing (sink, device, 4 bytes, is  */
/* written only if the xor of the data equals a constant).  While the timing  */
/* hook is on, the launch is recorded like a W4 launch with `bytes` as its    */
/* bytes.  Errors: EV_EINVAL, EV_EHIP.                                        */
int32_t ev_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EXACTVERIFY_H */
