// Verify step of a small decoder on gfx950: the whole model over the R rows of
// one drafted-decoding round, row-exact end to end.
//
// TensorFold README, exactness paragraph: a row of a multi-row verify pass gets
// the same bits as a one-row step, so drafted decoding commits the bytes serial
// decoding would.  Every kernel below keeps that property by construction:
//   * the W4 linears are the row-exact verify kernel (w4_verify.hip);
//   * norms, RoPE, cache writes and the residual stream are per row, with
//     reductions in a fixed tree that does not depend on R;
//   * attention splits the key slots at absolute boundaries (chunks whose size
//     follows from the cache size, online-softmax steps of 32 slots), so row r
//     at position p sees the same chunks, steps and updates whatever other rows
//     share the pass; a step with no slot <= p leaves the row's state untouched;
//     the chunks are merged in ascending order;
//   * row r writes cache slot p and reads slots <= p only, all of which hold the
//     bytes serial decoding wrote (slot p in this pass, from the same input).
//
// Launches per layer (a kernel boundary costs a few microseconds on this
// chip, more than most of these kernels' work, so the count is kept low):
// W4 q|k|v with RoPE and the fp16 cache write in its epilogue, attention
// partials, chunk merge, W4 o, split sum + residual + RMSNorm, W4 gate|up with
// SiLU * up in its epilogue, W4 down, split sum + residual + RMSNorm (with the
// next layer's gains or the final ones).  Then W4 LM head, split sum, keyed
// sample, accept prefix.  After the first kernel (embedding and norm, which
// takes the call's tokens and position) the step is captured once and
// replayed as a HIP graph.
#include <math.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <vector>

#include "w4_kernel.h"

namespace ev {

constexpr int kHD = 128;          // head dimension
constexpr int kHalf = kHD / 2;
constexpr int kKStep = 32;        // key slots per online-softmax step (absolute boundaries)
constexpr int kMaxChunks = 128;   // attention partials per (row, head) at most
constexpr int kMaxQ = 64;         // queries per kv head: R * heads / kv_heads
constexpr int kPartStride = kHD + 2;  // one attention partial: m, l, acc[128]

// The step's first position sits in the positions array at kPos0Slot (after
// the 16 rows' sampling positions); every kernel after embed_norm reads it
// there, so a captured step can be replayed at any position.

constexpr int kRowThreads = 512;  // threads per row in the row kernels (4 columns each per pass)

// Sum of one value per thread over a kRowThreads block, in a fixed tree.
__device__ __forceinline__ float row_sum(float v, float* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    const int tid = threadIdx.x;
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    float t = red[0];
#pragma unroll
    for (int w = 1; w < kRowThreads / 64; ++w) t += red[w];
    __syncthreads();
    return t;
}

// The gains of the columns the thread owns (4 (tid + kRowThreads j)), loaded
// before the row's own inputs so that the norm does not wait for them.
template <int NV>
__device__ __forceinline__ void gain_load(const float* __restrict__ gain, int H, f32x4 (&gv)[NV]) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = 4 * (threadIdx.x + kRowThreads * j);
        gv[j] = c < H ? *reinterpret_cast<const f32x4*>(gain + c) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// n = bf16(RMSNorm(x) * gain) of one row held as float4s by the block
// (thread tid owns columns 4 (tid + kRowThreads j), gains gv); ss = its sum
// of squares.
template <int NV>
__device__ __forceinline__ void norm_store(const f32x4 (&xv)[NV], const f32x4 (&gv)[NV], float ss, float eps,
                                           int H, uint16_t* __restrict__ nrow, float* red) {
    const float rs = 1.0f / sqrtf(row_sum(ss, red) / (float)H + eps);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = 4 * (threadIdx.x + kRowThreads * j);
        if (c >= H) continue;
        const f32x4 g = gv[j];
        uint32_t w0 = (uint32_t)f32_to_bf16_rne(xv[j][0] * rs * g[0]) | ((uint32_t)f32_to_bf16_rne(xv[j][1] * rs * g[1]) << 16);
        uint32_t w1 = (uint32_t)f32_to_bf16_rne(xv[j][2] * rs * g[2]) | ((uint32_t)f32_to_bf16_rne(xv[j][3] * rs * g[3]) << 16);
        *reinterpret_cast<uint2*>(nrow + c) = make_uint2(w0, w1);
    }
}

constexpr int kMaxRowVec = 4;  // H <= 4 * 4 * kRowThreads = 8192

// x[r] = embedding row of tokens[r] (bf16 -> fp32); n[r] = bf16(RMSNorm(x) *
// gain); positions[r] = pos0 + 1 + r (the positions the rows sample); the
// call's tokens and sampling parameters copied where the rest of the step
// reads them.
// A host round's tokens, passed by value to the first kernel of the step.
struct RowTokens {
    int32_t t[EV_MAX_LANES];
};

__global__ __launch_bounds__(kRowThreads) void embed_norm_kernel(const int* __restrict__ tokens, RowTokens ht,
                                                                 const uint16_t* __restrict__ embed, int H, int V,
                                                                 const float* __restrict__ gain, float eps,
                                                                 float* __restrict__ x, uint16_t* __restrict__ n,
                                                                 long long* __restrict__ positions, long long pos0,
                                                                 int* __restrict__ tok_copy, ev_sampling samp,
                                                                 ev_sampling* __restrict__ samp_copy) {
    __shared__ float red[kRowThreads / 64];
    const int r = blockIdx.x, tid = threadIdx.x;
    int tok = tokens ? tokens[r] : ht.t[r];  // device tokens, or the host round's by value
    if (tid == 0) tok_copy[r] = tok;  // the drafts, where the rest of the step reads them
    tok = tok < 0 ? 0 : (tok >= V ? V - 1 : tok);  // keeps the read inside the table
    const uint16_t* e = embed + (size_t)tok * H;
    f32x4 gv[kMaxRowVec], xv[kMaxRowVec];
    gain_load(gain, H, gv);
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxRowVec; ++j) {
        const int c = 4 * (tid + kRowThreads * j);
        xv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (c >= H) continue;
        const uint2 b = *reinterpret_cast<const uint2*>(e + c);
        const f32x4 v = {bf16_to_f32((uint16_t)(b.x & 0xffffu)), bf16_to_f32((uint16_t)(b.x >> 16)),
                         bf16_to_f32((uint16_t)(b.y & 0xffffu)), bf16_to_f32((uint16_t)(b.y >> 16))};
        xv[j] = v;
        *reinterpret_cast<f32x4*>(x + (size_t)r * H + c) = v;
        ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
    norm_store(xv, gv, ss, eps, H, n + (size_t)r * H, red);
    if (tid == 0) positions[r] = pos0 + 1 + r;
    if (tid == 0 && r == 0) {
        positions[kPos0Slot] = pos0;
        *samp_copy = samp;  // the sampler of the step reads its parameters here
    }
}

// x[r] += the linear's output row r, summed from its partials: split
// partials part[s][r] in ascending s (g.nwg == 0), or balanced segments of
// the column's block in ascending workgroup order; n[r] = bf16(RMSNorm(x[r])
// * gain).
__global__ __launch_bounds__(kRowThreads) void res_norm_kernel(const float* __restrict__ part, int S, SkGeom g,
                                                               int H, float* __restrict__ x,
                                                               const float* __restrict__ gain, float eps,
                                                               uint16_t* __restrict__ n) {
    __shared__ float red[kRowThreads / 64];
    const int r = blockIdx.x, tid = threadIdx.x;
    const size_t stride = (size_t)16 * H;
    f32x4 gv[kMaxRowVec], xv[kMaxRowVec];
    gain_load(gain, H, gv);
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxRowVec; ++j) {
        const int c = 4 * (tid + kRowThreads * j);
        xv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (c >= H) continue;
        const size_t o = (size_t)r * H + c;
        f32x4 lin;
        if (g.nwg > 0) {  // 16 segments' loads in flight at a time, added in order
            const int b = c / kBlockCols, cl = c % kBlockCols;
            const SkSpan sp = sk_span(part, g, b, r, cl);
            lin = *reinterpret_cast<const f32x4*>(sp.p0);
            for (int wb = sp.w0 + 1; wb <= sp.w1; wb += 16) {
                f32x4 p[16];
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    if (wb + u <= sp.w1) p[u] = *reinterpret_cast<const f32x4*>(sk_seg0(part, g, wb + u, r, cl));
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    if (wb + u <= sp.w1) lin += p[u];
            }
        } else {
            lin = *reinterpret_cast<const f32x4*>(part + o);
            for (int s0 = 1; s0 < S; s0 += 8) {  // 8 splits' loads in flight at a time, added in order
                f32x4 p[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (s0 + u < S) p[u] = *reinterpret_cast<const f32x4*>(part + (s0 + u) * stride + o);
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (s0 + u < S) lin += p[u];
            }
        }
        const f32x4 v = *reinterpret_cast<const f32x4*>(x + o) + lin;
        *reinterpret_cast<f32x4*>(x + o) = v;
        xv[j] = v;
        ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
    norm_store(xv, gv, ss, eps, H, n + (size_t)r * H, red);
}

// res_norm_kernel for S (1 or 2) split rows and NV float4s per thread
// (H <= NV * 4 * kRowThreads): the same sums in the same order, with every
// load (gain, residual, split rows) issued before the first is used.
template <int NV, int S>
__global__ __launch_bounds__(kRowThreads) void res_norm_rows_kernel(const float* __restrict__ part, int H,
                                                                    float* __restrict__ x,
                                                                    const float* __restrict__ gain, float eps,
                                                                    uint16_t* __restrict__ n) {
    __shared__ float red[kRowThreads / 64];
    const int r = blockIdx.x, tid = threadIdx.x;
    const size_t stride = (size_t)16 * H;
    f32x4 gv[NV], xv[NV], pv[NV][S];
#pragma unroll
    for (int j = 0; j < NV; ++j) {  // clamped to the row: a column past H reads column H - 4 and is dropped
        const int c = 4 * (tid + kRowThreads * j);
        const size_t o = (size_t)r * H + (c < H ? c : H - 4);
        gv[j] = *reinterpret_cast<const f32x4*>(gain + (c < H ? c : H - 4));
        xv[j] = *reinterpret_cast<const f32x4*>(x + o);
#pragma unroll
        for (int sp = 0; sp < S; ++sp) pv[j][sp] = *reinterpret_cast<const f32x4*>(part + sp * stride + o);
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = 4 * (tid + kRowThreads * j);
        f32x4 lin = pv[j][0];
#pragma unroll
        for (int sp = 1; sp < S; ++sp) lin += pv[j][sp];
        const f32x4 v = xv[j] + lin;
        if (c < H) {
            *reinterpret_cast<f32x4*>(x + (size_t)r * H + c) = v;
            ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
        }
        xv[j] = c < H ? v : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    norm_store(xv, gv, ss, eps, H, n + (size_t)r * H, red);
}

// Value cache layout: blocks of 32 slots, d-major inside a block
// ([kv_heads][C/32][128][32]), and within a block slot s at position
// vslot_pos32(s): positions 8j..8j+7 hold slots 4j..4j+3 and 16+4j..16+4j+3.
// That is the order in which one lane of the PV product's B operand (the
// probabilities, straight out of the score MFMA's accumulator layout) holds
// its 8 slots, so the values' A operand is one 16-byte load.  The q|k|v
// projection writes new slots in this order (its rotation epilogue).

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

struct AttnArgs {
    const float* q;      // [R][NH][128]
    const uint16_t* kc;  // this layer's keys [NKV][C][128] fp16
    const uint16_t* vc;  // this layer's values, blocked (vslot_pos32)
    float* part;         // [16][NH][nchunk_max][130]
    int R, NH, NKV, C, chunk, nchunk_max;
    const long long* positions;  // the step's first position at [kPos0Slot]
    float scale;                 // 1/sqrt(128)
};

// Buffer loads: a per-lane offset past the buffer reads zeros without touching
// memory, so a load that some lanes must skip stays one unconditional
// instruction (a load under a branch makes the compiler wait for it, and for
// everything issued before it, at the branch's end).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kNoLoad = 0x80000000u;  // offset beyond every buffer here
__device__ __forceinline__ rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// With NT the non-temporal hint (the nt bit of the cache-policy operand): the
// cache reads of passes that read each slot once (one tile of queries per kv
// head); with more tiles the other tiles' reads of the same slots find them
// cached.
template <bool NT>
__device__ __forceinline__ u32x4 buf_load128(rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0u, NT ? 2 : 0));
}

// Attention partial of one chunk of slots (blockIdx.x), one kv head
// (blockIdx.y) and one tile of 16 queries (blockIdx.z; query qi = row qi/gq,
// head g*gq + qi%gq), one wave:
//   S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_f16.  Q and P are
//   split into fp16 hi + lo (products exact, fp32 accumulation), Q after a
//   per-query power-of-two scale that keeps it inside the fp16 range; K and V
//   are fp16 already.  The score tile's accumulator layout (slot rows, query
//   columns) is exactly the B operand of the PV product (with the value
//   cache's slot order), so no data moves between the two.
//   Online softmax over steps of 32 slots; lane (grp, ln) keeps the state of
//   query ln (replicated over grp) and O^T rows d = 16 dt + 4 grp + v.
template <bool NT>
__global__ __launch_bounds__(64) void attn_partial_kernel(AttnArgs a) {
    const int lane = threadIdx.x, ln = lane & 15, grp = lane >> 4;
    const int gq = a.NH / a.NKV, nq = a.R * gq;
    const int chunk = blockIdx.x, g = blockIdx.y, qt = blockIdx.z;
    const int qi = qt * 16 + ln;
    const bool qok = qi < nq;
    const int r = qok ? qi / gq : 0;
    const int h = g * gq + (qok ? qi % gq : 0);
    // Q^T fragments: query ln, d = 32 ds + 8 grp + i (loaded before the
    // step's position, which they do not need)
    float qv[4][8];
    const rsrc_t rq = buf_rsrc(a.q, (uint32_t)(a.R * a.NH * kHD) * 4u);
    const uint32_t qo = qok ? (uint32_t)(((r * a.NH + h) * kHD + 8 * grp) * 4) : kNoLoad;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
        const f32x4 v0 = __builtin_bit_cast(f32x4, buf_load128<false>(rq, qo + 128u * ds));
        const f32x4 v1 = __builtin_bit_cast(f32x4, buf_load128<false>(rq, qo + 128u * ds + 16u));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qv[ds][i] = v0[i];
            qv[ds][4 + i] = v1[i];
        }
    }
    const long long pos0 = a.positions[kPos0Slot];
    const long long P = pos0 + r;
    const long long pmax = pos0 + a.R - 1;
    const long long cstart = (long long)chunk * a.chunk;
    if (cstart > pmax) return;  // the grid covers the whole cache; this chunk holds no slot yet
    const long long cend = min(cstart + a.chunk - 1, pmax);

    f16x8 qh[4], ql[4];  // the scaled query, split (set after the first keys are requested)
    float sback = 0.f;
    float m = -INFINITY, l = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    __shared__ f32x4 keep[8][64];  // the workgroup is one wave
    const uint16_t* kb = a.kc + (size_t)g * a.C * kHD;
    const uint16_t* vb = a.vc + (size_t)g * a.C * kHD;

    // K and V of the step at s0 into (kf, vf): keys rows slot = s0 + 16 t + ln,
    // d = 32 ds + 8 grp .. + 7; values V^T rows d = 16 dt + ln, positions
    // 8 grp .. + 7 of block s0 / 32
    // (buffer loads: a step past the chunk (live false) reads zeros, so the
    // loop can request the next step unconditionally)
    const rsrc_t rk = buf_rsrc(kb, (uint32_t)a.C * kHD * 2u);
    const rsrc_t rv = buf_rsrc(vb, (uint32_t)a.C * kHD * 2u);
    auto load_kv = [&](long long s0, f16x8 (&kf)[2][4], f16x8 (&vf)[8], bool live) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const long long slot = s0 + 16 * t + ln;
            const uint32_t ko = live && slot <= pmax ? (uint32_t)(slot * kHD + 8 * grp) * 2u : kNoLoad;  // 0 past the pass
#pragma unroll
            for (int ds = 0; ds < 4; ++ds) kf[t][ds] = __builtin_bit_cast(f16x8, buf_load128<NT>(rk, ko + 64u * ds));
        }
        const uint32_t vo =
            live ? (uint32_t)((s0 / kKStep) * kHD * kKStep + ln * kKStep + 8 * grp) * 2u : kNoLoad;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
            vf[dt] = __builtin_bit_cast(f16x8, buf_load128<NT>(rv, vo + (uint32_t)(16 * dt * kKStep) * 2u));
    };
    // one online-softmax step over the slots s0 .. s0 + 31 from (kf, vf)
    auto step = [&](long long s0, f16x8 (&kf)[2][4], f16x8 (&vf)[8]) {
        if (s0 + kKStep - 1 > pmax) {  // zero the slots past the pass (stale or never written)
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const long long slot = s0 + (kk < 4 ? 4 * grp + kk : 16 + 4 * grp + kk - 4);
                if (slot > pmax)
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) vf[dt][kk] = (_Float16)0.f;
            }
        }
        // scores S^T: lane holds slots s0 + 16 t + 4 grp + v for query ln
        f32x4 sc4[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ds = 0; ds < 4; ++ds) {
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[t][ds], qh[ds], c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[t][ds], ql[ds], c, 0, 0, 0);
            }
            sc4[t] = c;
        }
        const bool live = qok && s0 <= P;  // the query has a slot in this step
        float sv[8], mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const long long slot = s0 + 16 * t + 4 * grp + v;
                const float x = sc4[t][v] * sback;
                sv[4 * t + v] = slot <= P ? x : -INFINITY;
                mx = fmaxf(mx, sv[4 * t + v]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mnew = live ? fmaxf(m, mx) : m;
        const float scl = live ? expf(m - mnew) : 1.f;
        float p[8], ps = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = live ? expf(sv[i] - mnew) : 0.f;
            ps += p[i];
        }
        ps += __shfl_xor(ps, 16, 64);  // a butterfly: every lane gets the same sum
        ps += __shfl_xor(ps, 32, 64);
        if (live) {
            l = l * scl + ps;
            m = mnew;
        }
        f16x8 ph, pl;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const _Float16 hv = (_Float16)p[i];
            ph[i] = hv;
            pl[i] = (_Float16)(p[i] - (float)hv);
        }
        // O^T = O^T * scale + V^T P^T; a query without a slot here keeps its
        // state bit for bit.  Its copy waits in LDS, and only in the steps
        // where some query of the wave has no slot: as 32 more registers it
        // would hold the kernel to one wave per SIMD.
        const bool keep_any = __any(qok && !live);
        if (keep_any) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) keep[dt][lane] = acc[dt];
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            acc[dt] *= scl;
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[dt], ph, acc[dt], 0, 0, 0);
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[dt], pl, acc[dt], 0, 0, 0);
        }
        if (keep_any && !live) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) acc[dt] = keep[dt][lane];
        }
    };
    // The loads of step s + 1 are issued before step s is computed (two
    // register sets, swapped by unrolling), so each step's memory latency
    // hides behind the previous step's arithmetic.
    f16x8 kA[2][4], vA[8], kB[2][4], vB[8];
    long long s0 = cstart;
    load_kv(s0, kA, vA, true);
    // the query's scale and fp16 halves while the first keys and values load
    float amax = 0.f;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(qv[ds][i]));
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    int ex = 0;
    frexpf(amax, &ex);  // amax in [2^(ex-1), 2^ex)
    const int e = amax > 0.f ? max(-100, min(100, 15 - ex)) : 0;
    const float up = ldexpf(1.0f, e);
    sback = ldexpf(1.0f, -e) * a.scale;  // exact: a power of two times the scale
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float v = qv[ds][i] * up;
            const _Float16 hv = (_Float16)v;
            qh[ds][i] = hv;
            ql[ds][i] = (_Float16)(v - (float)hv);
        }

    for (;;) {
        const bool more = s0 + kKStep <= cend;
        load_kv(s0 + kKStep, kB, vB, more);
        step(s0, kA, vA);
        if (!more) break;
        s0 += kKStep;
        const bool more2 = s0 + kKStep <= cend;
        load_kv(s0 + kKStep, kA, vA, more2);
        step(s0, kB, vB);
        if (!more2) break;
        s0 += kKStep;
    }

    if (qok && P >= cstart) {
        float* o = a.part + (((size_t)r * a.NH + h) * a.nchunk_max + chunk) * kPartStride;
        if (grp == 0) {
            o[0] = m;
            o[1] = l;
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int v = 0; v < 4; ++v) o[2 + 16 * dt + 4 * grp + v] = acc[dt][v];
    }
}

// o[r][h][d] = bf16(sum_c acc_c[d] e^(m_c - M) / sum_c l_c e^(m_c - M)) over
// the chunks c = 0 .. nch-1, nch = (pos0 + r) / chunk + 1; M = max_c m_c.
// Four groups of kHD threads each sum a fixed quarter of the chunks (chunk
// order inside a quarter; the quarter's entries loaded up front), and the
// quarters are added in order 0, 1, 2, 3: a fixed order set by the row's own
// position.
constexpr int kMergeGroups = 4;
__global__ __launch_bounds__(kHD * kMergeGroups) void attn_merge_kernel(const float* __restrict__ part, int NH,
                                                                        int chunk, int nchunk_max,
                                                                        const long long* __restrict__ positions,
                                                                        uint16_t* __restrict__ o) {
    const long long pos0 = positions[kPos0Slot];
    __shared__ float sm[kMaxChunks], se[kMaxChunks], sl[kMaxChunks];
    __shared__ float red[kMergeGroups * kHD / 64];
    __shared__ float pacc[kMergeGroups][kHD];
    __shared__ float pl[kMergeGroups];
    const int r = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    const int d = tid % kHD, q = tid / kHD;
    const int nch = (int)((pos0 + r) / chunk) + 1;
    const float* b = part + ((size_t)r * NH + h) * nchunk_max * kPartStride;
    // this thread's accumulator entries (column d of its quarter's chunks),
    // loaded together with the maxima and sums below: one memory round trip
    constexpr int kPerMax = kMaxChunks / kMergeGroups;
    const int per = (nch + kMergeGroups - 1) / kMergeGroups;
    const int lo = q * per, hi = min(nch, lo + per);
    float v[kPerMax];
#pragma unroll
    for (int i = 0; i < kPerMax; ++i) v[i] = lo + i < hi ? b[(size_t)(lo + i) * kPartStride + 2 + d] : 0.f;
    float mv = -INFINITY;
    if (tid < nch) {
        mv = b[(size_t)tid * kPartStride];
        sm[tid] = mv;
        sl[tid] = b[(size_t)tid * kPartStride + 1];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mv = fmaxf(mv, __shfl_xor(mv, off, 64));
    if ((tid & 63) == 0) red[tid >> 6] = mv;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int i = 1; i < kMergeGroups * kHD / 64; ++i) M = fmaxf(M, red[i]);
    if (tid < nch) se[tid] = expf(sm[tid] - M);
    __syncthreads();
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int i = 0; i < kPerMax; ++i)
        if (lo + i < hi) {
            const float e = se[lo + i];
            L = fmaf(sl[lo + i], e, L);
            acc = fmaf(v[i], e, acc);
        }
    pacc[q][d] = acc;
    if (d == 0) pl[q] = L;
    __syncthreads();
    if (q == 0) {
        float Lt = pl[0], at = pacc[0][d];
#pragma unroll
        for (int g = 1; g < kMergeGroups; ++g) {
            Lt += pl[g];
            at += pacc[g][d];
        }
        o[((size_t)r * NH + h) * kHD + d] = f32_to_bf16_rne(at / Lt);
    }
}

// Workspace of a verify step, from the configuration and max_ctx only.
struct StepLayout {
    W4Plan p_qkv, p_o, p_gu, p_down, p_lm;
    SkPlan q_o, q_down, q_lm;  // balanced plans, used where use_sk holds
    bool sk_o, sk_down, sk_lm;
    bool parts_o, parts_down;  // K-parts launches writing kSplitsO / kSplitsDown split rows
    int chunk, nchunk_max;
    bool gu_pair;
    size_t off_x, off_n, off_o, off_q, off_part, off_hres, off_pg, off_pu, off_h, off_att, off_logits, off_pos, off_acc,
        off_sws, off_tok, off_samp, total;
};

}  // namespace ev

using namespace ev;

// A captured step (everything after embed_norm) for one set of baked
// arguments; replayed on the caller's stream.
struct StepGraph {
    int kind;  // 0: a verify step after embed_norm (top-k sampler); 1: a prefill pass's layers;
             // 2: a verify step whose sampler takes top-p over the whole vocabulary
    int R;
    const void* ws;
    int32_t* sampled;
    int32_t* n_commit;
    hipGraphExec_t exec;
};
constexpr size_t kMaxStepGraphs = 16;

struct ev_decoder {
    ev_decoder_config cfg;
    std::vector<ev_decoder_layer> layers;
    const uint16_t* embed;
    const float* final_norm;
    const void* w_lm;
    uint16_t* kc;
    uint16_t* vc;
    int C;
    float2* rot = nullptr;  // [C][64] (cos, sin) of slot p's rotation, fp32 of the fp64 values
    int32_t* hres = nullptr;  // pinned host copy of a host round's results (sampled[16], n_commit)
    int NQKV, DQ;
    StepLayout L;
    bool use_graphs = true;
    std::mutex graph_mu;            // the cache below
    hipStream_t capture = nullptr;  // capture stream, default priority
    std::vector<StepGraph> graphs;
    long long captures = 0;         // steps captured over the handle's life
    ~ev_decoder() {
        if (!graphs.empty()) (void)hipDeviceSynchronize();
        for (StepGraph& g : graphs) (void)hipGraphExecDestroy(g.exec);
        if (capture) (void)hipStreamDestroy(capture);
        if (rot) (void)hipFree(rot);
        if (hres) (void)hipHostFree(hres);
    }
};

// o and down as K-parts launches in these many K-splits (more workgroups,
// each reading less of the activations, for more partial rows per column in
// the row kernel after them).
constexpr int kSplitsO = 1, kSplitsDown = 2;

static StepLayout step_layout(const ev_decoder_config& c, int NQKV, int DQ, int C) {
    StepLayout L;
    const int H = c.hidden, I = c.intermediate, V = c.vocab;
    L.p_qkv = plan_w4_pair(NQKV, H);  // halved launch with the rotation epilogue
    L.p_o = plan_w4(H, DQ, 1);
    // paired gate/up: at the decoder's sizes every kernel boundary costs more
    // than the split launch's extra waves win back
    L.gu_pair = true;
    L.p_gu = L.gu_pair ? plan_w4_pair(I, H) : plan_w4(I, H, 2);
    L.p_down = plan_w4(H, I, 1);
    L.p_lm = plan_w4(V, H, 1);
    L.q_o = plan_w4_sk(H, DQ, 1);
    L.q_down = plan_w4_sk(H, I, 1);
    L.q_lm = plan_w4_sk(V, H, 1);
    L.sk_o = use_sk(L.q_o, L.p_o);
    L.sk_down = use_sk(L.q_down, L.p_down);
    // o and down as K-parts launches (one workgroup per tile, finished rows):
    // the row kernel after them then reads one row instead of the balanced
    // launch's segments
    L.parts_o = parts_fits(DQ, kSplitsO);
    L.parts_down = parts_fits(I, kSplitsDown);
    L.sk_lm = use_sk(L.q_lm, L.p_lm);
    // chunk: a multiple of 64 slots with at most kMaxChunks chunks in the cache
    L.chunk = 64 * ((C + 64 * kMaxChunks - 1) / (64 * kMaxChunks));
    L.nchunk_max = (C + L.chunk - 1) / L.chunk;
    // floats of the largest linear's partials (split rows or balanced segments)
    auto part_floats = [](bool sk, const SkPlan& q, const W4Plan& p, int N) {
        return sk ? sk_part_bytes(q) / sizeof(float) : (size_t)16 * p.S * N;
    };
    size_t part = (size_t)16 * std::max(kSplitsO, kSplitsDown) * H;  // K-parts o and down
    part = std::max(part, part_floats(L.sk_o, L.q_o, L.p_o, H));
    part = std::max(part, part_floats(L.sk_down, L.q_down, L.p_down, H));
    part = std::max(part, part_floats(L.sk_lm, L.q_lm, L.p_lm, V));
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    L.off_x = take(sizeof(float) * 16 * H);
    L.off_n = take(sizeof(uint16_t) * 16 * H);
    L.off_o = take(sizeof(uint16_t) * 16 * DQ);
    L.off_q = take(sizeof(float) * 16 * DQ);
    L.off_part = take(sizeof(float) * part);
    L.off_pg = take(L.gu_pair ? 0 : sizeof(float) * 16 * (size_t)L.p_gu.S * I);
    L.off_pu = take(L.gu_pair ? 0 : sizeof(float) * 16 * (size_t)L.p_gu.S * I);
    L.off_h = take(sizeof(uint16_t) * 16 * I);
    L.off_att = take(sizeof(float) * 16 * (size_t)c.heads * L.nchunk_max * kPartStride);
    L.off_logits = take(sizeof(float) * 16 * (size_t)V);
    L.off_pos = take(sizeof(long long) * (kPos0Slot + 1));
    L.off_acc = take(sizeof(int32_t) * 4);  // n_accept, the sampler's accept count
    L.off_sws = take(keyed_sample_workspace(V));
    L.off_tok = take(sizeof(int32_t) * 16);
    L.off_samp = take(sizeof(ev_sampling));
    L.off_hres = take(sizeof(int32_t) * (EV_MAX_LANES + 1));  // a host round's sampled[16], n_commit
    L.total = off;
    return L;
}

extern "C" int32_t toy_decoder_create(const ev_decoder_config* cfg, const ev_decoder_weights* w, uint16_t* k_cache,
                                      uint16_t* v_cache, int32_t max_ctx, ev_decoder** out) {
    clear_error();
    const char* who = "toy_decoder_create";
    if (!cfg || !w || !out || !w->layers) return fail(EV_EINVAL, "%s: NULL pointer", who);
    *out = nullptr;
    const ev_decoder_config c = *cfg;
    if (c.layers < 1 || c.layers > 1024) return fail(EV_EINVAL, "%s: layers=%d", who, c.layers);
    if (c.head_dim != kHD) return fail(EV_EUNSUPPORTED, "%s: head_dim=%d (128 only)", who, c.head_dim);
    if (c.heads < 1 || c.kv_heads < 1 || c.heads % c.kv_heads != 0)
        return fail(EV_EINVAL, "%s: heads=%d kv_heads=%d", who, c.heads, c.kv_heads);
    if ((c.heads / c.kv_heads) * EV_MAX_LANES > kMaxQ)
        return fail(EV_EUNSUPPORTED, "%s: heads / kv_heads = %d above 4", who, c.heads / c.kv_heads);
    if (c.vocab < 2 || c.vocab > 262144) return fail(EV_EUNSUPPORTED, "%s: vocab=%d (2..262144)", who, c.vocab);
    if (!(c.rope_base > 0.0) || !(c.rope_base < __builtin_huge_val()) || !(c.rms_eps >= 0.0) ||
        !(c.rms_eps < __builtin_huge_val()))
        return fail(EV_EINVAL, "%s: rope_base must be finite > 0 and rms_eps finite >= 0", who);
    if (c.hidden > 4 * kMaxRowVec * kRowThreads)
        return fail(EV_EUNSUPPORTED, "%s: hidden=%d above %d", who, c.hidden, 4 * kMaxRowVec * kRowThreads);
    if (max_ctx < 32 || max_ctx > (1 << 22) || max_ctx % 32 != 0)
        return fail(EV_EINVAL, "%s: max_ctx=%d (a multiple of 32, at most 2^22)", who, max_ctx);
    const int NQKV = (c.heads + 2 * c.kv_heads) * kHD, DQ = c.heads * kHD;
    int32_t rc;
    if ((rc = check_w4_dims(who, c.hidden, NQKV, c.group)) || (rc = check_w4_dims(who, DQ, c.hidden, c.group)) ||
        (rc = check_w4_dims(who, c.hidden, c.intermediate, c.group)) ||
        (rc = check_w4_dims(who, c.intermediate, c.hidden, c.group)) ||
        (rc = check_w4_dims(who, c.hidden, c.vocab, c.group)))
        return rc;
    if (!w->embed || !w->final_norm || !w->w_lm || !k_cache || !v_cache)
        return fail(EV_EINVAL, "%s: NULL pointer", who);
    if (!aligned(w->embed, 16) || !aligned(w->final_norm, 16) || !aligned(w->w_lm, 16) || !aligned(k_cache, 16) ||
        !aligned(v_cache, 16))
        return fail(EV_EINVAL, "%s: misaligned pointer", who);
    for (int l = 0; l < c.layers; ++l) {
        const ev_decoder_layer& y = w->layers[l];
        if (!y.attn_norm || !y.w_qkv || !y.w_o || !y.mlp_norm || !y.w_gate || !y.w_up || !y.w_down)
            return fail(EV_EINVAL, "%s: layer %d: NULL pointer", who, l);
        if (!aligned(y.attn_norm, 16) || !aligned(y.mlp_norm, 16) || !aligned(y.w_qkv, 16) || !aligned(y.w_o, 16) ||
            !aligned(y.w_gate, 16) || !aligned(y.w_up, 16) || !aligned(y.w_down, 16))
            return fail(EV_EINVAL, "%s: layer %d: misaligned pointer", who, l);
    }
    // (cos, sin) of every slot's rotation: angle p * base^(-2i/128) in fp64,
    // rounded to fp32
    std::vector<float2> rot((size_t)max_ctx * kHalf);
    double invf[kHalf];
    for (int i = 0; i < kHalf; ++i) invf[i] = pow(c.rope_base, -2.0 * i / kHD);
    for (int p = 0; p < max_ctx; ++p)
        for (int i = 0; i < kHalf; ++i) {
            const double ang = (double)p * invf[i];
            rot[(size_t)p * kHalf + i] = make_float2((float)cos(ang), (float)sin(ang));
        }
    float2* rot_dev = nullptr;
    if (hipMalloc(&rot_dev, rot.size() * sizeof(float2)) != hipSuccess)
        return fail(EV_EHIP, "%s: hipMalloc of the rotation table failed", who);
    if ((rc = check_hip(hipMemcpy(rot_dev, rot.data(), rot.size() * sizeof(float2), hipMemcpyHostToDevice),
                        "rotation table copy"))) {
        (void)hipFree(rot_dev);
        return rc;
    }
    int32_t* hres = nullptr;
    if (hipHostMalloc(reinterpret_cast<void**>(&hres), sizeof(int32_t) * (EV_MAX_LANES + 1), hipHostMallocDefault) !=
        hipSuccess) {
        (void)hipFree(rot_dev);
        return fail(EV_EHIP, "%s: pinned allocation of the round results failed", who);
    }
    ev_decoder* m = new ev_decoder;
    m->rot = rot_dev;
    m->hres = hres;
    m->cfg = c;
    m->layers.assign(w->layers, w->layers + c.layers);
    m->embed = w->embed;
    m->final_norm = w->final_norm;
    m->w_lm = w->w_lm;
    m->kc = k_cache;
    m->vc = v_cache;
    m->C = max_ctx;
    m->NQKV = NQKV;
    m->DQ = DQ;
    m->L = step_layout(c, NQKV, DQ, max_ctx);
    *out = m;
    return EV_OK;
}

extern "C" void toy_decoder_destroy(ev_decoder* m) { delete m; }

extern "C" size_t verify_step_workspace(const ev_decoder* m) { return m ? m->L.total : 0; }

extern "C" int32_t toy_decoder_set_graphs(ev_decoder* m, int32_t enable) {
    clear_error();
    if (!m) return fail(EV_EINVAL, "toy_decoder_set_graphs: NULL decoder");
    m->use_graphs = enable != 0;
    return EV_OK;
}

// Everything of a verify step after embed_norm, on stream st.  The step's
// position comes from the device (positions[kPos0Slot]) and the drafts from
// embed_norm's copy, so the same launches can be captured once and replayed
// at any position with any tokens.
static int32_t step_body(ev_decoder* m, int R, int32_t* sampled, int32_t* n_commit, float* logits,
                         unsigned char* b, hipStream_t st, bool head = true, bool topp_full = false) {
    int32_t rc;
    const StepLayout& L = m->L;
    const ev_decoder_config& c = m->cfg;
    const int H = c.hidden, I = c.intermediate, V = c.vocab, G = c.group, NH = c.heads, NKV = c.kv_heads;
    const float eps = (float)c.rms_eps;
    float* x = reinterpret_cast<float*>(b + L.off_x);
    uint16_t* n = reinterpret_cast<uint16_t*>(b + L.off_n);
    uint16_t* o = reinterpret_cast<uint16_t*>(b + L.off_o);
    float* q = reinterpret_cast<float*>(b + L.off_q);
    float* part = reinterpret_cast<float*>(b + L.off_part);
    float* pg = reinterpret_cast<float*>(b + L.off_pg);
    float* pu = reinterpret_cast<float*>(b + L.off_pu);
    uint16_t* h = reinterpret_cast<uint16_t*>(b + L.off_h);
    float* att = reinterpret_cast<float*>(b + L.off_att);
    float* lg = logits ? logits : reinterpret_cast<float*>(b + L.off_logits);
    const long long* pos = reinterpret_cast<const long long*>(b + L.off_pos);
    int32_t* n_accept = reinterpret_cast<int32_t*>(b + L.off_acc);
    const int32_t* toks = reinterpret_cast<const int32_t*>(b + L.off_tok);
    void* sws = b + L.off_sws;

    // a linear into the partials at `part`: balanced when sk, else split
    auto linear = [&](const void* wmat, const uint16_t* xin, int K, int N, const W4Plan& p, const SkPlan& q,
                      bool sk, bool parts, int splits = 1) {
        W4Args a{};
        a.w[0] = a.w[1] = reinterpret_cast<const uint8_t*>(wmat);
        a.x = xin;
        a.R = R;
        a.N = N;
        if (parts) {
            a.out[0] = a.out[1] = part;
            return launch_w4_plain_parts(a, K, G, st, splits);
        }
        if (sk) {
            a.sk_part = part;
            return launch_w4_sk(a, 1, q, K, G, st);
        }
        a.out[0] = a.out[1] = part;
        a.split_stride = (long)16 * N;
        return launch_w4(a, 1, p, K, G, st);
    };
    const SkGeom no_sk{0, 0, 0, 0};
    // x += the linear's rows (split rows of a K-parts launch: the specialised
    // kernel; segments or wider splits: the general one), then n = the norm
    auto res_norm = [&](bool parts, int S, const SkGeom& g, const float* gain) {
        const int nv = (H + 4 * kRowThreads - 1) / (4 * kRowThreads);
        if (parts && (S == 1 || S == 2) && nv <= kMaxRowVec) {
            if (S == 1 && nv == 1)
                hipLaunchKernelGGL((res_norm_rows_kernel<1, 1>), dim3(R), dim3(kRowThreads), 0, st, part, H, x,
                                   gain, eps, n);
            else if (nv == 1)
                hipLaunchKernelGGL((res_norm_rows_kernel<1, 2>), dim3(R), dim3(kRowThreads), 0, st, part, H, x,
                                   gain, eps, n);
            else if (S == 1)
                hipLaunchKernelGGL((res_norm_rows_kernel<kMaxRowVec, 1>), dim3(R), dim3(kRowThreads), 0, st, part,
                                   H, x, gain, eps, n);
            else
                hipLaunchKernelGGL((res_norm_rows_kernel<kMaxRowVec, 2>), dim3(R), dim3(kRowThreads), 0, st, part,
                                   H, x, gain, eps, n);
        } else {
            hipLaunchKernelGGL(res_norm_kernel, dim3(R), dim3(kRowThreads), 0, st, part, S, g, H, x, gain, eps, n);
        }
        return check_hip(hipGetLastError(), "res_norm launch");
    };

    const int nqt = (R * (NH / NKV) + 15) / 16;
    for (int l = 0; l < c.layers; ++l) {
        const ev_decoder_layer& y = m->layers[l];
        uint16_t* kcl = m->kc + (size_t)l * NKV * m->C * kHD;
        uint16_t* vcl = m->vc + (size_t)l * NKV * m->C * kHD;
        {  // q|k|v, rotated, straight to the query rows and the caches
            W4Args a{};
            a.w[0] = a.w[1] = reinterpret_cast<const uint8_t*>(y.w_qkv);
            a.x = n;
            a.R = R;
            a.N = m->NQKV;
            a.rope.rot = m->rot;
            a.rope.positions = pos;
            a.rope.q = q;
            a.rope.kc = kcl;
            a.rope.vc = vcl;
            a.rope.C = m->C;
            a.rope.NH = NH;
            a.rope.NKV = NKV;
            if ((rc = launch_w4_rope(a, L.p_qkv, H, G, st))) return rc;
        }
        AttnArgs aa{q, kcl, vcl, att, R, NH, NKV, m->C, L.chunk, L.nchunk_max, pos, 0.08838834764831845f};
        if (nqt == 1)
            hipLaunchKernelGGL(attn_partial_kernel<true>, dim3(L.nchunk_max, NKV, nqt), dim3(64), 0, st, aa);
        else
            hipLaunchKernelGGL(attn_partial_kernel<false>, dim3(L.nchunk_max, NKV, nqt), dim3(64), 0, st, aa);
        if ((rc = check_hip(hipGetLastError(), "attn_partial launch"))) return rc;
        hipLaunchKernelGGL(attn_merge_kernel, dim3(R, NH), dim3(kHD * kMergeGroups), 0, st, att, NH, L.chunk,
                           L.nchunk_max, pos, o);
        if ((rc = check_hip(hipGetLastError(), "attn_merge launch"))) return rc;
        if ((rc = linear(y.w_o, o, m->DQ, H, L.p_o, L.q_o, L.sk_o, L.parts_o, kSplitsO))) return rc;
        if ((rc = res_norm(L.parts_o, L.parts_o ? kSplitsO : L.p_o.S, L.sk_o && !L.parts_o ? sk_geom(L.q_o) : no_sk,
                           y.mlp_norm)))
            return rc;
        {  // h = SiLU(gate) * up: one paired launch, or gate|up + split sum with SiLU * up
            W4Args a{};
            a.w[0] = reinterpret_cast<const uint8_t*>(y.w_gate);
            a.w[1] = reinterpret_cast<const uint8_t*>(y.w_up);
            a.x = n;
            a.R = R;
            a.N = I;
            if (L.gu_pair) {
                a.h = h;
                if ((rc = launch_w4_pair(a, L.p_gu, H, G, st))) return rc;
            } else {
                a.out[0] = pg;
                a.out[1] = pu;
                a.split_stride = (long)16 * I;
                if ((rc = launch_w4(a, 2, L.p_gu, H, G, st))) return rc;
                if ((rc = launch_silu_reduce(pg, pu, L.p_gu.S, I, R, h, nullptr, 1, nullptr, nullptr, 0, 0, st)))
                    return rc;
            }
        }
        if ((rc = linear(y.w_down, h, I, H, L.p_down, L.q_down, L.sk_down, L.parts_down, kSplitsDown))) return rc;
        const float* next = l + 1 < c.layers ? m->layers[l + 1].attn_norm : m->final_norm;
        if ((rc = res_norm(L.parts_down, L.parts_down ? kSplitsDown : L.p_down.S,
                           L.sk_down && !L.parts_down ? sk_geom(L.q_down) : no_sk, next)))
            return rc;
    }
    if (!head) return EV_OK;  // prefill: the layers only (their cache entries)
    if ((rc = linear(m->w_lm, n, H, V, L.p_lm, L.q_lm, L.sk_lm, false))) return rc;
    if (L.sk_lm) {
        if ((rc = launch_sk_reduce(part, L.q_lm, 1, V, R, lg, nullptr, nullptr, st))) return rc;
    } else if ((rc = launch_splitk_reduce(part, L.p_lm.S, V, R, lg, st))) {
        return rc;
    }
    // the sampling parameters come from the workspace (written by embed_norm);
    // the host value only picks the launch sequence (top-k candidates, or top-p
    // over the whole vocabulary) and is never read by the kernels
    const ev_sampling any{1.0, topp_full ? 0 : EV_MAX_TOPK, 1.0, 0};
    // the accept prefix against the drafts (the step's tokens 1..R-1) by the
    // sampler's last workgroup; its count sits in the word after n_accept
    const FusedAccept acc{n_accept + 1, R > 1 ? toks + 1 : nullptr, R - 1, n_accept, n_commit};
    return launch_keyed_sample(lg, R, V, pos, any, reinterpret_cast<const ev_sampling*>(b + L.off_samp), sampled,
                               nullptr, sws, st, &acc);
}

// The captured step for these arguments: found in the cache, or captured on
// the decoder's own stream (nothing runs during capture) and kept.
static int32_t step_graph(ev_decoder* m, int R, int32_t* sampled, int32_t* n_commit, void* ws,
                          hipGraphExec_t* out, int kind = 0) {
    for (const StepGraph& g : m->graphs)
        if (g.kind == kind && g.R == R && g.ws == ws && g.sampled == sampled && g.n_commit == n_commit) {
            *out = g.exec;
            return EV_OK;
        }
    int32_t rc;
    if (!m->capture && (rc = check_hip(hipStreamCreateWithFlags(&m->capture, hipStreamNonBlocking), "capture stream")))
        return rc;
    if ((rc = check_hip(hipStreamBeginCapture(m->capture, hipStreamCaptureModeThreadLocal), "begin capture")))
        return rc;
    rc = step_body(m, R, sampled, n_commit, nullptr, reinterpret_cast<unsigned char*>(ws), m->capture, kind != 1,
                   kind == 2);
    hipGraph_t graph = nullptr;
    const hipError_t end = hipStreamEndCapture(m->capture, &graph);
    if (!rc) rc = check_hip(end, "end capture");
    hipGraphExec_t exec = nullptr;
    if (!rc) rc = check_hip(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0), "graph instantiate");
    if (graph) (void)hipGraphDestroy(graph);
    if (rc) return rc;
    if (m->graphs.size() >= kMaxStepGraphs) {  // the oldest goes; it may still be queued on some stream
        if ((rc = check_hip(hipDeviceSynchronize(), "graph eviction"))) {
            (void)hipGraphExecDestroy(exec);
            return rc;
        }
        (void)hipGraphExecDestroy(m->graphs.front().exec);
        m->graphs.erase(m->graphs.begin());
    }
    m->graphs.push_back(StepGraph{kind, R, ws, sampled, n_commit, exec});
    ++m->captures;
    *out = exec;
    return EV_OK;
}

// The step's launches after validation: tokens from device memory, or (tokens
// NULL) the host round's by value.
static int32_t step_launch(ev_decoder* m, const int32_t* tokens, const RowTokens& ht, int32_t R, int64_t pos0,
                           ev_sampling sampling, int32_t* sampled, int32_t* n_commit, float* logits, void* ws,
                           hipStream_t st) {
    int32_t rc;
    const StepLayout& L = m->L;
    const ev_decoder_config& c = m->cfg;
    unsigned char* b = reinterpret_cast<unsigned char*>(ws);
    // the step's per-call inputs: rows' tokens and positions, on the device
    hipLaunchKernelGGL(embed_norm_kernel, dim3(R), dim3(kRowThreads), 0, st, tokens, ht, m->embed, c.hidden,
                       c.vocab, m->layers[0].attn_norm, (float)c.rms_eps, reinterpret_cast<float*>(b + L.off_x),
                       reinterpret_cast<uint16_t*>(b + L.off_n), reinterpret_cast<long long*>(b + L.off_pos),
                       (long long)pos0, reinterpret_cast<int*>(b + L.off_tok), sampling,
                       reinterpret_cast<ev_sampling*>(b + L.off_samp));
    if ((rc = check_hip(hipGetLastError(), "embed_norm launch"))) return rc;
    const bool topp_full = sampling.temperature > 0.0 && sampling.top_k == 0;
    // the rest: one graph launch when the step can be replayed as captured
    // (no logits asked for, no per-launch measurement), else launch by launch
    if (m->use_graphs && !logits && !w4_timing_active()) {
        std::lock_guard<std::mutex> lk(m->graph_mu);
        hipGraphExec_t exec;
        if ((rc = step_graph(m, R, sampled, n_commit, ws, &exec, topp_full ? 2 : 0))) return rc;
        return check_hip(hipGraphLaunch(exec, st), "step graph launch");
    }
    return step_body(m, R, sampled, n_commit, logits, b, st, true, topp_full);
}

// Checks shared by verify_step and verify_step_host.
static int32_t check_step(const char* who, ev_decoder* m, int32_t R, int64_t pos0, ev_sampling sampling, void* ws,
                          size_t ws_bytes) {
    int32_t rc;
    if ((rc = check_lanes(who, R))) return rc;
    if (pos0 < 0 || pos0 + R > m->C)
        return fail(EV_EINVAL, "%s: slots %lld..%lld outside the cache of %d", who, (long long)pos0,
                    (long long)pos0 + R - 1, m->C);
    if ((rc = check_sampling(who, sampling))) return rc;
    return check_ws(who, ws, ws_bytes, m->L.total);
}

extern "C" int32_t verify_step(ev_decoder* m, const int32_t* tokens, int32_t R, int64_t pos0, ev_sampling sampling,
                               int32_t* sampled, int32_t* n_commit, float* logits, void* ws, size_t ws_bytes,
                               void* stream) {
    clear_error();
    const char* who = "verify_step";
    int32_t rc;
    if (!m) return fail(EV_EINVAL, "%s: NULL decoder", who);
    if (!tokens || !sampled || !n_commit) return fail(EV_EINVAL, "%s: NULL pointer", who);
    if (!aligned(tokens, 4) || !aligned(sampled, 4) || !aligned(n_commit, 4) || (logits && !aligned(logits, 16)))
        return fail(EV_EINVAL, "%s: misaligned pointer", who);
    if ((rc = check_step(who, m, R, pos0, sampling, ws, ws_bytes))) return rc;
    return step_launch(m, tokens, RowTokens{}, R, pos0, sampling, sampled, n_commit, logits, ws,
                       reinterpret_cast<hipStream_t>(stream));
}

extern "C" int32_t verify_step_host(ev_decoder* m, const int32_t* tokens, int32_t R, int64_t pos0,
                                    ev_sampling sampling, int32_t* sampled, int32_t* n_commit, void* ws,
                                    size_t ws_bytes, void* stream) {
    clear_error();
    const char* who = "verify_step_host";
    int32_t rc;
    if (!m) return fail(EV_EINVAL, "%s: NULL decoder", who);
    if (!tokens || !sampled || !n_commit) return fail(EV_EINVAL, "%s: NULL pointer", who);
    if ((rc = check_step(who, m, R, pos0, sampling, ws, ws_bytes))) return rc;
    RowTokens ht{};
    std::memcpy(ht.t, tokens, sizeof(int32_t) * (size_t)R);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // the results at a fixed place in ws (so that the captured step is the
    // same for every host round with this R and ws), one copy back
    int32_t* dres = reinterpret_cast<int32_t*>(reinterpret_cast<unsigned char*>(ws) + m->L.off_hres);
    if ((rc = step_launch(m, nullptr, ht, R, pos0, sampling, dres, dres + EV_MAX_LANES, nullptr, ws, st))) return rc;
    if ((rc = check_hip(hipMemcpyAsync(m->hres, dres, sizeof(int32_t) * (EV_MAX_LANES + 1), hipMemcpyDeviceToHost,
                                       st),
                        "round results copy")))
        return rc;
    if ((rc = check_hip(hipStreamSynchronize(st), "round synchronise"))) return rc;
    std::memcpy(sampled, m->hres, sizeof(int32_t) * (size_t)R);
    *n_commit = m->hres[EV_MAX_LANES];
    return EV_OK;
}

// Grid-aligned chunked prefill (650 Group, "Faster, provably the same model",
// "The regression it published against itself": prompts processed in chunks
// aligned to a fixed grid of 2,048 tokens, caches kept only at grid points, so
// that a chunk's bits do not depend on where a conversation resumed).  The
// inputs tokens[0..n) go to slots pos0 .. pos0+n-1 in passes of at most 16
// rows that never cross a multiple of 16 or of `grid`, so a pass's rows are a
// function of the absolute slots alone; each pass is the verify step's
// embedding and layers (no LM head, no sampling), replayed from a captured
// graph per row count.
extern "C" int32_t toy_decoder_prefill(ev_decoder* m, const int32_t* tokens, int32_t n, int64_t pos0, int32_t grid,
                                       void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    const char* who = "toy_decoder_prefill";
    int32_t rc;
    if (!m) return fail(EV_EINVAL, "%s: NULL decoder", who);
    if (n < 0 || (n > 0 && !tokens)) return fail(EV_EINVAL, "%s: n=%d or NULL tokens", who, n);
    if (n > 0 && !aligned(tokens, 4)) return fail(EV_EINVAL, "%s: misaligned tokens", who);
    if (grid < 16 || grid % 16 != 0) return fail(EV_EINVAL, "%s: grid=%d (a positive multiple of 16)", who, grid);
    if (pos0 < 0 || pos0 + n > m->C)
        return fail(EV_EINVAL, "%s: slots %lld..%lld outside the cache of %d", who, (long long)pos0,
                    (long long)pos0 + n - 1, m->C);
    const StepLayout& L = m->L;
    if ((rc = check_ws(who, ws, ws_bytes, L.total))) return rc;
    const ev_decoder_config& c = m->cfg;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    unsigned char* b = reinterpret_cast<unsigned char*>(ws);
    const ev_sampling none{0.0, 1, 1.0, 0};
    for (long long p = pos0; p < pos0 + n;) {
        long long e = (p / 16 + 1) * 16;
        const long long g = (p / grid + 1) * grid;
        if (g < e) e = g;
        if (pos0 + n < e) e = pos0 + n;
        const int R = (int)(e - p);
        hipLaunchKernelGGL(embed_norm_kernel, dim3(R), dim3(kRowThreads), 0, st, tokens + (p - pos0), RowTokens{},
                           m->embed,
                           c.hidden, c.vocab, m->layers[0].attn_norm, (float)c.rms_eps,
                           reinterpret_cast<float*>(b + L.off_x), reinterpret_cast<uint16_t*>(b + L.off_n),
                           reinterpret_cast<long long*>(b + L.off_pos), p, reinterpret_cast<int*>(b + L.off_tok),
                           none, reinterpret_cast<ev_sampling*>(b + L.off_samp));
        if ((rc = check_hip(hipGetLastError(), "embed_norm launch"))) return rc;
        if (m->use_graphs && !w4_timing_active()) {
            std::lock_guard<std::mutex> lk(m->graph_mu);
            hipGraphExec_t exec;
            if ((rc = step_graph(m, R, nullptr, nullptr, ws, &exec, 1))) return rc;
            if ((rc = check_hip(hipGraphLaunch(exec, st), "prefill graph launch"))) return rc;
        } else if ((rc = step_body(m, R, nullptr, nullptr, nullptr, b, st, false))) {
            return rc;
        }
        p = e;
    }
    return EV_OK;
}

extern "C" int32_t toy_decoder_graph_stats(const ev_decoder* m, int64_t* captures, int32_t* cached) {
    clear_error();
    if (!m) return fail(EV_EINVAL, "toy_decoder_graph_stats: NULL decoder");
    std::lock_guard<std::mutex> lk(const_cast<ev_decoder*>(m)->graph_mu);
    if (captures) *captures = m->captures;
    if (cached) *cached = (int32_t)m->graphs.size();
    return EV_OK;
}

// ---- exactness probe --------------------------------------------------------
// The TensorFold README's model notes: a model checks at load that drafted
// rows reproduce one-row decoding on the machine it runs on, and drafts only
// when they do.  verify_probe runs that check on the handle's live shapes: one
// R-row verify step, then the same R rows as R one-row steps, and counts the
// 32-bit words of logits, sampled tokens and written cache entries that differ.

namespace ev {
namespace {

// Probe workspace after the step's own: two logits areas [16][V] fp32, two
// sampled areas [16] int32, a commit slot, two cache copies and the count.
struct ProbeLayout {
    size_t off_la, off_lb, off_sa, off_sb, off_nc, off_ka, off_kb, off_cnt, total;
    size_t kv_words;  // 32-bit words of one cache copy
};

// Words of one cache copy: per (layer, kv head), 16 key slots of 128 fp16 and
// the two 32-slot value blocks that can hold 16 consecutive slots.
inline size_t probe_kv_words(const ev_decoder_config& c) {
    return (size_t)c.layers * c.kv_heads * (16 * kHD + 2 * 32 * kHD) / 2;
}

ProbeLayout probe_layout(const ev_decoder_config& c, size_t step_total) {
    ProbeLayout P;
    size_t off = step_total;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    P.kv_words = probe_kv_words(c);
    P.off_la = take(sizeof(float) * 16 * (size_t)c.vocab);
    P.off_lb = take(sizeof(float) * 16 * (size_t)c.vocab);
    P.off_sa = take(sizeof(int32_t) * 16);
    P.off_sb = take(sizeof(int32_t) * 16);
    P.off_nc = take(sizeof(int32_t) * 4);
    P.off_ka = take(sizeof(uint32_t) * P.kv_words);
    P.off_kb = take(sizeof(uint32_t) * P.kv_words);
    P.off_cnt = take(sizeof(int32_t) * 4);
    P.total = off;
    return P;
}

}  // namespace

// Copies the cache entries of slots pos0 .. pos0 + R - 1 of every layer and kv
// head: the R key slots, and the one or two value blocks that hold them (in
// full; their other slots are written by neither pass).  Grid (layers,
// kv_heads), 256 threads.  The rest of each head's area (keys past R slots, a
// second value block that is not needed) is written as zeros, so that two
// copies compare equal exactly when the entries do.
__global__ __launch_bounds__(256) void probe_save_kernel(const uint16_t* __restrict__ kc,
                                                          const uint16_t* __restrict__ vc, int C, long long pos0,
                                                          int R, uint32_t* __restrict__ out) {
    const int l = blockIdx.x, g = blockIdx.y, NKV = gridDim.y;
    const size_t head = ((size_t)l * NKV + g) * (size_t)C * kHD;
    uint32_t* o = out + ((size_t)l * NKV + g) * (16 * kHD + 2 * 32 * kHD) / 2;
    const uint32_t* k = reinterpret_cast<const uint32_t*>(kc + head + (size_t)pos0 * kHD);
    const int kw = R * kHD / 2;
    for (int i = threadIdx.x; i < 16 * kHD / 2; i += 256) o[i] = i < kw ? k[i] : 0u;
    const long long b0 = pos0 / 32, b1 = (pos0 + R - 1) / 32;
    const uint32_t* v = reinterpret_cast<const uint32_t*>(vc + head + (size_t)b0 * 32 * kHD);
    const int vw = (int)(b1 - b0 + 1) * 32 * kHD / 2;
    for (int i = threadIdx.x; i < 2 * 32 * kHD / 2; i += 256) o[16 * kHD / 2 + i] = i < vw ? v[i] : 0u;
}

// cnt[0] += the number of positions i < n where a[i] != b[i] (words).
__global__ __launch_bounds__(256) void probe_compare_kernel(const uint32_t* __restrict__ a,
                                                             const uint32_t* __restrict__ b, long n,
                                                             int* __restrict__ cnt) {
    int d = 0;
    for (long i = blockIdx.x * 256l + threadIdx.x; i < n; i += (long)gridDim.x * 256)
        d += a[i] != b[i];
    // one atomic per wave (a vector atomic on global memory)
    for (int off = 32; off >= 1; off >>= 1) d += __shfl_xor(d, off, 64);
    if ((threadIdx.x & 63) == 0 && d) atomicAdd(cnt, d);
}

__global__ void probe_clear_kernel(int* __restrict__ cnt) {
    if (threadIdx.x == 0) cnt[0] = 0;
}

__global__ void probe_result_kernel(const int* __restrict__ cnt, int32_t* __restrict__ mismatch) {
    if (threadIdx.x == 0) mismatch[0] = cnt[0];
}

}  // namespace ev

extern "C" size_t verify_probe_workspace(const ev_decoder* m) {
    return m ? probe_layout(m->cfg, m->L.total).total : 0;
}

extern "C" int32_t verify_probe(ev_decoder* m, const int32_t* tokens, int32_t R, int64_t pos0,
                                ev_sampling sampling, int32_t* mismatch, void* ws, size_t ws_bytes,
                                void* stream) {
    clear_error();
    const char* who = "verify_probe";
    int32_t rc;
    if (!m) return fail(EV_EINVAL, "%s: NULL decoder", who);
    if ((rc = check_lanes(who, R))) return rc;
    if (!tokens || !mismatch) return fail(EV_EINVAL, "%s: NULL pointer", who);
    if (!aligned(tokens, 4) || !aligned(mismatch, 4)) return fail(EV_EINVAL, "%s: misaligned pointer", who);
    if (pos0 < 0 || pos0 + R > m->C)
        return fail(EV_EINVAL, "%s: slots %lld..%lld outside the cache of %d", who, (long long)pos0,
                    (long long)pos0 + R - 1, m->C);
    if ((rc = check_sampling(who, sampling))) return rc;
    const ProbeLayout P = probe_layout(m->cfg, m->L.total);
    if ((rc = check_ws(who, ws, ws_bytes, P.total))) return rc;
    const ev_decoder_config& c = m->cfg;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    unsigned char* b = reinterpret_cast<unsigned char*>(ws);
    const size_t V = (size_t)c.vocab;
    float* la = reinterpret_cast<float*>(b + P.off_la);
    float* lb = reinterpret_cast<float*>(b + P.off_lb);
    int32_t* sa = reinterpret_cast<int32_t*>(b + P.off_sa);
    int32_t* sb = reinterpret_cast<int32_t*>(b + P.off_sb);
    int32_t* nc = reinterpret_cast<int32_t*>(b + P.off_nc);
    uint32_t* ka = reinterpret_cast<uint32_t*>(b + P.off_ka);
    uint32_t* kb = reinterpret_cast<uint32_t*>(b + P.off_kb);
    int* cnt = reinterpret_cast<int*>(b + P.off_cnt);
    const dim3 kvgrid((unsigned)c.layers, (unsigned)c.kv_heads);
    // the R-row pass (eager: logits are asked for), its cache entries saved
    if ((rc = verify_step(m, tokens, R, pos0, sampling, sa, nc, la, ws, m->L.total, stream))) return rc;
    hipLaunchKernelGGL(probe_save_kernel, kvgrid, dim3(256), 0, st, m->kc, m->vc, m->C, (long long)pos0, R, ka);
    if ((rc = check_hip(hipGetLastError(), "probe save launch"))) return rc;
    // the same rows one at a time, from the same cache
    for (int r = 0; r < R; ++r)
        if ((rc = verify_step(m, tokens + r, 1, pos0 + r, sampling, sb + r, nc, lb + (size_t)r * V, ws, m->L.total,
                              stream)))
            return rc;
    hipLaunchKernelGGL(probe_save_kernel, kvgrid, dim3(256), 0, st, m->kc, m->vc, m->C, (long long)pos0, R, kb);
    hipLaunchKernelGGL(probe_clear_kernel, dim3(1), dim3(64), 0, st, cnt);
    const long nl = (long)R * (long)V;
    hipLaunchKernelGGL(probe_compare_kernel, dim3(256), dim3(256), 0, st, reinterpret_cast<const uint32_t*>(la),
                       reinterpret_cast<const uint32_t*>(lb), nl, cnt);
    hipLaunchKernelGGL(probe_compare_kernel, dim3(1), dim3(256), 0, st, reinterpret_cast<const uint32_t*>(sa),
                       reinterpret_cast<const uint32_t*>(sb), (long)R, cnt);
    hipLaunchKernelGGL(probe_compare_kernel, dim3(64), dim3(256), 0, st, ka, kb, (long)P.kv_words, cnt);
    hipLaunchKernelGGL(probe_result_kernel, dim3(1), dim3(64), 0, st, cnt, mismatch);
    return check_hip(hipGetLastError(), "probe compare launch");
}

// ---- MTP-style draft chain ----------------------------------------------------
// The TensorFold README's options table: --mtp-drafts N caps the drafts a
// round (3, or 6 on CUDA), and on CUDA the chain also stops under 30 %
// confidence.  The head here is the simplest multi-token-prediction head on
// the decoder's own parts: from the final-normed hidden row h of the last
// committed token t,
//   a = bf16(h + embed[t]);  z = W_draft a  (W4, H -> H);
//   h' = bf16(RMSNorm(z) * final_norm);  logits = W_lm h'  (the shared head);
//   draft = argmax logits (lower id on ties), confidence = its softmax
//   probability 1 / sum_j exp(l_j - l_max);
// then again from (h', draft).  Drafts only change how many rows a round
// verifies, never what is committed.

namespace ev {
namespace {

struct DraftLayout {
    size_t off_a, off_z, off_h, off_logits, off_state, off_lin, total;
};

DraftLayout draft_layout(const ev_decoder_config& c) {
    DraftLayout D;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    D.off_a = take(sizeof(uint16_t) * (size_t)c.hidden);
    D.off_z = take(sizeof(float) * (size_t)c.hidden);
    D.off_h = take(sizeof(uint16_t) * (size_t)c.hidden);
    D.off_logits = take(sizeof(float) * (size_t)c.vocab);
    D.off_state = take(sizeof(int32_t) * 4);
    D.off_lin = take(std::max(verify_linear_w4_workspace(c.hidden, c.hidden, c.group),
                              verify_linear_w4_workspace(c.hidden, c.vocab, c.group)));
    D.total = off;
    return D;
}

}  // namespace

// state[0] = 1 once the chain has stopped; n_drafts = 0.
__global__ void draft_init_kernel(int32_t* __restrict__ state, int32_t* __restrict__ n_drafts) {
    if (threadIdx.x == 0) {
        state[0] = 0;
        n_drafts[0] = 0;
    }
}

// a = bf16(h + embed[t]), one row: draft 0 starts from the verify step's row
// n_commit - 1 (its final-normed hidden and its sample), later drafts from the
// previous draft's h' and token.
__global__ __launch_bounds__(kRowThreads) void draft_input_kernel(
    const uint16_t* __restrict__ nrows, const int32_t* __restrict__ n_commit, const int32_t* __restrict__ sampled,
    const uint16_t* __restrict__ h_prev, const int32_t* __restrict__ drafts, int i, const uint16_t* __restrict__ embed,
    int H, int V, const int32_t* __restrict__ state, uint16_t* __restrict__ a) {
    if (state[0]) return;  // the chain has stopped: nothing of this draft is used
    const int nc = n_commit[0];
    const uint16_t* h = i == 0 ? nrows + (size_t)(nc - 1) * H : h_prev;
    int t = i == 0 ? sampled[nc - 1] : drafts[i - 1];
    t = t < 0 ? 0 : (t >= V ? V - 1 : t);
    const uint16_t* e = embed + (size_t)t * H;
    for (int c = threadIdx.x; c < H; c += kRowThreads) a[c] = f32_to_bf16_rne(bf16_to_f32(h[c]) + bf16_to_f32(e[c]));
}

// h' = bf16(RMSNorm(z) * gain), one row.
__global__ __launch_bounds__(kRowThreads) void draft_norm_kernel(const float* __restrict__ z, int H,
                                                                 const float* __restrict__ gain, float eps,
                                                                 const int32_t* __restrict__ state,
                                                                 uint16_t* __restrict__ h) {
    __shared__ float red[kRowThreads / 64];
    if (state[0]) return;
    f32x4 gv[kMaxRowVec], xv[kMaxRowVec];
    gain_load(gain, H, gv);
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxRowVec; ++j) {
        const int c = 4 * (threadIdx.x + kRowThreads * j);
        xv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (c >= H) continue;
        xv[j] = *reinterpret_cast<const f32x4*>(z + c);
        ss += xv[j][0] * xv[j][0] + xv[j][1] * xv[j][1] + xv[j][2] * xv[j][2] + xv[j][3] * xv[j][3];
    }
    norm_store(xv, gv, ss, eps, H, h, red);
}

// drafts[i] = argmax of the logits row (lower id on ties); its confidence p =
// 1 / sum_j exp(l_j - l_max), summed in a fixed order.  The chain keeps the
// draft while p >= min_conf and stops at the first draft below it.
__global__ __launch_bounds__(1024) void draft_pick_kernel(const float* __restrict__ logits, int V, int i,
                                                          float min_conf, int32_t* __restrict__ state,
                                                          int32_t* __restrict__ drafts,
                                                          int32_t* __restrict__ n_drafts) {
    __shared__ unsigned long long kred[16];
    __shared__ float fred[16];
    if (state[0]) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    unsigned long long best = 0ull;
    for (int j = tid; j < V; j += 1024) {
        const unsigned long long k = order_key(logits[j], j);
        best = k > best ? k : best;
    }
    best = wave_max_u64(best);
    if (lane == 0) kred[w] = best;
    __syncthreads();
    unsigned long long top = kred[0];
    for (int u = 1; u < 16; ++u) top = kred[u] > top ? kred[u] : top;
    const float lmax = key_logit(top);
    float sum = 0.f;  // each thread in ascending j, then the waves' sums in a fixed tree
    for (int j = tid; j < V; j += 1024) sum += expf(logits[j] - lmax);
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (lane == 0) fred[w] = sum;
    __syncthreads();
    if (tid == 0) {
        float z = 0.f;
        for (int u = 0; u < 16; ++u) z += fred[u];
        const float p = 1.0f / z;
        drafts[i] = key_id(top);
        if (p >= min_conf)
            n_drafts[0] = i + 1;
        else
            state[0] = 1;
    }
}

}  // namespace ev

extern "C" size_t toy_decoder_draft_workspace(const ev_decoder* m) { return m ? draft_layout(m->cfg).total : 0; }

extern "C" int32_t toy_decoder_draft(ev_decoder* m, const void* w_draft, const int32_t* n_commit,
                                     const int32_t* sampled, int32_t max_drafts, double min_conf, int32_t* drafts,
                                     int32_t* n_drafts, const void* step_ws, void* ws, size_t ws_bytes,
                                     void* stream) {
    clear_error();
    const char* who = "toy_decoder_draft";
    int32_t rc;
    if (!m) return fail(EV_EINVAL, "%s: NULL decoder", who);
    if (!w_draft || !n_commit || !sampled || !drafts || !n_drafts || !step_ws)
        return fail(EV_EINVAL, "%s: NULL pointer", who);
    if (!aligned(w_draft, 16) || !aligned(n_commit, 4) || !aligned(sampled, 4) || !aligned(drafts, 4) ||
        !aligned(n_drafts, 4) || !aligned(step_ws, 256))
        return fail(EV_EINVAL, "%s: misaligned pointer", who);
    if (max_drafts < 1 || max_drafts > EV_MAX_LANES - 1)
        return fail(EV_EINVAL, "%s: max_drafts=%d outside 1..15", who, max_drafts);
    if (!(min_conf >= 0.0 && min_conf <= 1.0)) return fail(EV_EINVAL, "%s: min_conf outside [0, 1]", who);
    const DraftLayout D = draft_layout(m->cfg);
    if ((rc = check_ws(who, ws, ws_bytes, D.total))) return rc;
    const ev_decoder_config& c = m->cfg;
    const int H = c.hidden, V = c.vocab, G = c.group;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    unsigned char* b = reinterpret_cast<unsigned char*>(ws);
    uint16_t* a = reinterpret_cast<uint16_t*>(b + D.off_a);
    float* z = reinterpret_cast<float*>(b + D.off_z);
    uint16_t* h = reinterpret_cast<uint16_t*>(b + D.off_h);
    float* lg = reinterpret_cast<float*>(b + D.off_logits);
    int32_t* state = reinterpret_cast<int32_t*>(b + D.off_state);
    void* lin = b + D.off_lin;
    const size_t lin_bytes = D.total - D.off_lin;
    const uint16_t* nrows = reinterpret_cast<const uint16_t*>(reinterpret_cast<const unsigned char*>(step_ws) +
                                                              m->L.off_n);
    hipLaunchKernelGGL(draft_init_kernel, dim3(1), dim3(64), 0, st, state, n_drafts);
    if ((rc = check_hip(hipGetLastError(), "draft init launch"))) return rc;
    for (int i = 0; i < max_drafts; ++i) {
        hipLaunchKernelGGL(draft_input_kernel, dim3(1), dim3(kRowThreads), 0, st, nrows, n_commit, sampled, h,
                           drafts, i, m->embed, H, V, state, a);
        if ((rc = check_hip(hipGetLastError(), "draft input launch"))) return rc;
        if ((rc = verify_linear_w4(a, 1, H, w_draft, H, G, z, lin, lin_bytes, stream))) return rc;
        hipLaunchKernelGGL(draft_norm_kernel, dim3(1), dim3(kRowThreads), 0, st, z, H, m->final_norm,
                           (float)c.rms_eps, state, h);
        if ((rc = check_hip(hipGetLastError(), "draft norm launch"))) return rc;
        if ((rc = verify_linear_w4(h, 1, H, m->w_lm, V, G, lg, lin, lin_bytes, stream))) return rc;
        hipLaunchKernelGGL(draft_pick_kernel, dim3(1), dim3(1024), 0, st, lg, V, i, (float)min_conf, state, drafts,
                           n_drafts);
        if ((rc = check_hip(hipGetLastError(), "draft pick launch"))) return rc;
    }
    return EV_OK;
}
