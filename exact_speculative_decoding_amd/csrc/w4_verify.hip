// W4 verify linear and the dense SiLU-gated MLP slice on gfx950.
//
// The multi-row verify pass computes y[r][n] = sum_k x[r][k] * w[n][k] for the
// R <= 16 draft rows of one pass, with 4-bit weights w = s*q + b in groups of
// 32 or 64 (TensorFold README, exactness paragraph and checkpoint list; blog
// "The differentiator: byte-exact drafted decoding": several draft rows share
// one forward pass, so the weights are read once for all of them).
//
// Row exactness by construction: the R rows are always padded to the 16 rows
// of one bf16 MFMA tile, so R = 1 and R = 16 execute the same instruction
// stream; an MFMA output element depends only on its own A row and B column;
// the split of K over waves, and therefore every reduction order, is a
// function of (N, K, G) only.
//
// Kernel shape: a workgroup of 4 waves shares one K-split of `cps` chunks of
// 128 k; each wave owns kNT tiles of 16 output rows, on the packed weight
// layout of w4_layout.h.
//   * per chunk and tile one contiguous 1 KB load gives the B fragments of the
//     four 32-k MFMA steps, and one 8/16 B load the (scale, bias) pairs;
//   * the activations of 4 chunks (a 512-k superchunk) are loaded once per
//     workgroup, 1 KB of one row per wave load, reordered into MFMA A fragments
//     on the way into a double-buffered LDS slab, and read back with
//     conflict-free ds_read_b128 (one barrier per superchunk);
//   * nibbles decode exactly into bf16 as 16 + q (0x4180 | q << 3: a shift and
//     an and-or per pair); one more MFMA against an all-ones B gives the group
//     sum xs of every row, and the fold is y += s * acc + (b - 16 s) * xs;
//   * a ring of kPD chunks of loads is kept in flight per wave; loads past the
//     split's last chunk use an out-of-range per-lane offset, which the buffer
//     range check turns into zeros without touching memory;
//   * in the balanced launch and the dense plain split launches a wave's issue
//     priority falls as it gets through its run (progress_priority), so the
//     workgroups that share a CU end together;
//   * dense launches that need a K-split run balanced (w4_sk_kernel): 768
//     workgroups each take an equal contiguous run of (matrix, column block,
//     superchunk) units and write one partial segment per block their run
//     touches (whole 128-B lines, turned through LDS); a second kernel adds
//     a block's segments in ascending workgroup order (fused with SiLU * up
//     for the MLP gate/up pair).  Launches whose
//     columns alone fill the chip (the LM head) and the grouped MoE down
//     passes run split (w4_verify_kernel: a plan of S splits, partials
//     [S][16][N] added in ascending split order, or direct outputs at S = 1);
//     a gate/up pair with enough tiles to fill the chip on its own, every
//     grouped MoE gate/up pass and the decoder's gate/up and q|k|v run as one
//     launch that splits K in two halves inside the workgroup and writes its
//     finished outputs itself, with no partial rows.
#include <algorithm>
#include <mutex>
#include <vector>

#include "w4_kernel.h"

namespace ev {

constexpr uint32_t kOOB = 0x80000000u;  // per-lane offset beyond every buffer: reads 0
constexpr int kLoadNT = 2;  // cache-policy operand of a buffer load: the non-temporal (nt) bit
constexpr int kSlab = kSC * kXChunkBytes;  // LDS bytes of one superchunk of activations

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// A pointer every lane holds the same value of, moved to scalar registers.
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// voff: per-lane byte offset (range-checked); soff: wave-uniform byte offset
__device__ __forceinline__ u32x4 bload128(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 bload64(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
// Weight loads: with NT the non-temporal hint (the lines are streamed once;
// the caches keep the activations and partial rows instead).
template <bool NT>
__device__ __forceinline__ u32x4 wload128(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, NT ? kLoadNT : 0));
}
template <bool NT>
__device__ __forceinline__ u32x2 wload64(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, NT ? kLoadNT : 0));
}

// A packed dword (nibbles, low to high, q0 q2 q4 q6 q1 q3 q5 q7: q_{2m} and
// q_{2m+1} 16 bits apart) -> four bf16 pairs holding 16 + q in k order (q0,q1)
// (q2,q3) (q4,q5) (q6,q7): bf16 0x4180 is 16, and q goes to mantissa bits
// 3..6.  Exact.  The offset 16 (rather than 128 with q
// in the low mantissa bits, which would save one shift in four) keeps
// b - 16 s exact in fp32 for every fp16 pair (s, b), so a one-hot row reads
// back s * q + b with a single rounding.
constexpr float kDecodeOffset = 16.f;
constexpr uint32_t kDecodeMask = 0x00780078u, kDecodeOr = 0x41804180u;
__device__ __forceinline__ u32x4 decode_nibbles(uint32_t d, uint32_t m, uint32_t off) {
    u32x4 r;
    r[0] = ((d << 3) & m) | off;
    r[1] = ((d >> 1) & m) | off;
    r[2] = ((d >> 5) & m) | off;
    r[3] = ((d >> 9) & m) | off;
    return r;
}

// Issue priority from a wave's progress through its own run of chunks: 3 in
// the first quarter, 2, 1, then 0 in the last.  Waves that share a CU are
// otherwise served oldest first, so the workgroups dispatched first finish
// early and the last ones run the end of the launch on a part-empty CU; with
// the priority falling as a wave gets ahead, the ones behind are served first
// and the runs of a CU end together.  Only the order in which ready waves
// issue changes, never what they compute.
__device__ __forceinline__ void progress_priority(int done, int total) {
    const int lv = (4 * done >= total) + (4 * done >= 2 * total) + (4 * done >= 3 * total);
    if (lv == 0)
        __builtin_amdgcn_s_setprio(3);
    else if (lv == 1)
        __builtin_amdgcn_s_setprio(2);
    else if (lv == 2)
        __builtin_amdgcn_s_setprio(1);
    else
        __builtin_amdgcn_s_setprio(0);
}

__device__ __forceinline__ float half_lo(uint32_t w) { return f16_to_f32((uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float half_hi(uint32_t w) { return f16_to_f32((uint16_t)(w >> 16)); }

// bf16_rne(silu(g) * u), silu(g) = g / (1 + e^-g): the one formula of the
// MLP glue, shared by the paired gate/up epilogue and silu_reduce_kernel.
__device__ __forceinline__ uint16_t silu_mul_bf16(float g, float u) {
    const float sg = g / (1.0f + expf(-g));
    return f32_to_bf16_rne(sg * u);
}

enum W4Mode { kPlain = 0, kPairMode = 1, kRopeMode = 2 };

// Weight formats the plain W4 launches stream:
//  * kAffine: uint4 codes with an fp16 (scale, bias) pair per group of G;
//  * kNvfp4: FP4 E2M1 codes with an FP8 E4M3 scale per block of 16 and one
//    fp32 tensor scale (the NVFP4-style checkpoints the blog's "The honest
//    limits" section names).  Same tile-chunk size as affine G = 64: 1 KB of
//    codes, then 8 scale bytes per row (block b of the chunk at byte b).
enum W4Format { kAffine = 0, kNvfp4 = 1 };

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Four E2M1 codes (one 16-bit half of a packed dword, low nibble first) ->
// four bf16, exact (the conversion's scale 1.0 leaves them unscaled).
__device__ __forceinline__ bf16x4 e2m1x4_to_bf16(uint32_t d, int half) {
    const bf16x2 lo = half ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 2)
                           : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 0);
    const bf16x2 hi = half ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 3)
                           : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 1);
    return bf16x4{lo[0], lo[1], hi[0], hi[1]};
}

// Byte `b` (0..3) of a dword as an FP8 E4M3 value, exact in fp32.
__device__ __forceinline__ float e4m3_byte(uint32_t d, int b) {
    switch (b) {
        case 0: return __builtin_amdgcn_cvt_f32_fp8((int)d, 0);
        case 1: return __builtin_amdgcn_cvt_f32_fp8((int)d, 1);
        case 2: return __builtin_amdgcn_cvt_f32_fp8((int)d, 2);
        default: return __builtin_amdgcn_cvt_f32_fp8((int)d, 3);
    }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// NVFP4 activation staging: the 16 x 16 x 16 MFMA steps of a 32-k step take
// lane (r, j)'s A fragment as x[r][4j .. 4j+3] of the step's first 16 k (one
// scale block) and x[r][16+4j .. 16+4j+3] of its second, which sit side by
// side in the lane's 16 bytes.  o holds x[r][8 xj .. 8 xj + 7] of step xst.
__device__ __forceinline__ void xstore_nvfp4(uint8_t* slab, int xc, int xst, int xj, int r, const u32x4& o) {
    const size_t base = (size_t)(xc * 4 + xst) * 64;
    const int j0 = 2 * (xj & 1), off = 8 * (xj >> 1);
    *reinterpret_cast<u32x2*>(slab + (base + r + 16 * j0) * 16 + off) = u32x2{o[0], o[1]};
    *reinterpret_cast<u32x2*>(slab + (base + r + 16 * (j0 + 1)) * 16 + off) = u32x2{o[2], o[3]};
}

// One NVFP4 chunk of kNT tiles: per 32-k step and tile, two 16 x 16 x 16 MFMA
// (one per scale block) on exactly decoded E2M1 weights, each folded into y
// with its block's E4M3 scale.  Chunks loaded as zeros (past the end) add 0.
template <int NT_>
__device__ __forceinline__ void nvfp4_chunk(const u32x4 (&q)[NT_], const uint32_t (&sb)[NT_][2],
                                            const uint8_t* xchunk, int lane, f32x4 (&y)[NT_]) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const u32x4 xa = *reinterpret_cast<const u32x4*>(xchunk + (size_t)(st * 64 + lane) * 16);
        const s16x4 A0 = __builtin_bit_cast(s16x4, u32x2{xa[0], xa[1]});
        const s16x4 A1 = __builtin_bit_cast(s16x4, u32x2{xa[2], xa[3]});
#pragma unroll
        for (int t = 0; t < NT_; ++t) {
            const uint32_t d = q[t][st];
            const f32x4 a0 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                A0, __builtin_bit_cast(s16x4, e2m1x4_to_bf16(d, 0)), zero, 0, 0, 0);
            const f32x4 a1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                A1, __builtin_bit_cast(s16x4, e2m1x4_to_bf16(d, 1)), zero, 0, 0, 0);
            const uint32_t sc = sb[t][st >> 1];
            const float s0 = e4m3_byte(sc, 2 * (st & 1)), s1 = e4m3_byte(sc, 2 * (st & 1) + 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                y[t][i] = fmaf(s0, a0[i], y[t][i]);
                y[t][i] = fmaf(s1, a1[i], y[t][i]);
            }
        }
    }
}

// One workgroup of a W4 pass.
//  * kPlain (kWaves waves): workgroup blk computes its waves' kNT tiles of
//    one matrix over one K-split and writes them to the split's partial (or
//    output) rows.
//  * The halved modes (2 kWaves waves): the first kWaves waves take the first
//    half of K (a.cps chunks), the others the rest, each half with its own
//    activation slabs; the halves meet in LDS (first half + second half) and
//    the workgroup writes finished values, with no partial rows and no second
//    kernel.
//    - kPairMode: wave w's two tiles are the gate and the up tile of the
//      same 16 columns; h = bf16(silu(g) * u).
//    - kRopeMode (the q|k|v projection): workgroup b is head b (8 tiles);
//      wave w's two tiles are tiles w and w + 4 of the head, so a lane holds
//      both members (d, d + 64) of its rotation pairs.  Query and key heads
//      are turned by the row's position (the (cos, sin) table of the slot),
//      queries go to the fp32 query rows and keys to their cache slot in
//      fp16; value heads go to the blocked value cache in fp16.
template <int G, int MODE, bool NT, int FMT = kAffine>
__device__ __forceinline__ void w4_block(const W4Args& a, long blk, uint8_t (*xlds)[kSlab]) {
    static_assert(FMT == kAffine || (MODE == kPlain && G == 64), "NVFP4 streams plain launches of 1152-B tile-chunks");
    constexpr bool PAIR = MODE != kPlain;  // the two K-halves in one workgroup
    constexpr int GPC = kKC / G;                // groups per chunk
    constexpr int SBW = GPC;                    // (scale, bias) dwords per lane per chunk
    constexpr uint32_t CB = 1024 + 64 * GPC;    // packed bytes per tile-chunk
    static_assert(kSC % kPD == 0, "ring depth must divide the superchunk");
    static_assert(!PAIR || kNT == 2, "a halved-mode wave holds two tiles");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform indices (readfirstlane keeps them, the matrix and the buffer
    // descriptors in scalar registers)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = PAIR ? wave / kWaves : 0;
    const int wv = wave - half * kWaves;    // wave within its half
    const int xt = tid - half * kThreads;   // thread within its half (activation staging)
    int cgb, split, mi, grp;
    if (PAIR) {
        cgb = (int)(blk % a.ncgb);
        grp = (int)(blk / a.ncgb);
        split = half;
        mi = 0;
    } else {
        cgb = (int)(blk % a.ncgb);
        long rest = blk / a.ncgb;
        split = (int)(rest % a.S);
        rest /= a.S;
        mi = (int)(rest % a.nmat);
        grp = (int)(rest / a.nmat);
    }
    const int cg = cgb * kWaves + wv;  // a wave past the last tile group computes zeros
    const int c0 = split * a.cps;      // a multiple of kSC
    const int c1 = min(a.nchunks, c0 + a.cps);
    const int ln = lane & 15, j = lane >> 4;

    // rows of this workgroup's pass, their activation rows, weights and outputs
    int rows = a.R;
    const uint8_t* wmat = a.w[mi];
    const uint8_t* wmat1 = MODE == kPairMode ? a.w[1] : a.w[0];  // the second tile's matrix
    float* out = a.out[mi] + (size_t)split * a.split_stride;
    uint16_t* hout = a.h;
    uint16_t* hcopy = a.h_copy;
    // activation staging: a superchunk is 16 rows of kSC * 128 k; thread tid
    // loads 16 B (8 k) of row tid / kXL + kXR * m at k = 8 (tid % kXL), m < kXP
    constexpr int kXL = 16 * kSC;          // lanes per row
    constexpr int kXR = kThreads / kXL;    // rows per pass of the workgroup
    constexpr int kXP = 16 / kXR;          // passes
    static_assert(kXR * kXP == 16, "the workgroup's passes must cover the 16 rows");
    const int xr0 = xt / kXL, col = xt % kXL;
    int xrow[kXP];
#pragma unroll
    for (int m = 0; m < kXP; ++m) xrow[m] = xr0 + kXR * m;
    if (a.gexp) {
        // every table entry of a launched group is in bounds: all of them are
        // requested before the count is tested (the empty asm takes them as
        // inputs, so none is sunk past the test into a wait of its own)
        const int gc = a.gcount[0], cnt = a.gcnt[grp], ge = a.gexp[grp];
        // the row gather as a buffer load (an empty descriptor without a
        // table reads zeros), so that no branch sits between the loads
        const rsrc_t rg = make_rsrc(uniform_ptr(a.grows), a.grows ? (uint32_t)(16 * (grp + 1)) * 4u : 0u);
        int gr[kXP];
#pragma unroll
        for (int m = 0; m < kXP; ++m)
            gr[m] = (int)__builtin_amdgcn_raw_buffer_load_b32(rg, (uint32_t)(16 * grp + xrow[m]) * 4u, 0u, 0);
        static_assert(kXP == 2, "the asm below takes both gathered rows");
        asm volatile("" ::"v"(gc), "v"(cnt), "v"(ge), "v"(gr[0]), "v"(gr[1]));
#pragma unroll
        for (int m = 0; m < kXP; ++m) xrow[m] = a.grows ? gr[m] : 16 * grp + xrow[m];
        if (grp >= gc) return;  // whole workgroup: no barrier reached
        rows = cnt;
        wmat += (size_t)ge * a.wstride;
        wmat1 += (size_t)ge * a.wstride;
        out += (size_t)grp * a.ogstride;
        hout += (size_t)grp * a.hgstride;
    }

    // the buffer descriptors in scalar registers whatever the compiler proved
    const uint32_t wbytes = __builtin_amdgcn_readfirstlane(a.wbytes);
    const rsrc_t rw = make_rsrc(uniform_ptr(wmat), wbytes);
    const rsrc_t rw1 = MODE == kPairMode ? make_rsrc(uniform_ptr(wmat1), wbytes) : rw;
    const rsrc_t rx = make_rsrc(uniform_ptr(a.x), __builtin_amdgcn_readfirstlane(a.xbytes));
    uint32_t tbase[kNT];
    bool tok[kNT];
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
        const int tile = MODE == kPairMode ? cg : (MODE == kRopeMode ? 8 * cgb + wv + 4 * t : cg * kNT + t);
        tok[t] = tile < a.tiles;
        tbase[t] = tok[t] ? (uint32_t)tile * CB : 0u;
    }
    const uint32_t cstride = (uint32_t)a.tiles * CB;  // bytes per chunk step (chunk-major tiles)
    const uint32_t vq = 16u * lane;
    const uint32_t vsb = 1024u + 4u * GPC * ln;
    // the mask stays scalar, the or-constant goes to a vector register: gfx9
    // VALU ops read at most one scalar operand, and this lets each decoded pair
    // be one v_and_or_b32
    const uint32_t dm = a.dmask;
    uint32_t doff;
    asm volatile("v_mov_b32 %0, %1" : "=v"(doff) : "s"(a.doff));

    // ---- activations: one superchunk = kSC chunks of the 16 rows.  Rows >= R
    // and k >= K read zeros.
    const int xc = col >> 4, xst = (col >> 2) & 3, xj = col & 3;
    u32x4 xin[kXP];
    auto xload = [&](int sc) {
        const int k = sc * (kSC * kKC) + 8 * col;
#pragma unroll
        for (int m = 0; m < kXP; ++m) {
            const bool ok = xr0 + kXR * m < rows && k < a.K;
            xin[m] = bload128(rx, ok ? (uint32_t)(xrow[m] * a.K + k) * 2u : kOOB, 0u);
        }
    };
    // store as the A fragment of lane r + 16 xj of step xst of chunk xc (the
    // 8 k in their natural order, as the nibble decode pairs them)
    auto xstore = [&](int buf) {
#pragma unroll
        for (int m = 0; m < kXP; ++m) {
            const int r = xr0 + kXR * m;
            const u32x4 o = xin[m];
            if constexpr (FMT == kNvfp4)
                xstore_nvfp4(&xlds[2 * half + buf][0], xc, xst, xj, r, o);
            else
                *reinterpret_cast<u32x4*>(&xlds[2 * half + buf][(size_t)((xc * 4 + xst) * 64 + r + 16 * xj) * 16]) = o;
        }
    };

    // ---- weights: register ring of kPD chunks.  Offsets within the chunk are
    // per-lane constants, the chunk and tile offsets a scalar; chunks at or past
    // c1 (and tiles past the last) get an out-of-range per-lane offset, so
    // every slot is written on every path and the ring never has to be copied.
    u32x4 qr[kPD][kNT];
    uint32_t sbr[kPD][kNT][SBW];
    auto fetch = [&](int c, int slot) {
        const bool live = c < c1;
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
            const bool ok = live && tok[t];
            const uint32_t so = tbase[t] + (uint32_t)c * cstride;
            const rsrc_t r = (MODE == kPairMode && t == 1) ? rw1 : rw;
            qr[slot][t] = wload128<NT>(r, ok ? vq : kOOB, so);
            if (GPC == 2) {
                const u32x2 v = wload64<NT>(r, ok ? vsb : kOOB, so);
                sbr[slot][t][0] = v[0];
                sbr[slot][t][GPC - 1] = v[1];
            } else {
                const u32x4 v = wload128<NT>(r, ok ? vsb : kOOB, so);
#pragma unroll
                for (int g = 0; g < SBW; ++g) sbr[slot][t][g] = v[g & 3];
            }
        }
    };

    const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    f32x4 y[kNT];
#pragma unroll
    for (int t = 0; t < kNT; ++t) y[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One chunk: per 32-k step, one MFMA for the group sums of x and one per
    // tile; per group, y += s * acc + (b - 16 s) * xs.  A chunk that was
    // loaded as zeros (past c1) adds exactly zero.
    auto compute = [&](int slot, const uint8_t* xchunk) {
        if constexpr (FMT == kNvfp4) {
            nvfp4_chunk<kNT>(qr[slot], sbr[slot], xchunk, lane, y);
            return;
        }
        f32x4 acc[kNT], xs = {0.f, 0.f, 0.f, 0.f};
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const u32x4 xa = *reinterpret_cast<const u32x4*>(xchunk + (size_t)(st * 64 + lane) * 16);
            const bf16x8 A = __builtin_bit_cast(bf16x8, xa);
            const bool first = (G == 32) || ((st & 1) == 0);
            xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, ones),
                                                        first ? zero : xs, 0, 0, 0);
#pragma unroll
            for (int t = 0; t < kNT; ++t) {
                const bf16x8 B = __builtin_bit_cast(bf16x8, decode_nibbles(qr[slot][t][st], dm, doff));
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, first ? zero : acc[t], 0, 0, 0);
            }
            const bool last = (G == 32) || ((st & 1) == 1);
            if (last) {
                const int gc = (32 * st) / G;  // group within the chunk
#pragma unroll
                for (int t = 0; t < kNT; ++t) {
                    const uint32_t sb = sbr[slot][t][gc];
                    const float sv = half_lo(sb), bv = half_hi(sb);
                    const float bp = fmaf(-kDecodeOffset, sv, bv);  // removes the decode offset
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        y[t][i] = fmaf(sv, acc[t][i], y[t][i]);
                        y[t][i] = fmaf(bp, xs[i], y[t][i]);
                    }
                }
            }
        }
    };

    // kRopeMode: the step's position, read first; each row's (cos, sin) is
    // requested after the prologue, so that neither waits at the epilogue
    long long rp0 = 0;
    if constexpr (MODE == kRopeMode) rp0 = a.rope.positions[kPos0Slot];

    // Prologue: superchunk 0 of the split loaded, the first kPD chunks of
    // weights in flight behind it, the superchunk into LDS slab 0, superchunk 1
    // in registers.
    const bool prio = MODE == kPlain && !a.gexp;  // uniform: dense plain launches
    if (prio) progress_priority(0, 1);
    const int sc0 = c0 / kSC;
    xload(sc0);
#pragma unroll
    for (int p = 0; p < kPD; ++p) {
        __builtin_amdgcn_sched_barrier(0);
        fetch(c0 + p, p);
    }
    __builtin_amdgcn_sched_barrier(0);
    xstore(0);  // waits for the activations only: they were loaded before the ring
    xload(sc0 + 1);
    __syncthreads();
    float2 rcs[4];  // kRopeMode, the first half: (cos, sin) of rows 4j + i at pair index d
    if constexpr (MODE == kRopeMode) {
        const int hd = cgb, d = 16 * wv + ln;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * j + i;
            rcs[i] = half == 0 && r < rows && hd < a.rope.NH + a.rope.NKV ? a.rope.rot[(size_t)(rp0 + r) * 64 + d]
                                                                            : float2{0.f, 0.f};
        }
    }

    // Main loop over superchunks: kSC chunks of compute on slab `buf`, each
    // refilling its ring slot; then the next superchunk's activations go to
    // the other slab, the one after is loaded, and the workgroup syncs.
    // sched_barrier keeps each refill where it is written, so the loads of the
    // other ring slots stay in flight across the compute of this one.  Both
    // halves of a paired workgroup run a.cps / kSC superchunks (chunks past
    // the end of K read zeros), so every wave reaches the same barriers.
    const int ntrip = PAIR ? a.cps / kSC : (c1 - c0 + kSC - 1) / kSC;
    int buf = 0;
    for (int it = 0, cb = c0; it < ntrip; ++it, cb += kSC) {
#pragma unroll
        for (int p = 0; p < kSC; ++p) {
            if (prio) progress_priority(kSC * it + p, kSC * ntrip);
            __builtin_amdgcn_sched_barrier(0);
            compute(p % kPD, &xlds[2 * half + buf][(size_t)p * kXChunkBytes]);
            __builtin_amdgcn_sched_barrier(0);
            fetch(cb + p + kPD, p % kPD);
        }
        __builtin_amdgcn_sched_barrier(0);
        xstore(buf ^ 1);
        xload(cb / kSC + 2);
        __syncthreads();
        buf ^= 1;
    }
    __builtin_amdgcn_sched_barrier(0);

    if (PAIR) {
        // the second half's accumulators through LDS (the slabs are no longer
        // read), then h for rows r = 4j + i of columns 16 cg + ln
        f32x4* ex = reinterpret_cast<f32x4*>(&xlds[0][0]);
        static_assert(kWaves * kNT * 64 * 16 <= 2 * kSlab, "exchange fits the first half's slabs");
        if (half == 1) {
#pragma unroll
            for (int t = 0; t < kNT; ++t) ex[(wv * kNT + t) * 64 + lane] = y[t];
        }
        __syncthreads();
        if (half == 0 && MODE == kRopeMode) {
#pragma unroll
            for (int t = 0; t < kNT; ++t) y[t] += ex[(wv * kNT + t) * 64 + lane];
            const int hd = cgb, d = 16 * wv + ln;  // head, and d < 64 of the pair (d, d + 64)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * j + i;
                if (r >= rows) continue;
                const long long P = rp0 + r;
                const float va = y[0][i], vb = y[1][i];
                if (hd < a.rope.NH + a.rope.NKV) {
                    // one fused step each, written out so that the compiler
                    // has no contraction to choose
                    const float2 cs = rcs[i];
                    const float a2 = fmaf(va, cs.x, -(vb * cs.y));
                    const float b2 = fmaf(vb, cs.x, va * cs.y);
                    if (hd < a.rope.NH) {
                        float* q = a.rope.q + ((size_t)r * a.rope.NH + hd) * 128;
                        q[d] = a2;
                        q[d + 64] = b2;
                    } else {
                        uint16_t* k = a.rope.kc + ((size_t)(hd - a.rope.NH) * a.rope.C + P) * 128;
                        k[d] = f32_to_f16_sat(a2);
                        k[d + 64] = f32_to_f16_sat(b2);
                    }
                } else {
                    const int g = hd - a.rope.NH - a.rope.NKV;
                    uint16_t* v = a.rope.vc + (size_t)g * a.rope.C * 128 + (size_t)(P / 32) * 128 * 32 +
                                  vslot_pos32((int)(P % 32));
                    v[(size_t)d * 32] = f32_to_f16_sat(va);
                    v[(size_t)(d + 64) * 32] = f32_to_f16_sat(vb);
                }
            }
        }
        if (half == 0 && MODE == kPairMode) {
#pragma unroll
            for (int t = 0; t < kNT; ++t) y[t] += ex[(wv * kNT + t) * 64 + lane];
            const int n = cg * 16 + ln;
            if (tok[0] && n < a.N) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * j + i;
                    if (r < rows) {
                        const uint16_t hv = silu_mul_bf16(y[0][i], y[1][i]);
                        hout[(size_t)r * a.N + n] = hv;
                        if (hcopy) hcopy[(size_t)r * a.N + n] = hv;
                    }
                }
            }
        }
        return;
    }

    // rows r = 4j + i of columns 16 * tile + ln
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
        const int n = (cg * kNT + t) * 16 + ln;
        if (tok[t] && n < a.N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * j + i;
                if (r < rows) out[(size_t)r * a.N + n] = FMT == kNvfp4 ? y[t][i] * a.tscale : y[t][i];
            }
        }
    }
}

template <int G, bool NT, int FMT = kAffine>
__global__ __launch_bounds__(kThreads) void w4_verify_kernel(W4Args a) {
    __shared__ __align__(16) uint8_t xlds[2][kSlab];
    if (a.tstamp && threadIdx.x == 0) a.tstamp[2 * blockIdx.x] = wall_clock64();
    w4_block<G, kPlain, NT, FMT>(a, blockIdx.x, xlds);
    if (a.tstamp) {  // uniform; grouped launches (which may return early) are never timed
        __syncthreads();
        if (threadIdx.x == 0) a.tstamp[2 * blockIdx.x + 1] = wall_clock64();
    }
}

// Balanced (stream-K) W4 pass.  Workgroup w runs the units [w U / nwg,
// (w + 1) U / nwg) of the launch's unit list (matrix, column block,
// superchunk), so every workgroup streams the same weight bytes to within one
// superchunk and, with nwg equal to the resident capacity of the chip, every
// CU holds the same number of workgroups: no CU is left with an extra
// workgroup to finish after the others.  The walk keeps the pipeline of the
// split pass across unit and block boundaries (the ring of weight chunks and
// the next superchunk's activations stay in flight); when the next unit starts
// another block, the workgroup writes its accumulators as one partial segment
// and starts again from zero.  The segments of a block are added in ascending
// workgroup order by sk_reduce_kernel.
template <int G, bool NT, int FMT = kAffine>
__device__ __forceinline__ void w4_sk_block(const W4Args& a, int w, uint8_t (*xlds)[kSlab]) {
    static_assert(FMT == kAffine || G == 64, "NVFP4 tile-chunks have the 1152-B size of G = 64");
    constexpr int GPC = kKC / G;
    constexpr int SBW = GPC;
    constexpr uint32_t CB = 1024 + 64 * GPC;
    static_assert(kSC % kPD == 0, "ring depth must divide the superchunk");

    const int U = a.sk_units, nwg = a.sk_nwg, nsc = a.sk_nsc;
    const int u0 = (int)((unsigned)w * (unsigned)U / (unsigned)nwg);
    const int u1 = (int)((unsigned)(w + 1) * (unsigned)U / (unsigned)nwg);
    if (u0 >= u1) return;  // whole workgroup (nwg <= U keeps every run non-empty)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15, j = lane >> 4;
    const int rows = a.R;

    constexpr int kXL = 16 * kSC;
    constexpr int kXR = kThreads / kXL;
    constexpr int kXP = 16 / kXR;
    static_assert(kXR * kXP == 16, "the workgroup's passes must cover the 16 rows");
    const int xr0 = tid / kXL, col = tid % kXL;
    const uint32_t wbytes = __builtin_amdgcn_readfirstlane(a.wbytes);
    const rsrc_t rx = make_rsrc(uniform_ptr(a.x), __builtin_amdgcn_readfirstlane(a.xbytes));
    const uint32_t cstride = (uint32_t)a.tiles * CB;
    const uint32_t vq = 16u * lane;
    const uint32_t vsb = 1024u + 4u * GPC * ln;
    const uint32_t dm = a.dmask;
    uint32_t doff;
    asm volatile("v_mov_b32 %0, %1" : "=v"(doff) : "s"(a.doff));

    // A unit's place: superchunk sc of column block cb of matrix m.
    struct Unit {
        int sc, cb, m;
    };
    auto next = [&](Unit v) {
        if (++v.sc == nsc) {
            v.sc = 0;
            if (++v.cb == a.ncgb) {
                v.cb = 0;
                ++v.m;
            }
        }
        return v;
    };
    Unit cur;
    {
        const int blk = u0 / nsc;
        cur.sc = u0 - blk * nsc;
        cur.m = blk / a.ncgb;
        cur.cb = blk - cur.m * a.ncgb;
    }

    // activations of superchunk sc (zeros when !live, for rows >= R, k >= K)
    const int xc = col >> 4, xst = (col >> 2) & 3, xj = col & 3;
    u32x4 xin[kXP];
    auto xload = [&](bool live, int sc) {
        const int k = sc * (kSC * kKC) + 8 * col;
#pragma unroll
        for (int m = 0; m < kXP; ++m) {
            const int r = xr0 + kXR * m;
            const bool ok = live && r < rows && k < a.K;
            xin[m] = bload128(rx, ok ? (uint32_t)(r * a.K + k) * 2u : kOOB, 0u);
        }
    };
    auto xstore = [&](int buf) {
#pragma unroll
        for (int m = 0; m < kXP; ++m) {
            const int r = xr0 + kXR * m;
            const u32x4 o = xin[m];
            if constexpr (FMT == kNvfp4)
                xstore_nvfp4(&xlds[buf][0], xc, xst, xj, r, o);
            else
                *reinterpret_cast<u32x4*>(&xlds[buf][(size_t)((xc * 4 + xst) * 64 + r + 16 * xj) * 16]) = o;
        }
    };

    // chunk p of unit v for the wave's kNT tiles of the unit's block, into
    // ring slot `slot` (zeros when !live, past the last chunk or tile)
    u32x4 qr[kPD][kNT];
    uint32_t sbr[kPD][kNT][SBW];
    auto fetch = [&](bool live, Unit v, int p, int slot) {
        const int c = v.sc * kSC + p;
        // the descriptor from a pointer moved to scalar registers, so the
        // matrix select can never turn it into a per-lane value
        const rsrc_t r = make_rsrc(uniform_ptr(v.m ? a.w[1] : a.w[0]), wbytes);
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
            const int tile = (v.cb * kWaves + wave) * kNT + t;
            const bool ok = live && c < a.nchunks && tile < a.tiles;
            const uint32_t so = ok ? (uint32_t)tile * CB + (uint32_t)c * cstride : 0u;
            qr[slot][t] = wload128<NT>(r, ok ? vq : kOOB, so);
            if (GPC == 2) {
                const u32x2 x2 = wload64<NT>(r, ok ? vsb : kOOB, so);
                sbr[slot][t][0] = x2[0];
                sbr[slot][t][GPC - 1] = x2[1];
            } else {
                const u32x4 x4 = wload128<NT>(r, ok ? vsb : kOOB, so);
#pragma unroll
                for (int g = 0; g < SBW; ++g) sbr[slot][t][g] = x4[g & 3];
            }
        }
    };

    const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    f32x4 y[kNT];
#pragma unroll
    for (int t = 0; t < kNT; ++t) y[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // one chunk, exactly as in the split pass
    auto compute = [&](int slot, const uint8_t* xchunk) {
        if constexpr (FMT == kNvfp4) {
            nvfp4_chunk<kNT>(qr[slot], sbr[slot], xchunk, lane, y);
            return;
        }
        f32x4 acc[kNT], xs = {0.f, 0.f, 0.f, 0.f};
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const u32x4 xa = *reinterpret_cast<const u32x4*>(xchunk + (size_t)(st * 64 + lane) * 16);
            const bf16x8 A = __builtin_bit_cast(bf16x8, xa);
            const bool first = (G == 32) || ((st & 1) == 0);
            xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, ones),
                                                        first ? zero : xs, 0, 0, 0);
#pragma unroll
            for (int t = 0; t < kNT; ++t) {
                const bf16x8 B = __builtin_bit_cast(bf16x8, decode_nibbles(qr[slot][t][st], dm, doff));
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, first ? zero : acc[t], 0, 0, 0);
            }
            const bool last = (G == 32) || ((st & 1) == 1);
            if (last) {
                const int gc = (32 * st) / G;
#pragma unroll
                for (int t = 0; t < kNT; ++t) {
                    const uint32_t sb = sbr[slot][t][gc];
                    const float sv = half_lo(sb), bv = half_hi(sb);
                    const float bp = fmaf(-kDecodeOffset, sv, bv);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        y[t][i] = fmaf(sv, acc[t][i], y[t][i]);
                        y[t][i] = fmaf(bp, xs[i], y[t][i]);
                    }
                }
            }
        }
    };
    // segment s of the run: the wave's 16 rows x (kNT * 16) columns
    // (block columns (wave, tile) * 16 + ln hold rows 4j + i) are turned
    // through a wave-private LDS tile, so that a lane stores 4 consecutive
    // columns of one row and every store writes whole 128-B lines (rows
    // >= R are not written); the accumulators start again from zero
    static_assert(kNT * 16 == 32, "a lane stores a quarter of a wave's 128-B row");
    __shared__ __align__(16) float segx[kWaves][16 * 32];
    float* const sx = segx[wave];
    const rsrc_t rp = make_rsrc(uniform_ptr(a.sk_part),
                                (uint32_t)((size_t)a.sk_nwg * a.sk_segmax * 16 * kBlockCols * sizeof(float)));
    auto flush = [&](int s) {
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sx[(4 * j + i) * 32 + t * 16 + ln] = FMT == kNvfp4 ? y[t][i] * a.tscale : y[t][i];
            y[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const uint32_t seg = (uint32_t)(((size_t)w * a.sk_segmax + s) * 16 * kBlockCols * sizeof(float));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = (lane >> 3) + 8 * h, c4 = 4 * (lane & 7);
            const u32x4 v = *reinterpret_cast<const u32x4*>(&sx[r * 32 + c4]);
            const uint32_t off = seg + (uint32_t)(r * kBlockCols + wave * 32 + c4) * 4u;
            __builtin_amdgcn_raw_buffer_store_b128(v, rp, r < rows ? off : kOOB, 0u, 0);
        }
    };

    // Prologue: unit u0's activations loaded, its first kPD chunks of weights
    // in flight behind them, the activations into slab 0, unit u0 + 1's
    // activations in registers.
    progress_priority(0, 1);
    Unit nxt = next(cur);
    xload(true, cur.sc);
#pragma unroll
    for (int p = 0; p < kPD; ++p) {
        __builtin_amdgcn_sched_barrier(0);
        fetch(true, cur, p, p);
    }
    __builtin_amdgcn_sched_barrier(0);
    xstore(0);  // waits for the activations only: they were loaded before the ring
    xload(u0 + 1 < u1, nxt.sc);
    __syncthreads();

    // One unit per trip: kSC chunks of compute on slab `buf`, each refilling
    // its ring slot with the chunk kPD ahead (in this unit or the next); a
    // segment ends where the next unit starts a block (or the run ends); then
    // the next unit's activations go to the other slab, the one after is
    // loaded, and the workgroup syncs.
    int buf = 0, seg = 0;
    for (int u = u0; u < u1; ++u) {
        const bool live1 = u + 1 < u1;
#pragma unroll
        for (int p = 0; p < kSC; ++p) {
            progress_priority(kSC * (u - u0) + p, kSC * (u1 - u0));
            __builtin_amdgcn_sched_barrier(0);
            compute(p % kPD, &xlds[buf][(size_t)p * kXChunkBytes]);
            __builtin_amdgcn_sched_barrier(0);
            if (p + kPD < kSC)
                fetch(true, cur, p + kPD, p % kPD);
            else
                fetch(live1, nxt, p + kPD - kSC, p % kPD);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (!live1 || nxt.sc == 0) flush(seg++);
        const Unit nn = next(nxt);
        xstore(buf ^ 1);
        xload(u + 2 < u1, nn.sc);
        __syncthreads();
        buf ^= 1;
        cur = nxt;
        nxt = nn;
    }
}

template <int G, bool NT, int FMT = kAffine>
__global__ __launch_bounds__(kThreads) void w4_sk_kernel(W4Args a) {
    __shared__ __align__(16) uint8_t xlds[2][kSlab];
    if (a.tstamp && threadIdx.x == 0) a.tstamp[2 * blockIdx.x] = wall_clock64();
    w4_sk_block<G, NT, FMT>(a, blockIdx.x, xlds);
    if (a.tstamp) {
        __syncthreads();
        if (threadIdx.x == 0) a.tstamp[2 * blockIdx.x + 1] = wall_clock64();
    }
}

template <int G, int MODE, bool NT>
__global__ __launch_bounds__(2 * kThreads) void w4_pair_kernel(W4Args a) {
    __shared__ __align__(16) uint8_t xlds[4][kSlab];
    if (a.tstamp && threadIdx.x == 0) a.tstamp[2 * blockIdx.x] = wall_clock64();
    w4_block<G, MODE, NT>(a, blockIdx.x, xlds);
    if (a.tstamp) {
        __syncthreads();
        if (threadIdx.x == 0) a.tstamp[2 * blockIdx.x + 1] = wall_clock64();
    }
}

// K-parts launch for dense matrices with at most PARTS * PC chunks of K: a
// workgroup of PARTS waves owns one column unit and wave p takes the p-th run
// of a.cps <= PC chunks of K.  The unit is
//   * kPlain: one tile of 16 columns of one of a.S K-splits (workgroup
//     split * tiles + tile); the workgroup writes the split's fp32 rows at
//     out + split * split_stride, to be added in ascending split order;
//   * kPairMode: the gate and the up tile of 16 columns; h = bf16(silu(g)*u);
//   * kRopeMode: tiles u and u + 4 of head hd, the rotation pairs (d, d + 64)
//     with d = 16 u + ln, rotated and written as w4_block's epilogue does.
// A wave requests its whole run at once, the activation fragments straight
// from memory (lane r + 16 xj of step st of chunk c holds x[r][128 c + 32 st
// + 8 xj .. + 7], the layout the LDS slabs of w4_block hold) and its tiles'
// weights.  The parts meet in LDS and wave 0 adds them in ascending p, an
// order fixed by K alone.  One workgroup per tile (four per head) spreads a
// decoder-sized matrix over many CUs: at these sizes a CU's share of the
// bytes, not the chip's bandwidth, sets the time.
template <int G, int MODE, bool NT, int PARTS, int PC>
__device__ __forceinline__ void w4_parts_block(const W4Args& a, f32x4 (*ex)[MODE == kPlain ? 1 : 2][64]) {
    constexpr int NTW = MODE == kPlain ? 1 : 2;  // tiles per wave
    constexpr int GPC = kKC / G;
    constexpr int SBW = GPC;
    constexpr uint32_t CB = 1024 + 64 * GPC;
    constexpr int PD = PC;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int part = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15, j = lane >> 4;
    const int rows = a.R;
    const int split = MODE == kPlain ? blockIdx.x / a.tiles : 0;
    const int unit = blockIdx.x - split * (MODE == kPlain ? a.tiles : 0);
    const int hd = MODE == kRopeMode ? unit >> 2 : 0, u = MODE == kRopeMode ? unit & 3 : 0;
    const int tile0 = MODE == kRopeMode ? 8 * hd + u : unit;
    const int tile1 = MODE == kRopeMode ? tile0 + 4 : unit;  // unused in kPlain
    const int c0 = (split * PARTS + part) * a.cps;
    const int c1 = min(a.nchunks, c0 + a.cps);

    const uint32_t wbytes = __builtin_amdgcn_readfirstlane(a.wbytes);
    const rsrc_t rw0 = make_rsrc(uniform_ptr(a.w[0]), wbytes);
    const rsrc_t rw1 = MODE == kPairMode ? make_rsrc(uniform_ptr(a.w[1]), wbytes) : rw0;
    const rsrc_t rx = make_rsrc(uniform_ptr(a.x), __builtin_amdgcn_readfirstlane(a.xbytes));
    const bool tok[2] = {tile0 < a.tiles, tile1 < a.tiles};
    const uint32_t tbase[2] = {tok[0] ? (uint32_t)tile0 * CB : 0u, tok[1] ? (uint32_t)tile1 * CB : 0u};
    const uint32_t cstride = (uint32_t)a.tiles * CB;
    const uint32_t vq = 16u * lane;
    const uint32_t vsb = 1024u + 4u * GPC * ln;
    const uint32_t dm = a.dmask;
    uint32_t doff;
    asm volatile("v_mov_b32 %0, %1" : "=v"(doff) : "s"(a.doff));
    const bool xrow_ok = ln < rows;
    const uint32_t xoff = (uint32_t)(ln * a.K + 8 * j) * 2u;

    // the run: activation fragments and both tiles' weights of PD chunks;
    // chunks at or past c1 read zeros and add exactly zero
    u32x4 xa[PD][4];
    u32x4 qr[PD][NTW];
    uint32_t sbr[PD][NTW][SBW];
    auto fetch = [&](int c, int slot) {
        const bool live = c < c1;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int k = 128 * c + 32 * st;
            const bool ok = live && xrow_ok && k + 8 * j < a.K;
            xa[slot][st] = bload128(rx, ok ? xoff + (uint32_t)k * 2u : kOOB, 0u);
        }
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
            const bool ok = live && tok[t];
            const uint32_t so = tbase[t] + (uint32_t)c * cstride;
            const rsrc_t r = t == 1 ? rw1 : rw0;
            qr[slot][t] = wload128<NT>(r, ok ? vq : kOOB, so);
            if (GPC == 2) {
                const u32x2 v = wload64<NT>(r, ok ? vsb : kOOB, so);
                sbr[slot][t][0] = v[0];
                sbr[slot][t][GPC - 1] = v[1];
            } else {
                const u32x4 v = wload128<NT>(r, ok ? vsb : kOOB, so);
#pragma unroll
                for (int g = 0; g < SBW; ++g) sbr[slot][t][g] = v[g & 3];
            }
        }
    };

    const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    f32x4 y[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) y[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // one chunk, the arithmetic of w4_block's affine chunk: per 32-k step one
    // MFMA for the group sums of x and one per tile; per group
    // y += s * acc + (b - 16 s) * xs
    auto compute = [&](int slot) {
        f32x4 acc[NTW], xs = {0.f, 0.f, 0.f, 0.f};
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const bf16x8 A = __builtin_bit_cast(bf16x8, xa[slot][st]);
            const bool first = (G == 32) || ((st & 1) == 0);
            xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, ones), first ? zero : xs, 0,
                                                        0, 0);
#pragma unroll
            for (int t = 0; t < NTW; ++t) {
                const bf16x8 B = __builtin_bit_cast(bf16x8, decode_nibbles(qr[slot][t][st], dm, doff));
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, first ? zero : acc[t], 0, 0, 0);
            }
            const bool last = (G == 32) || ((st & 1) == 1);
            if (last) {
                const int gc = (32 * st) / G;
#pragma unroll
                for (int t = 0; t < NTW; ++t) {
                    const uint32_t sb = sbr[slot][t][gc];
                    const float sv = half_lo(sb), bv = half_hi(sb);
                    const float bp = fmaf(-kDecodeOffset, sv, bv);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        y[t][i] = fmaf(sv, acc[t][i], y[t][i]);
                        y[t][i] = fmaf(bp, xs[i], y[t][i]);
                    }
                }
            }
        }
    };

    // kRopeMode: the step's position first, then the run, then the rows'
    // (cos, sin), so that the epilogue waits for none of them
    long long rp0 = 0;
    if constexpr (MODE == kRopeMode) rp0 = a.rope.positions[kPos0Slot];
#pragma unroll
    for (int p = 0; p < PD; ++p) {
        __builtin_amdgcn_sched_barrier(0);
        fetch(c0 + p, p);
    }
    __builtin_amdgcn_sched_barrier(0);
    float2 rcs[4];
    if constexpr (MODE == kRopeMode) {
        const int d = 16 * u + ln;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * j + i;
            rcs[i] = part == 0 && r < rows && hd < a.rope.NH + a.rope.NKV ? a.rope.rot[(size_t)(rp0 + r) * 64 + d]
                                                                           : float2{0.f, 0.f};
        }
    }
#pragma unroll
    for (int p = 0; p < PD; ++p) {
        __builtin_amdgcn_sched_barrier(0);
        compute(p);
    }
    __builtin_amdgcn_sched_barrier(0);

    // parts 1.. through LDS; wave 0 adds them in ascending part order
    if (part > 0) {
#pragma unroll
        for (int t = 0; t < NTW; ++t) ex[part - 1][t][lane] = y[t];
    }
    __syncthreads();
    if (part != 0) return;
#pragma unroll
    for (int p = 1; p < PARTS; ++p) {
#pragma unroll
        for (int t = 0; t < NTW; ++t) y[t] += ex[p - 1][t][lane];
    }
    if constexpr (MODE == kPlain) {
        const int n = unit * 16 + ln;
        if (tok[0] && n < a.N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * j + i;
                if (r < rows) a.out[0][(size_t)split * a.split_stride + (size_t)r * a.N + n] = y[0][i];
            }
        }
    } else if constexpr (MODE == kRopeMode) {
        const int d = 16 * u + ln;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * j + i;
            if (r >= rows) continue;
            const long long P = rp0 + r;
            const float va = y[0][i], vb = y[1][i];
            if (hd < a.rope.NH + a.rope.NKV) {
                // one fused step each, written out so that the compiler has
                // no contraction to choose
                const float2 cs = rcs[i];
                const float a2 = fmaf(va, cs.x, -(vb * cs.y));
                const float b2 = fmaf(vb, cs.x, va * cs.y);
                if (hd < a.rope.NH) {
                    float* q = a.rope.q + ((size_t)r * a.rope.NH + hd) * 128;
                    q[d] = a2;
                    q[d + 64] = b2;
                } else {
                    uint16_t* k = a.rope.kc + ((size_t)(hd - a.rope.NH) * a.rope.C + P) * 128;
                    k[d] = f32_to_f16_sat(a2);
                    k[d + 64] = f32_to_f16_sat(b2);
                }
            } else {
                const int g = hd - a.rope.NH - a.rope.NKV;
                uint16_t* v = a.rope.vc + (size_t)g * a.rope.C * 128 + (size_t)(P / 32) * 128 * 32 +
                              vslot_pos32((int)(P % 32));
                v[(size_t)d * 32] = f32_to_f16_sat(va);
                v[(size_t)(d + 64) * 32] = f32_to_f16_sat(vb);
            }
        }
    } else {
        const int n = unit * 16 + ln;
        if (tok[0] && n < a.N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * j + i;
                if (r < rows) {
                    const uint16_t hv = silu_mul_bf16(y[0][i], y[NTW - 1][i]);
                    a.h[(size_t)r * a.N + n] = hv;
                    if (a.h_copy) a.h_copy[(size_t)r * a.N + n] = hv;
                }
            }
        }
    }
}

template <int G, int MODE, bool NT, int PARTS, int PC>
__global__ __launch_bounds__(64 * PARTS) void w4_parts_kernel(W4Args a) {
    __shared__ f32x4 ex[PARTS - 1][MODE == kPlain ? 1 : 2][64];
    if (a.tstamp && threadIdx.x == 0) a.tstamp[2 * blockIdx.x] = wall_clock64();
    w4_parts_block<G, MODE, NT, PARTS, PC>(a, ex);
    if (a.tstamp) {
        __syncthreads();
        if (threadIdx.x == 0) a.tstamp[2 * blockIdx.x + 1] = wall_clock64();
    }
}

// y[r][n] = sum over s = 0..S-1, ascending, of part[s][r][n].  One thread per
// 4 consecutive n of one row; the loads of all splits are issued ahead of the
// additions, which run in ascending s.
__global__ __launch_bounds__(64) void splitk_reduce_kernel(const float* __restrict__ part, int S, int N,
                                                           float* __restrict__ y) {
    const int n4 = (blockIdx.x * 64 + threadIdx.x) * 4;
    const int r = blockIdx.y;
    if (n4 >= N) return;
    const size_t stride = (size_t)16 * N;
    const size_t o = (size_t)r * N + n4;
    const bool vec = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(part) & 15) == 0;
    if (vec) {
        // every split's load of a batch is issued before the batch's additions
        // (one memory round trip per 32 splits), which still run in ascending s
        constexpr int kB = 32;
        f32x4 acc = *reinterpret_cast<const f32x4*>(part + o);
        for (int s0 = 1; s0 < S; s0 += kB) {
            f32x4 v[kB];
#pragma unroll
            for (int u = 0; u < kB; ++u)
                if (s0 + u < S) v[u] = *reinterpret_cast<const f32x4*>(part + (size_t)(s0 + u) * stride + o);
#pragma unroll
            for (int u = 0; u < kB; ++u)
                if (s0 + u < S) acc += v[u];
        }
        *reinterpret_cast<f32x4*>(y + o) = acc;
    } else {
        for (int i = 0; i < 4 && n4 + i < N; ++i) {
            float acc = part[o + i];
            for (int s = 1; s < S; ++s) acc += part[s * stride + o + i];
            y[o + i] = acc;
        }
    }
}

// g, u = split sums (ascending s); h = bf16_rne(silu(g) * u) for rows < R.
// One thread per 8 consecutive k of one row; h is written to `h` (the down
// projection's input) and, when asked, to `h_copy`.  Grouped (gcnt != NULL):
// grid z is the group, rows < gcnt[z] of groups < *gcount.
__global__ __launch_bounds__(64) void silu_reduce_kernel(const float* __restrict__ pg,
                                                         const float* __restrict__ pu, int S, int I,
                                                         uint16_t* __restrict__ h,
                                                         uint16_t* __restrict__ h_copy,
                                                         const int* __restrict__ gcount,
                                                         const int* __restrict__ gcnt, long gstride_p,
                                                         long gstride_h) {
    const int m = blockIdx.x * 64 + threadIdx.x;  // I % 32 == 0: groups of 8 never straddle rows
    const int r = blockIdx.y;
    if (8 * m >= I) return;
    if (gcnt) {
        const int g = blockIdx.z;
        if (g >= gcount[0] || r >= gcnt[g]) return;
        pg += g * gstride_p;
        pu += g * gstride_p;
        h += g * gstride_h;
    }
    const size_t stride = (size_t)16 * I;
    const size_t o = (size_t)r * I + 8 * m;
    // all loads of a batch of 8 splits are issued before its additions, which
    // run in ascending split order
    f32x4 g0 = {0.f, 0.f, 0.f, 0.f}, g1 = g0, u0 = g0, u1 = g0;
    for (int s0 = 0; s0 < S; s0 += 8) {
        f32x4 v[8][4];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < S) {
                const size_t so = (size_t)(s0 + u) * stride + o;
                v[u][0] = *reinterpret_cast<const f32x4*>(pg + so);
                v[u][1] = *reinterpret_cast<const f32x4*>(pg + so + 4);
                v[u][2] = *reinterpret_cast<const f32x4*>(pu + so);
                v[u][3] = *reinterpret_cast<const f32x4*>(pu + so + 4);
            }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < S) {
                if (s0 + u == 0) {
                    g0 = v[u][0];
                    g1 = v[u][1];
                    u0 = v[u][2];
                    u1 = v[u][3];
                } else {
                    g0 += v[u][0];
                    g1 += v[u][1];
                    u0 += v[u][2];
                    u1 += v[u][3];
                }
            }
    }
    uint16_t hv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float g = i < 4 ? g0[i] : g1[i - 4];
        const float u = i < 4 ? u0[i] : u1[i - 4];
        hv[i] = silu_mul_bf16(g, u);
    }
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)hv[2 * i] | ((uint32_t)hv[2 * i + 1] << 16);
    *reinterpret_cast<u32x4*>(h + o) = w;
    if (h_copy) *reinterpret_cast<u32x4*>(h_copy + o) = w;
}

// y[r][n] = the sum of column n's block segments over first(b) .. last(b),
// ascending, rows r < R (grid y).  One thread per 4 consecutive n; the loads
// of a batch of 32 workgroups are issued before its additions.
__global__ __launch_bounds__(64) void sk_reduce_kernel(const float* __restrict__ part, SkGeom g, int N,
                                                       float* __restrict__ y) {
    const int n4 = (blockIdx.x * 64 + threadIdx.x) * 4;
    const int r = blockIdx.y;
    if (n4 >= N) return;
    const int b = n4 / kBlockCols, cl = n4 % kBlockCols;
    const SkSpan sp = sk_span(part, g, b, r, cl);
    f32x4 acc = *reinterpret_cast<const f32x4*>(sp.p0);
    constexpr int kB = 32;
    for (int wb = sp.w0 + 1; wb <= sp.w1; wb += kB) {
        f32x4 v[kB];
#pragma unroll
        for (int i = 0; i < kB; ++i)
            if (wb + i <= sp.w1) v[i] = *reinterpret_cast<const f32x4*>(sk_seg0(part, g, wb + i, r, cl));
#pragma unroll
        for (int i = 0; i < kB; ++i)
            if (wb + i <= sp.w1) acc += v[i];
    }
    float* o = y + (size_t)r * N + n4;
    if ((N & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0) {
        *reinterpret_cast<f32x4*>(o) = acc;
    } else {
        for (int i = 0; i < 4 && n4 + i < N; ++i) o[i] = acc[i];
    }
}

// h[r][k] = bf16_rne(silu(g) * u), g and u the segment sums (ascending
// workgroups) of column k's block in the gate (blocks 0..ncgb-1) and the up
// matrix (blocks ncgb..); one thread per 4 consecutive k.  The loads of a
// batch of 8 workgroups of each matrix are issued together.
__global__ __launch_bounds__(64) void sk_silu_reduce_kernel(const float* __restrict__ part, SkGeom g, int ncgb,
                                                            int I, uint16_t* __restrict__ h,
                                                            uint16_t* __restrict__ h_copy) {
    const int k4 = (blockIdx.x * 64 + threadIdx.x) * 4;
    const int r = blockIdx.y;
    if (k4 >= I) return;
    const int b = k4 / kBlockCols, cl = k4 % kBlockCols;
    const SkSpan sg = sk_span(part, g, b, r, cl), su = sk_span(part, g, ncgb + b, r, cl);
    f32x4 gs = *reinterpret_cast<const f32x4*>(sg.p0), us = *reinterpret_cast<const f32x4*>(su.p0);
    constexpr int kB = 8;
    for (int i0 = 1; sg.w0 + i0 <= sg.w1 || su.w0 + i0 <= su.w1; i0 += kB) {
        f32x4 vg[kB], vu[kB];
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            if (sg.w0 + i0 + i <= sg.w1) vg[i] = *reinterpret_cast<const f32x4*>(sk_seg0(part, g, sg.w0 + i0 + i, r, cl));
            if (su.w0 + i0 + i <= su.w1) vu[i] = *reinterpret_cast<const f32x4*>(sk_seg0(part, g, su.w0 + i0 + i, r, cl));
        }
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            if (sg.w0 + i0 + i <= sg.w1) gs += vg[i];
            if (su.w0 + i0 + i <= su.w1) us += vu[i];
        }
    }
    uint32_t w2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        w2[i] = (uint32_t)silu_mul_bf16(gs[2 * i], us[2 * i]) |
                ((uint32_t)silu_mul_bf16(gs[2 * i + 1], us[2 * i + 1]) << 16);
    const size_t o = (size_t)r * I + k4;
    const u32x2 wv = {w2[0], w2[1]};
    *reinterpret_cast<u32x2*>(h + o) = wv;
    if (h_copy) *reinterpret_cast<u32x2*>(h_copy + o) = wv;
}

int32_t launch_sk_reduce(const float* part, const SkPlan& q, int nmat, int N, int R, float* y, uint16_t* h,
                         uint16_t* h_copy, hipStream_t st) {
    const SkGeom g = sk_geom(q);
    if (nmat == 1) {
        dim3 grid((unsigned)((N + 255) / 256), (unsigned)R);
        hipLaunchKernelGGL(sk_reduce_kernel, grid, dim3(64), 0, st, part, g, N, y);
    } else {
        if (N % 32 != 0) return fail(EV_EINVAL, "sk reduce: I=%d is not a multiple of 32", N);
        dim3 grid((unsigned)((N / 4 + 63) / 64), (unsigned)R);
        hipLaunchKernelGGL(sk_silu_reduce_kernel, grid, dim3(64), 0, st, part, g, q.ncgb, N, h, h_copy);
    }
    return check_hip(hipGetLastError(), "sk reduce launch");
}

int32_t launch_splitk_reduce(const float* part, int S, int N, int R, float* y, hipStream_t st) {
    dim3 grid((unsigned)((N + 255) / 256), (unsigned)R);
    hipLaunchKernelGGL(splitk_reduce_kernel, grid, dim3(64), 0, st, part, S, N, y);
    return check_hip(hipGetLastError(), "splitk_reduce launch");
}

int32_t launch_silu_reduce(const float* pg, const float* pu, int S, int I, int R, uint16_t* h,
                           uint16_t* h_copy, int ngroups, const int* gcount, const int* gcnt,
                           long gstride_p, long gstride_h, hipStream_t st) {
    dim3 grid((unsigned)((I / 8 + 63) / 64), (unsigned)R, (unsigned)ngroups);
    hipLaunchKernelGGL(silu_reduce_kernel, grid, dim3(64), 0, st, pg, pu, S, I, h, h_copy, gcount, gcnt,
                       gstride_p, gstride_h);
    return check_hip(hipGetLastError(), "silu_reduce launch");
}

// Measurement hook: when on, each W4 kernel launch gets a run of slots in a
// device buffer, one (start, end) pair of device wall-clock stamps per
// workgroup; a launch's execution interval runs from its earliest start to its
// latest end.  Plain stores to distinct slots, so timing adds no contention.
// The buffer is allocated when the hook is first switched on, never in a
// verify call.
constexpr long kTimingSlots = 1l << 20;  // workgroups recorded between reads
struct W4Timing {
    std::mutex mu;
    bool on = false;
    unsigned long long* slots = nullptr;  // [kTimingSlots][2]
    long used = 0;
    std::vector<long> first, count;  // per launch: first slot, workgroups
    std::vector<double> bytes;       // per launch: algorithmic bytes
};
static W4Timing g_timing;

static double w4_algo_bytes(int nmat, int R, int K, int N, int G) {
    const double w = (double)N * K * 0.5 + 4.0 * (double)N * (K / G);
    return nmat * (w + 2.0 * R * K + 4.0 * R * N);
}

// Fills the plan-derived fields of a W4 launch.
static void prep_w4(W4Args& args, int nmat, const W4Plan& p, int K, int G, int ngroups) {
    args.K = K;
    args.nmat = nmat;
    args.nchunks = p.nchunks;
    args.tiles = w4_tiles(args.N);
    args.cps = p.cps;
    args.S = p.S;
    args.ncg = p.ncg;
    args.ncgb = (p.ncg + kWaves - 1) / kWaves;
    args.blocks = (long)ngroups * nmat * p.S * args.ncgb;
    args.wbytes = (uint32_t)w4_blob_bytes(args.N, K, G);
    if (!args.gexp) args.xbytes = (uint32_t)((size_t)args.R * K * 2);  // grouped: set by the caller
    args.dmask = kDecodeMask;
    args.doff = kDecodeOr;
    args.tstamp = nullptr;
}

// Launches that stream at least kNtBytes of weights load them with the
// non-temporal hint; smaller ones (the decoder's per-layer matrices, read
// again every round) load them plainly.
constexpr double kNtBytes = 32.0 * (1 << 20);
static bool stream_hint(double weight_bytes) { return weight_bytes >= kNtBytes; }

// Timing slots for a launch of `blocks` workgroups moving `bytes` algorithmic
// bytes, or NULL when the hook is off.
static int32_t timing_slots(long blocks, double bytes, unsigned long long** out) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    *out = nullptr;
    if (!g_timing.on) return EV_OK;
    if (g_timing.used + blocks > kTimingSlots)
        return fail(EV_EINVAL, "w4 timing: more than %ld workgroups recorded without a read", kTimingSlots);
    *out = g_timing.slots + 2 * g_timing.used;
    g_timing.first.push_back(g_timing.used);
    g_timing.count.push_back(blocks);
    g_timing.used += blocks;
    g_timing.bytes.push_back(bytes);
    return EV_OK;
}

int32_t launch_w4(W4Args args, int nmat, const W4Plan& p, int K, int G, hipStream_t st, int ngroups) {
    prep_w4(args, nmat, p, K, G, ngroups);
    if (!args.gexp) {  // grouped launches' bytes depend on the routing: not timed
        int32_t rc = timing_slots(args.blocks, w4_algo_bytes(nmat, args.R, K, args.N, G), &args.tstamp);
        if (rc) return rc;
    }
    const unsigned blocks = (unsigned)args.blocks;
    const bool nt = stream_hint((double)args.wbytes * nmat * ngroups);
    if (args.fmt == kNvfp4) {
        if (nt)
            hipLaunchKernelGGL((w4_verify_kernel<64, true, kNvfp4>), dim3(blocks), dim3(kThreads), 0, st, args);
        else
            hipLaunchKernelGGL((w4_verify_kernel<64, false, kNvfp4>), dim3(blocks), dim3(kThreads), 0, st, args);
    } else if (G == 64 && nt)
        hipLaunchKernelGGL((w4_verify_kernel<64, true>), dim3(blocks), dim3(kThreads), 0, st, args);
    else if (G == 64)
        hipLaunchKernelGGL((w4_verify_kernel<64, false>), dim3(blocks), dim3(kThreads), 0, st, args);
    else if (nt)
        hipLaunchKernelGGL((w4_verify_kernel<32, true>), dim3(blocks), dim3(kThreads), 0, st, args);
    else
        hipLaunchKernelGGL((w4_verify_kernel<32, false>), dim3(blocks), dim3(kThreads), 0, st, args);
    return check_hip(hipGetLastError(), "w4_verify_kernel launch");
}

int32_t launch_w4_sk(W4Args args, int nmat, const SkPlan& q, int K, int G, hipStream_t st) {
    if (!q.ok || !args.sk_part || nmat < 1 || nmat > 2 || args.gexp)
        return fail(EV_EINVAL, "w4 balanced launch: unsupported (N=%d K=%d nmat=%d)", args.N, K, nmat);
    args.K = K;
    args.nmat = nmat;
    args.nchunks = w4_chunks(K);
    args.tiles = w4_tiles(args.N);
    args.ncgb = q.ncgb;
    args.blocks = q.nwg;
    args.wbytes = (uint32_t)w4_blob_bytes(args.N, K, G);
    args.xbytes = (uint32_t)((size_t)args.R * K * 2);
    args.dmask = kDecodeMask;
    args.doff = kDecodeOr;
    args.sk_units = q.units;
    args.sk_nwg = q.nwg;
    args.sk_nsc = q.nsc;
    args.sk_segmax = q.segmax;
    args.tstamp = nullptr;
    int32_t rc = timing_slots(q.nwg, w4_algo_bytes(nmat, args.R, K, args.N, G), &args.tstamp);
    if (rc) return rc;
    const bool nt = stream_hint((double)args.wbytes * nmat);
    if (args.fmt == kNvfp4) {
        if (nt)
            hipLaunchKernelGGL((w4_sk_kernel<64, true, kNvfp4>), dim3(q.nwg), dim3(kThreads), 0, st, args);
        else
            hipLaunchKernelGGL((w4_sk_kernel<64, false, kNvfp4>), dim3(q.nwg), dim3(kThreads), 0, st, args);
    } else if (G == 64 && nt)
        hipLaunchKernelGGL((w4_sk_kernel<64, true>), dim3(q.nwg), dim3(kThreads), 0, st, args);
    else if (G == 64)
        hipLaunchKernelGGL((w4_sk_kernel<64, false>), dim3(q.nwg), dim3(kThreads), 0, st, args);
    else if (nt)
        hipLaunchKernelGGL((w4_sk_kernel<32, true>), dim3(q.nwg), dim3(kThreads), 0, st, args);
    else
        hipLaunchKernelGGL((w4_sk_kernel<32, false>), dim3(q.nwg), dim3(kThreads), 0, st, args);
    return check_hip(hipGetLastError(), "w4_sk_kernel launch");
}

// A halved-mode launch: paired gate/up (ncgb = column blocks of kWaves
// tiles) or q|k|v with rotation (ncgb = heads).
static int32_t launch_w4_halved(W4Args args, const W4Plan& p, int K, int G, hipStream_t st, int ngroups,
                                bool rope) {
    args.K = K;
    args.nmat = rope ? 1 : 2;
    args.nchunks = p.nchunks;
    args.tiles = w4_tiles(args.N);
    args.cps = p.cps;
    args.S = 2;
    args.ncg = p.ncg;
    args.ncgb = rope ? args.N / 128 : (p.ncg + kWaves - 1) / kWaves;
    args.blocks = (long)ngroups * args.ncgb;
    args.wbytes = (uint32_t)w4_blob_bytes(args.N, K, G);
    if (!args.gexp) args.xbytes = (uint32_t)((size_t)args.R * K * 2);  // grouped: set by the caller
    args.dmask = kDecodeMask;
    args.doff = kDecodeOr;
    args.tstamp = nullptr;
    if (!args.gexp) {
        int32_t rc = timing_slots(args.blocks, w4_algo_bytes(args.nmat, args.R, K, args.N, G), &args.tstamp);
        if (rc) return rc;
    }
    const unsigned blocks = (unsigned)args.blocks;
    const bool nt = stream_hint((double)args.wbytes * args.nmat * ngroups);
    if (rope) {
        if (G == 64 && nt)
            hipLaunchKernelGGL((w4_pair_kernel<64, kRopeMode, true>), dim3(blocks), dim3(2 * kThreads), 0, st, args);
        else if (G == 64)
            hipLaunchKernelGGL((w4_pair_kernel<64, kRopeMode, false>), dim3(blocks), dim3(2 * kThreads), 0, st, args);
        else if (nt)
            hipLaunchKernelGGL((w4_pair_kernel<32, kRopeMode, true>), dim3(blocks), dim3(2 * kThreads), 0, st, args);
        else
            hipLaunchKernelGGL((w4_pair_kernel<32, kRopeMode, false>), dim3(blocks), dim3(2 * kThreads), 0, st, args);
    } else {
        if (G == 64 && nt)
            hipLaunchKernelGGL((w4_pair_kernel<64, kPairMode, true>), dim3(blocks), dim3(2 * kThreads), 0, st, args);
        else if (G == 64)
            hipLaunchKernelGGL((w4_pair_kernel<64, kPairMode, false>), dim3(blocks), dim3(2 * kThreads), 0, st, args);
        else if (nt)
            hipLaunchKernelGGL((w4_pair_kernel<32, kPairMode, true>), dim3(blocks), dim3(2 * kThreads), 0, st, args);
        else
            hipLaunchKernelGGL((w4_pair_kernel<32, kPairMode, false>), dim3(blocks), dim3(2 * kThreads), 0, st, args);
    }
    return check_hip(hipGetLastError(), "w4 halved-mode launch");
}

// K-parts shapes: 8 waves of up to 2 chunks (K <= 2048), or 16 waves of up
// to 3 (K <= 6144, plain launches).
template <int MODE, int PARTS, int PC>
static void launch_parts_g(const W4Args& args, int G, bool nt, unsigned blocks, hipStream_t st) {
    const dim3 th(64 * PARTS);
    if (G == 64 && nt)
        hipLaunchKernelGGL((w4_parts_kernel<64, MODE, true, PARTS, PC>), dim3(blocks), th, 0, st, args);
    else if (G == 64)
        hipLaunchKernelGGL((w4_parts_kernel<64, MODE, false, PARTS, PC>), dim3(blocks), th, 0, st, args);
    else if (nt)
        hipLaunchKernelGGL((w4_parts_kernel<32, MODE, true, PARTS, PC>), dim3(blocks), th, 0, st, args);
    else
        hipLaunchKernelGGL((w4_parts_kernel<32, MODE, false, PARTS, PC>), dim3(blocks), th, 0, st, args);
}

// A K-parts launch (dense only): one workgroup per tile and K-split (plain),
// per gate/up tile, or four per q|k|v head.  Chunks per workgroup up to 16:
// 8 waves of 2; up to 24: 8 of 3; up to 48: 16 of 3.
static int32_t launch_w4_parts(W4Args args, int K, int G, hipStream_t st, int mode, int S = 1) {
    args.K = K;
    args.nmat = mode == kPairMode ? 2 : 1;
    args.nchunks = w4_chunks(K);
    args.tiles = w4_tiles(args.N);
    args.S = S;
    args.split_stride = (long)16 * args.N;
    const int cpw = (args.nchunks + S - 1) / S;  // chunks per workgroup
    const int shape = cpw <= 16 ? 0 : cpw <= 24 ? 1 : 2;
    const int waves = shape == 2 ? 16 : 8;
    args.cps = (args.nchunks + S * waves - 1) / (S * waves);
    args.blocks = mode == kRopeMode ? 4l * (args.N / 128) : (long)S * args.tiles;
    args.wbytes = (uint32_t)w4_blob_bytes(args.N, K, G);
    args.xbytes = (uint32_t)((size_t)args.R * K * 2);
    args.dmask = kDecodeMask;
    args.doff = kDecodeOr;
    args.tstamp = nullptr;
    int32_t rc = timing_slots(args.blocks, w4_algo_bytes(args.nmat, args.R, K, args.N, G), &args.tstamp);
    if (rc) return rc;
    const unsigned blocks = (unsigned)args.blocks;
    const bool nt = stream_hint((double)args.wbytes * args.nmat);
    if (mode == kRopeMode)
        launch_parts_g<kRopeMode, 8, 2>(args, G, nt, blocks, st);
    else if (mode == kPairMode)
        launch_parts_g<kPairMode, 8, 2>(args, G, nt, blocks, st);
    else if (shape == 2)
        launch_parts_g<kPlain, 16, 3>(args, G, nt, blocks, st);
    else if (shape == 1)
        launch_parts_g<kPlain, 8, 3>(args, G, nt, blocks, st);
    else
        launch_parts_g<kPlain, 8, 2>(args, G, nt, blocks, st);
    return check_hip(hipGetLastError(), "w4 K-parts launch");
}

// Dense halved-mode launches whose K fits 8 runs of 2 chunks take K-parts.
static bool use_parts(int K) { return w4_chunks(K) <= 16; }

bool parts_fits(int K, int S) { return S >= 1 && S <= 4 && (w4_chunks(K) + S - 1) / S <= 48; }

int32_t launch_w4_plain_parts(W4Args args, int K, int G, hipStream_t st, int S) {
    if (!parts_fits(K, S)) return fail(EV_EINVAL, "w4 K-parts launch: K=%d in %d splits (at most 48 chunks each)", K, S);
    return launch_w4_parts(args, K, G, st, kPlain, S);
}

int32_t launch_w4_pair(W4Args args, const W4Plan& p, int K, int G, hipStream_t st, int ngroups) {
    if (ngroups == 1 && !args.gexp && use_parts(K)) return launch_w4_parts(args, K, G, st, kPairMode);
    return launch_w4_halved(args, p, K, G, st, ngroups, false);
}

int32_t launch_w4_rope(W4Args args, const W4Plan& p, int K, int G, hipStream_t st) {
    if (args.N % 128 != 0 || args.N / 128 != args.rope.NH + 2 * args.rope.NKV)
        return fail(EV_EINVAL, "w4 rope launch: N=%d is not (NH + 2 NKV) heads of 128", args.N);
    if (use_parts(K)) return launch_w4_parts(args, K, G, st, kRopeMode);
    return launch_w4_halved(args, p, K, G, st, 1, true);
}

// Workspace of verify_linear_w4: balanced partial segments, or split partials
// [S][16][N] (none if S == 1).
struct LinLayout {
    bool sk;
    SkPlan q;
    W4Plan p;
    size_t total;
};
static LinLayout lin_layout(int K, int N) {
    LinLayout L;
    L.q = plan_w4_sk(N, K, 1);
    L.p = plan_w4(N, K, 1);
    L.sk = use_sk(L.q, L.p);
    L.total = L.sk ? sk_part_bytes(L.q) : (L.p.S > 1 ? (size_t)L.p.S * 16 * N * sizeof(float) : 0);
    return L;
}

// Workspace of the MLP slice: h [16][I] bf16, then the gate/up partials
// (balanced segments of both matrices at off_pg, or split partials [S1][16][I]
// at off_pg and off_pu; none when paired), then the down partials at off_pd
// (balanced segments, or [S2][16][H] if S2 > 1).
struct MlpLayout {
    bool pair, sk1, sk2;
    SkPlan q1, q2;
    W4Plan p1, p2;
    size_t off_pg, off_pu, off_pd, total;
};
static MlpLayout mlp_layout(int H, int I) {
    MlpLayout L;
    L.pair = use_pair(I);
    L.q1 = plan_w4_sk(I, H, 2);
    L.q2 = plan_w4_sk(H, I, 1);
    L.p1 = L.pair ? plan_w4_pair(I, H) : plan_w4(I, H, 2);
    L.p2 = plan_w4(H, I, 1);
    L.sk1 = !L.pair && use_sk(L.q1, L.p1);
    L.sk2 = use_sk(L.q2, L.p2);
    const size_t part1 = L.pair || L.sk1 ? 0 : align256((size_t)L.p1.S * 16 * I * sizeof(float));
    L.off_pg = align256((size_t)16 * I * sizeof(uint16_t));
    L.off_pu = L.off_pg + part1;
    L.off_pd = L.off_pu + (L.sk1 ? align256(sk_part_bytes(L.q1)) : part1);
    L.total = L.off_pd + (L.sk2 ? sk_part_bytes(L.q2) : (L.p2.S > 1 ? (size_t)L.p2.S * 16 * H * sizeof(float) : 0));
    return L;
}

int32_t check_lanes(const char* who, int R) {
    if (R < 1 || R > EV_MAX_LANES) return fail(EV_EINVAL, "%s: R=%d outside 1..16", who, R);
    return EV_OK;
}

int32_t check_ws(const char* who, void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return EV_OK;
    if (!ws || ws_bytes < need)
        return fail(EV_EWORKSPACE, "%s: workspace needs %zu bytes, got %zu", who, need,
                    ws ? ws_bytes : (size_t)0);
    if (!aligned(ws, 256)) return fail(EV_EINVAL, "%s: workspace must be 256-byte aligned", who);
    return EV_OK;
}

bool w4_timing_active() {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    return g_timing.on;
}

}  // namespace ev

using namespace ev;

static void timing_reset() {
    g_timing.used = 0;
    g_timing.first.clear();
    g_timing.count.clear();
    g_timing.bytes.clear();
}

extern "C" int32_t ev_w4_timing(int32_t enable) {
    clear_error();
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (enable && !g_timing.slots) {
        if (hipMalloc(&g_timing.slots, sizeof(unsigned long long) * 2 * kTimingSlots) != hipSuccess)
            return fail(EV_EHIP, "w4 timing: hipMalloc failed");
        timing_reset();
    }
    g_timing.on = enable != 0;
    return EV_OK;
}

extern "C" int32_t ev_w4_timing_read(int64_t* launches, double* total_ms, double* total_bytes) {
    clear_error();
    std::lock_guard<std::mutex> lk(g_timing.mu);
    double ms = 0.0, bytes = 0.0;
    const long n = (long)g_timing.first.size();
    if (n > 0) {
        std::vector<unsigned long long> h(2 * (size_t)g_timing.used);
        int rate_khz = 0, dev = 0;
        if (hipDeviceSynchronize() != hipSuccess ||
            hipMemcpy(h.data(), g_timing.slots, sizeof(unsigned long long) * h.size(), hipMemcpyDeviceToHost) !=
                hipSuccess)
            return fail(EV_EHIP, "ev_w4_timing_read: copy failed");
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || rate_khz <= 0)
            return fail(EV_EHIP, "ev_w4_timing_read: wall clock rate unavailable");
        for (long i = 0; i < n; ++i) {
            unsigned long long t0 = ~0ull, t1 = 0ull;
            for (long w = g_timing.first[i]; w < g_timing.first[i] + g_timing.count[i]; ++w) {
                t0 = std::min(t0, h[2 * w]);
                t1 = std::max(t1, h[2 * w + 1]);
            }
            if (t1 > t0) ms += (double)(t1 - t0) / (double)rate_khz;
            bytes += g_timing.bytes[i];
        }
        timing_reset();
    }
    if (launches) *launches = n;
    if (total_ms) *total_ms = ms;
    if (total_bytes) *total_bytes = bytes;
    return EV_OK;
}

extern "C" int32_t ev_w4_timing_stamps(uint64_t* stamps, int64_t max_pairs, int32_t* counts, int32_t max_launches,
                                       int32_t* n_launches) {
    clear_error();
    std::lock_guard<std::mutex> lk(g_timing.mu);
    const long n = (long)g_timing.first.size();
    if (!stamps || !counts || !n_launches) return fail(EV_EINVAL, "ev_w4_timing_stamps: NULL pointer");
    if (n > max_launches || g_timing.used > max_pairs)
        return fail(EV_EINVAL, "ev_w4_timing_stamps: %ld launches / %ld workgroups recorded, room for %d / %lld", n,
                    g_timing.used, max_launches, (long long)max_pairs);
    if (g_timing.used > 0) {
        if (hipDeviceSynchronize() != hipSuccess ||
            hipMemcpy(stamps, g_timing.slots, sizeof(unsigned long long) * 2 * g_timing.used, hipMemcpyDeviceToHost) !=
                hipSuccess)
            return fail(EV_EHIP, "ev_w4_timing_stamps: copy failed");
    }
    for (long i = 0; i < n; ++i) counts[i] = (int32_t)g_timing.count[i];
    *n_launches = (int32_t)n;
    return EV_OK;
}

// Practical ceiling of a streaming read: the whole grid sweeps the buffer in
// 1 KB wave blocks (wave w reads blocks w, w + nwaves, ..., four in flight),
// as a plain read kernel would; timed by the same per-workgroup stamps.  The
// xor of the data is stored only if it equals a constant, which keeps the
// loads without writing anything in practice.
constexpr int kProbeBlocks = 1024;
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ p, long n16,
                                                         uint32_t* __restrict__ sink,
                                                         unsigned long long* __restrict__ tstamp) {
    if (tstamp && threadIdx.x == 0) tstamp[2 * blockIdx.x] = wall_clock64();
    const long wave = (blockIdx.x * 256l + threadIdx.x) >> 6, nwaves = gridDim.x * 4l;
    const int lane = threadIdx.x & 63;
    uint32_t acc = 0;
    for (long base = wave * 256; base < n16; base += nwaves * 256) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const long i = base + u * 64 + lane;
            v[u] = i < n16 ? p[i] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
    if (tstamp) {
        __syncthreads();
        if (threadIdx.x == 0) tstamp[2 * blockIdx.x + 1] = wall_clock64();
    }
}

extern "C" int32_t ev_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    clear_error();
    if (!buf || !sink) return fail(EV_EINVAL, "ev_read_probe: NULL pointer");
    if (bytes == 0 || bytes % 16 != 0 || !aligned(buf, 16) || !aligned(sink, 4))
        return fail(EV_EINVAL, "ev_read_probe: %zu bytes (a multiple of 16, 16-byte aligned)", bytes);
    unsigned long long* tstamp = nullptr;
    int32_t rc = timing_slots(kProbeBlocks, (double)bytes, &tstamp);
    if (rc) return rc;
    hipLaunchKernelGGL(read_probe_kernel, dim3(kProbeBlocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       reinterpret_cast<const u32x4*>(buf), (long)(bytes / 16), sink, tstamp);
    return check_hip(hipGetLastError(), "read_probe launch");
}

extern "C" size_t verify_linear_w4_workspace(int32_t K, int32_t N, int32_t G) {
    if (K <= 0 || N <= 0 || (G != 32 && G != 64)) return 0;
    return lin_layout(K, N).total;
}

extern "C" int32_t verify_linear_w4(const uint16_t* x, int32_t R, int32_t K, const void* w, int32_t N,
                                    int32_t G, float* y, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    const char* who = "verify_linear_w4";
    int32_t rc;
    if ((rc = check_lanes(who, R)) || (rc = check_w4_dims(who, K, N, G))) return rc;
    if (!x || !w || !y) return fail(EV_EINVAL, "%s: NULL pointer", who);
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 4))
        return fail(EV_EINVAL, "%s: misaligned pointer (x, w 16 B; y 4 B)", who);
    const LinLayout L = lin_layout(K, N);
    if ((rc = check_ws(who, ws, ws_bytes, L.total))) return rc;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    float* part = reinterpret_cast<float*>(ws);
    W4Args a{};
    a.w[0] = a.w[1] = reinterpret_cast<const uint8_t*>(w);
    a.out[0] = a.out[1] = L.p.S > 1 ? part : y;
    a.x = x;
    a.R = R;
    a.N = N;
    if (L.sk) {
        a.sk_part = part;
        if ((rc = launch_w4_sk(a, 1, L.q, K, G, st))) return rc;
        return launch_sk_reduce(part, L.q, 1, N, R, y, nullptr, nullptr, st);
    }
    a.split_stride = L.p.S > 1 ? (long)16 * N : 0;
    if ((rc = launch_w4(a, 1, L.p, K, G, st))) return rc;
    if (L.p.S > 1 && (rc = launch_splitk_reduce(part, L.p.S, N, R, y, st))) return rc;
    return EV_OK;
}

// NVFP4: the same launches as verify_linear_w4 at G = 64 (the tile-chunks have
// that size), with the NVFP4 decode and the tensor scale.
extern "C" size_t verify_linear_nvfp4_workspace(int32_t K, int32_t N) {
    if (K <= 0 || N <= 0) return 0;
    return lin_layout(K, N).total;
}

extern "C" int32_t verify_linear_nvfp4(const uint16_t* x, int32_t R, int32_t K, const void* w, int32_t N,
                                       float tensor_scale, float* y, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    const char* who = "verify_linear_nvfp4";
    int32_t rc;
    // K a multiple of 32 (whole 16-k scale blocks, whole 32-k MFMA steps)
    if ((rc = check_lanes(who, R)) || (rc = check_w4_dims(who, K, N, 32))) return rc;
    if (!(tensor_scale == tensor_scale) || tensor_scale == __builtin_huge_valf() || tensor_scale == -__builtin_huge_valf())
        return fail(EV_EINVAL, "%s: tensor scale must be finite", who);
    if (!x || !w || !y) return fail(EV_EINVAL, "%s: NULL pointer", who);
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 4))
        return fail(EV_EINVAL, "%s: misaligned pointer (x, w 16 B; y 4 B)", who);
    const LinLayout L = lin_layout(K, N);
    if ((rc = check_ws(who, ws, ws_bytes, L.total))) return rc;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    float* part = reinterpret_cast<float*>(ws);
    W4Args a{};
    a.w[0] = a.w[1] = reinterpret_cast<const uint8_t*>(w);
    a.out[0] = a.out[1] = L.p.S > 1 ? part : y;
    a.x = x;
    a.R = R;
    a.N = N;
    a.fmt = kNvfp4;
    a.tscale = tensor_scale;
    if (L.sk) {
        a.sk_part = part;
        if ((rc = launch_w4_sk(a, 1, L.q, K, 64, st))) return rc;
        return launch_sk_reduce(part, L.q, 1, N, R, y, nullptr, nullptr, st);
    }
    a.split_stride = L.p.S > 1 ? (long)16 * N : 0;
    if ((rc = launch_w4(a, 1, L.p, K, 64, st))) return rc;
    if (L.p.S > 1 && (rc = launch_splitk_reduce(part, L.p.S, N, R, y, st))) return rc;
    return EV_OK;
}

extern "C" size_t verify_mlp_w4_workspace(int32_t H, int32_t I, int32_t G) {
    if (H <= 0 || I <= 0 || (G != 32 && G != 64)) return 0;
    return mlp_layout(H, I).total;
}

// Argument checks shared by the MLP entry points (EV_OK or the error code).
static int32_t check_mlp_args(const char* who, const uint16_t* x, int32_t R, int32_t H, int32_t I, int32_t G,
                              const void* w_gate, const void* w_up, const void* w_down, const float* y,
                              const uint16_t* h_out) {
    int32_t rc;
    if ((rc = check_lanes(who, R)) || (rc = check_w4_dims(who, H, I, G)) ||
        (rc = check_w4_dims(who, I, H, G)))
        return rc;
    if (!x || !w_gate || !w_up || !w_down || !y) return fail(EV_EINVAL, "%s: NULL pointer", who);
    if (!aligned(x, 16) || !aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(w_down, 16) ||
        !aligned(y, 4) || (h_out && !aligned(h_out, 16)))
        return fail(EV_EINVAL, "%s: misaligned pointer (x, weights, h 16 B; y 4 B)", who);
    return EV_OK;
}

// The MLP slice's launches on a checked workspace `ws` of at least
// mlp_layout(H, I).total bytes.
static int32_t mlp_launches(const uint16_t* x, int32_t R, int32_t H, int32_t I, int32_t G, const void* w_gate,
                            const void* w_up, const void* w_down, float* y, uint16_t* h_out, void* ws,
                            void* stream) {
    int32_t rc;
    const MlpLayout L = mlp_layout(H, I);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    unsigned char* wsb = reinterpret_cast<unsigned char*>(ws);
    uint16_t* h = reinterpret_cast<uint16_t*>(wsb);
    float* pg = reinterpret_cast<float*>(wsb + L.off_pg);
    float* pu = reinterpret_cast<float*>(wsb + L.off_pu);
    float* pd = reinterpret_cast<float*>(wsb + L.off_pd);
    // h = SiLU(gate) * up (one paired launch, or gate|up + split sum with
    // SiLU * up), then down and its split sum
    W4Args a{};
    a.w[0] = reinterpret_cast<const uint8_t*>(w_gate);
    a.w[1] = reinterpret_cast<const uint8_t*>(w_up);
    a.x = x;
    a.R = R;
    a.N = I;
    if (L.pair) {
        a.h = h;
        a.h_copy = h_out;
        if ((rc = launch_w4_pair(a, L.p1, H, G, st))) return rc;
    } else if (L.sk1) {
        a.sk_part = pg;
        if ((rc = launch_w4_sk(a, 2, L.q1, H, G, st))) return rc;
        if ((rc = launch_sk_reduce(pg, L.q1, 2, I, R, nullptr, h, h_out, st))) return rc;
    } else {
        a.out[0] = pg;
        a.out[1] = pu;
        a.split_stride = (long)16 * I;
        if ((rc = launch_w4(a, 2, L.p1, H, G, st))) return rc;
        if ((rc = launch_silu_reduce(pg, pu, L.p1.S, I, R, h, h_out, 1, nullptr, nullptr, 0, 0, st))) return rc;
    }
    W4Args d{};
    d.w[0] = d.w[1] = reinterpret_cast<const uint8_t*>(w_down);
    d.out[0] = d.out[1] = L.p2.S > 1 ? pd : y;
    d.x = h;
    d.R = R;
    d.N = H;
    if (L.sk2) {
        d.sk_part = pd;
        if ((rc = launch_w4_sk(d, 1, L.q2, I, G, st))) return rc;
        return launch_sk_reduce(pd, L.q2, 1, H, R, y, nullptr, nullptr, st);
    }
    d.split_stride = L.p2.S > 1 ? (long)16 * H : 0;
    if ((rc = launch_w4(d, 1, L.p2, I, G, st))) return rc;
    if (L.p2.S > 1 && (rc = launch_splitk_reduce(pd, L.p2.S, H, R, y, st))) return rc;
    return EV_OK;
}

extern "C" int32_t verify_mlp_w4(const uint16_t* x, int32_t R, int32_t H, int32_t I, int32_t G,
                                 const void* w_gate, const void* w_up, const void* w_down, float* y,
                                 uint16_t* h_out, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    const char* who = "verify_mlp_w4";
    int32_t rc;
    if ((rc = check_mlp_args(who, x, R, H, I, G, w_gate, w_up, w_down, y, h_out))) return rc;
    if ((rc = check_ws(who, ws, ws_bytes, mlp_layout(H, I).total))) return rc;
    return mlp_launches(x, R, H, I, G, w_gate, w_up, w_down, y, h_out, ws, stream);
}

// ---- the same slice for callers that cannot allocate ----------------------
// Its workspace is `scratch`, a device array of the library (one per GPU,
// held until the process ends).  Host code never passes the array's name to a
// kernel: that is a host-side stand-in, not a device address.  The device
// address is looked up once per device with hipGetSymbolAddress and kept.
static __device__ __align__(256) unsigned char scratch[EV_MLP_SCRATCH_BYTES];
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

static int32_t scratch_on_current_device(void** out) {
    int dev = -1;
    int32_t rc;
    if ((rc = check_hip(hipGetDevice(&dev), "hipGetDevice"))) return rc;
    if (dev < 0 || dev >= 64) return fail(EV_EUNSUPPORTED, "device %d: only devices 0..63", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if ((rc = check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "scratch address"))) return rc;
        if (!p) return fail(EV_EHIP, "scratch address: NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return EV_OK;
}

extern "C" int32_t verify_mlp_w4_noalloc(const uint16_t* x, int32_t R, int32_t H, int32_t I, int32_t G,
                                         const void* w_gate, const void* w_up, const void* w_down, float* y,
                                         uint16_t* h_out, void* stream) {
    clear_error();
    const char* who = "verify_mlp_w4_noalloc";
    int32_t rc;
    if ((rc = check_mlp_args(who, x, R, H, I, G, w_gate, w_up, w_down, y, h_out))) return rc;
    const size_t need = mlp_layout(H, I).total;
    if (need > (size_t)EV_MLP_SCRATCH_BYTES)
        return fail(EV_EWORKSPACE, "%s: H=%d I=%d needs %zu bytes of scratch, above the %zu of the library", who,
                    H, I, need, (size_t)EV_MLP_SCRATCH_BYTES);
    void* ws = nullptr;
    if ((rc = scratch_on_current_device(&ws))) return rc;
    return mlp_launches(x, R, H, I, G, w_gate, w_up, w_down, y, h_out, ws, stream);
}
