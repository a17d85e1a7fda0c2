// The W4 verify kernel's launch interface, shared by the dense entry points
// (w4_verify.hip) and the grouped MoE layer (moe.hip).  Internal to
// libexactverify.
#pragma once

#include "ev_internal.h"
#include "w4_layout.h"

namespace ev {

int32_t check_w4_dims(const char* who, int K, int N, int G);

// Tuning constants of the W4 launches (each measured against its neighbours
// on the MLP slice, the LM head and the decoder's matrices).
constexpr int kWaves = 4;            // waves per workgroup, sharing one activation slab
constexpr int kThreads = 64 * kWaves;
constexpr int kNT = 2;               // 16-row tiles per wave
constexpr int kPD = 2;               // chunks of weight loads in flight per wave
constexpr int kSC = 2;               // chunks per activation superchunk (staged in LDS together)
constexpr long kTargetWaves = 4096;  // waves a split plan aims at (four per SIMD)
constexpr int kMinCps = 4;           // at least this many chunks per K-split when K allows

struct W4Plan {
    int S;        // K-splits
    int cps;      // chunks per split
    int nchunks;  // chunks of 128 k
    int ncg;      // tile groups of kNT tiles
    long items;   // waves = nmat * S * ncg
};

// Split plan from (N, K) and the number of matrices of the launch, never R:
// every reduction order of an output element follows from the plan.
inline W4Plan plan_w4(int N, int K, int nmat) {
    W4Plan p;
    p.nchunks = w4_chunks(K);
    p.ncg = (w4_tiles(N) + kNT - 1) / kNT;
    const long base = (long)p.ncg * nmat;
    long S = (kTargetWaves + base - 1) / base;
    long smax = p.nchunks / kMinCps;
    if (smax < 1) smax = 1;
    if (S > smax) S = smax;
    if (S < 1) S = 1;
    p.cps = (int)((p.nchunks + S - 1) / S);
    p.cps = (p.cps + kSC - 1) / kSC * kSC;  // splits start on superchunk boundaries
    p.S = (p.nchunks + p.cps - 1) / p.cps;
    p.items = base * p.S;
    return p;
}

// Balanced (stream-K) plan of a plain launch.  The work of the launch is a
// list of units, one superchunk (kSC chunks of 128 k) of one column block
// (kBlockCols columns: the kWaves * kNT tiles of a workgroup) of one matrix,
// ordered by matrix, block, superchunk; workgroup w of nwg takes units
// [w U / nwg, (w + 1) U / nwg).  nwg is three workgroups of four waves per
// CU (768 on 256 CUs), or U when there are fewer units: about twelve
// streaming waves per CU give this part its best streaming rate (measured:
// five per CU, the register-limited maximum, is 20 % slower, two 7 %).
// Workgroup w writes one partial segment [16][kBlockCols] per block its run
// touches, at slot w * segmax + (block - first block of the run).  All of it
// follows from (N, K, nmat), never from R.
constexpr int kBlockCols = kWaves * kNT * 16;
constexpr int kSkWGs = 256 * 3;  // three workgroups on each of the 256 CUs
struct SkPlan {
    int nsc;     // superchunks per column block
    int ncgb;    // column blocks per matrix
    int nwg;     // workgroups
    int segmax;  // partial segments per workgroup, at most
    int units;   // nmat * ncgb * nsc
    bool ok;     // the unit arithmetic fits 32 bits (units * nwg < 2^31), the segments 4 GiB
};
inline SkPlan plan_w4_sk(int N, int K, int nmat) {
    SkPlan p;
    p.nsc = (w4_chunks(K) + kSC - 1) / kSC;
    p.ncgb = (w4_tiles(N) + kWaves * kNT - 1) / (kWaves * kNT);
    const long U = (long)nmat * p.ncgb * p.nsc;
    const long nwg = U < kSkWGs ? U : kSkWGs;
    p.ok = U * nwg < (1l << 31);
    p.units = (int)U;
    p.nwg = (int)nwg;
    const long L = (U + nwg - 1) / nwg;  // longest run
    p.segmax = (int)((L + p.nsc - 2) / p.nsc + 1);
    // the segments are stored through a buffer descriptor: 32-bit byte range
    p.ok = p.ok && (double)nwg * p.segmax * 16 * kBlockCols * 4 < 4294967296.0;
    return p;
}
// A plain launch runs balanced when its split plan would need partial rows
// anyway (S > 1); a launch whose columns alone fill the chip (S == 1, as the
// LM head) writes its outputs directly and needs no second kernel.
inline bool use_sk(const SkPlan& q, const W4Plan& p) { return q.ok && p.S > 1; }
inline size_t sk_part_bytes(const SkPlan& p) { return (size_t)p.nwg * p.segmax * 16 * kBlockCols * sizeof(float); }

// Geometry of a balanced launch, as the kernels that add its segments need it.
struct SkGeom {
    int U, nwg, nsc, segmax;
};
// The workgroup whose run holds unit u: the largest w with w U / nwg <= u,
// i.e. ceil((u + 1) nwg / U) - 1 (U * nwg < 2^31).
__device__ __forceinline__ int sk_owner(int u, const SkGeom& g) {
    return (int)(((unsigned)(u + 1) * (unsigned)g.nwg + (unsigned)g.U - 1u) / (unsigned)g.U) - 1;
}
// The workgroups whose runs touch block b are first(b) .. last(b) (the owners
// of the block's first and last unit).  Every one after first(b) starts its
// run inside the block, so the block is its segment 0; in first(b) it is
// segment b - start(first(b)) / nsc.
struct SkSpan {
    int w0, w1;
    const float* p0;  // first(b)'s segment, row r, column cl
};
__device__ __forceinline__ SkSpan sk_span(const float* part, const SkGeom& g, int b, int r, int cl) {
    SkSpan sp;
    sp.w0 = sk_owner(b * g.nsc, g);
    sp.w1 = sk_owner((b + 1) * g.nsc - 1, g);
    const int s0 = b - (int)((unsigned)sp.w0 * (unsigned)g.U / (unsigned)g.nwg) / g.nsc;
    sp.p0 = part + (((size_t)sp.w0 * g.segmax + s0) * 16 + r) * kBlockCols + cl;
    return sp;
}
// segment 0 of workgroup w, row r, column cl
__device__ __forceinline__ const float* sk_seg0(const float* part, const SkGeom& g, int w, int r, int cl) {
    return part + ((size_t)w * g.segmax * 16 + r) * kBlockCols + cl;
}
inline SkGeom sk_geom(const SkPlan& q) { return SkGeom{q.units, q.nwg, q.nsc, q.segmax}; }

struct W4Args {
    const uint8_t* w[2];  // packed weights; the workgroup's matrix index picks one
    float* out[2];        // split s writes rows at out + s * split_stride
    const uint16_t* x;    // activations [rows][K] bf16
    int R, K, N, nchunks, tiles;
    int cps, S, ncg, ncgb;  // ncgb: workgroups per (matrix, split), of kWaves tile groups
    int nmat;               // matrices per group (1 or 2)
    long blocks;
    long split_stride;
    uint32_t wbytes, xbytes;
    // nibble-decode constants, passed as arguments so that they sit in
    // registers (gfx9 VOP3 encodings cannot carry 32-bit literals)
    uint32_t dmask, doff;
    // NVFP4 launches: the tensor scale every output is multiplied by
    float tscale;
    int fmt;  // W4Format of the launch
    // measurement: when non-NULL, workgroup b stores the device wall clock at
    // its start in tstamp[2b] and at its end in tstamp[2b + 1]
    unsigned long long* tstamp;
    // Grouped launch (one group per touched MoE expert); gexp == NULL for a
    // plain launch.  Group g (< *gcount, else its workgroups exit at once)
    // streams matrix w[m] + gexp[g] * wstride over rows 0..gcnt[g]-1, whose
    // activations are x rows grows[16 g + r] (grows == NULL: rows 16 g + r),
    // and writes its outputs at out[m] + g * ogstride + split * split_stride.
    const int* gcount;
    const int* gexp;
    const int* gcnt;
    const int* grows;
    long wstride, ogstride;
    // Paired gate/up launch only: h = bf16(silu(gate) * up) rows [R][N] (group
    // g at h + g * hgstride), and a second copy at h_copy when non-NULL.
    uint16_t* h;
    uint16_t* h_copy;
    long hgstride;
    // Balanced launch only: partial segments [nwg][segmax][16][kBlockCols].
    float* sk_part;
    int sk_units, sk_nwg, sk_nsc, sk_segmax;
    // q|k|v launch with rotation only (N = (NH + 2 NKV) * 128 columns, heads
    // q..., k..., v...): row r sits at position positions[kPos0Slot] + r.
    struct {
        const float2* rot;             // [C][64] (cos, sin) per slot
        const long long* positions;    // the step's first position at [kPos0Slot]
        float* q;                      // [R][NH][128] fp32
        uint16_t* kc;                  // [NKV][C][128] fp16
        uint16_t* vc;                  // [NKV][C/32][128][32] fp16, slot order vslot_pos32
        int C, NH, NKV;
    } rope;
};

// Slot of the step's first position in the decoder's positions array (after
// the 16 rows' sampling positions).
constexpr int kPos0Slot = 16;

// Value cache: blocks of 32 slots, d-major inside a block, slot s at position
// vslot_pos32(s): positions 8j..8j+7 hold slots 4j..4j+3 and 16+4j..16+4j+3.
__host__ __device__ inline int vslot_pos32(int s) {
    return s < 16 ? 8 * (s >> 2) + (s & 3) : 8 * ((s - 16) >> 2) + 4 + (s & 3);
}

// Launch the W4 kernel over `ngroups` groups (1 for a plain launch) of
// `nmat` matrices each.  Fills the plan-derived fields of `args`.
int32_t launch_w4(W4Args args, int nmat, const W4Plan& p, int K, int G, hipStream_t st,
                  int ngroups = 1);

// Plan of the paired gate/up launch: K in two halves of cps chunks (a
// multiple of kSC), one workgroup of 2 kWaves waves per kWaves tiles.
inline W4Plan plan_w4_pair(int N, int K) {
    W4Plan p;
    p.nchunks = w4_chunks(K);
    p.ncg = w4_tiles(N);
    const int half = (p.nchunks + 1) / 2;
    p.cps = (half + kSC - 1) / kSC * kSC;
    p.S = 2;
    p.items = 2l * p.ncg;
    return p;
}

// Paired gate/up launch (args.w = {gate, up}, args.h / h_copy / hgstride set):
// h = bf16(silu(x W_gate^T) * (x W_up^T)) for the launch's rows, per group.
int32_t launch_w4_pair(W4Args args, const W4Plan& p, int K, int G, hipStream_t st, int ngroups = 1);

// q|k|v projection with rotation (args.w[0] = the q|k|v matrix, args.rope
// set; plan from plan_w4_pair(N, K)): one workgroup per head.
int32_t launch_w4_rope(W4Args args, const W4Plan& p, int K, int G, hipStream_t st);

// K-parts plain launch (dense, one matrix): y = x W^T in S K-splits (1..4)
// as fp32 rows [S][16][N] at args.out[0] (split stride 16 N), added in
// ascending split order by the consumer; one workgroup per 16-column tile
// and split, whose waves each take a run of K (at most 48 chunks per split:
// parts_fits).
bool parts_fits(int K, int S);
int32_t launch_w4_plain_parts(W4Args args, int K, int G, hipStream_t st, int S);

// A dense gate/up pair (I x H each) runs paired when its tiles alone give the
// target wave count; otherwise as a split launch of both matrices followed by
// silu_reduce, whose extra split waves outweigh the partial rows.
inline bool use_pair(int I) { return 2l * w4_tiles(I) >= kTargetWaves; }

// y[r][n] = sum over s ascending of part[s][r][n] (split stride 16 * N), r < R.
int32_t launch_splitk_reduce(const float* part, int S, int N, int R, float* y, hipStream_t st);

// h[r][k] = bf16_rne(silu(sum_s pg[s][r][k]) * sum_s pu[s][r][k]) for rows
// r < R, splits added in ascending s (split stride 16 * I).  Grouped when gcnt
// != NULL: group g < *gcount (grid z) covers rows < gcnt[g] at offsets
// g * gstride_p (partials) and g * gstride_h (h).
int32_t launch_silu_reduce(const float* pg, const float* pu, int S, int I, int R, uint16_t* h,
                           uint16_t* h_copy, int ngroups, const int* gcount, const int* gcnt,
                           long gstride_p, long gstride_h, hipStream_t st);

// Balanced launch of nmat (1 or 2) matrices (args.sk_part set, plan from
// plan_w4_sk(N, K, nmat)); then launch_sk_reduce.
int32_t launch_w4_sk(W4Args args, int nmat, const SkPlan& q, int K, int G, hipStream_t st);

// After a balanced launch: nmat == 1: y[r][n] = the sum of the segments of
// column n's block, in ascending workgroup order, for r < R (y [R][N] fp32);
// nmat == 2 (gate, up): h[r][k] = bf16_rne(silu(g) * u) of the two sums (h and
// h_copy [R][N] bf16, h_copy may be NULL).
int32_t launch_sk_reduce(const float* part, const SkPlan& q, int nmat, int N, int R, float* y, uint16_t* h,
                         uint16_t* h_copy, hipStream_t st);

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int32_t check_lanes(const char* who, int R);

// True while the per-workgroup timing hook records W4 launches.
bool w4_timing_active();
int32_t check_ws(const char* who, void* ws, size_t ws_bytes, size_t need);

}  // namespace ev
