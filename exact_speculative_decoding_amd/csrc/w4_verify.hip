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
// Kernel shape: every wave is an independent work item (no LDS, no barriers):
// kNT 16-column MFMA tiles over one K-split of `cps` chunks of 128.
//   * A operand = the 16 activation rows (rows >= R read as zero through the
//     buffer range check), loaded per 32-k step straight from L2, each 8-element
//     group reordered [0,4,1,5,2,6,3,7] to match the nibble decode;
//   * B operand = 16 columns of packed nibbles: each lane streams 16 B of one
//     row per tile per chunk (a wave load covers 16 rows x 64 B), and a 4x4
//     dword transpose across the four 16-lane rows (v_permlane32_swap /
//     v_permlane16_swap) turns them into per-step fragments;
//   * nibbles decode exactly into bf16 as 16 + q (0x4180 | q << 3: a shift and
//     an and-or per pair); one more MFMA against an all-ones B gives the group
//     sum xs of every row, and the fold is p += s * acc + (b - 16 s) * xs into
//     a per-chunk partial p that is added to y once per chunk;
//   * a ring of kPD chunks of loads is kept in flight per wave; all loads are
//     buffer loads, so out-of-range rows/columns read zero without branches;
//   * K-split partial sums go to a workspace [S][16][N] and are added in
//     ascending split order by a second kernel (fused with SiLU * up for the
//     MLP gate/up pair).
#include <mutex>
#include <vector>

#include "ev_internal.h"

#ifndef EV_W4_NT
#define EV_W4_NT 4  // 16-column tiles per wave
#endif
#ifndef EV_W4_PD
#define EV_W4_PD 2  // chunks of loads in flight per wave
#endif
#ifndef EV_W4_TARGET_WAVES
#define EV_W4_TARGET_WAVES 2048
#endif
#ifndef EV_W4_MIN_CPS
#define EV_W4_MIN_CPS 8  // at least this many chunks per K-split when K allows
#endif

namespace ev {

constexpr int kThreads = 256;  // 4 independent waves per workgroup
constexpr int kNT = EV_W4_NT;
constexpr int kPD = EV_W4_PD;
constexpr int kWaveCols = 16 * kNT;
constexpr int kKC = 128;  // k per chunk (4 MFMA steps of 32)
constexpr uint32_t kOOB = 0x80000000u;  // offset beyond every buffer: reads 0

struct W4Plan {
    int S;        // K-splits
    int cps;      // chunks per split
    int nchunks;  // ceil(K / 128)
    int ncg;      // column groups of kWaveCols
    long items;   // waves = nmat * S * ncg
};

// Split plan from (N, K) and the number of matrices of the launch, never R.
static W4Plan plan_w4(int N, int K, int nmat) {
    W4Plan p;
    p.nchunks = (K + kKC - 1) / kKC;
    p.ncg = (N + kWaveCols - 1) / kWaveCols;
    const long base = (long)p.ncg * nmat;
    long S = (EV_W4_TARGET_WAVES + base - 1) / base;
    long smax = p.nchunks / EV_W4_MIN_CPS;
    if (smax < 1) smax = 1;
    if (S > smax) S = smax;
    if (S < 1) S = 1;
    p.cps = (int)((p.nchunks + S - 1) / S);
    p.S = (p.nchunks + p.cps - 1) / p.cps;
    p.items = base * p.S;
    return p;
}

struct W4Mat {
    const uint8_t* q;
    const uint16_t* s;
    const uint16_t* b;
    float* out;  // split s writes rows at out + s * split_stride
};

struct W4Args {
    W4Mat m[2];  // the item's matrix index picks one (gate/up share one launch)
    const uint16_t* x;
    int R, K, N;
    int nchunks, cps, S, ncg;
    long items;
    long split_stride;  // floats between consecutive splits' outputs
    // nibble-decode constants, passed as arguments so that they sit in
    // registers (gfx9 VOP3 encodings cannot carry 32-bit literals)
    uint32_t dmask, doff;
};

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// voff: per-lane byte offset; soff: wave-uniform byte offset (scalar register)
__device__ __forceinline__ u32x4 bload128(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t bload32(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint16_t bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

// Eight nibbles q0..q7 (q_i in bits 4i..4i+3) -> four bf16 pairs holding
// 16 + q in the order (q0,q4) (q1,q5) (q2,q6) (q3,q7).  Exact.
__device__ __forceinline__ u32x4 decode_nibbles(uint32_t d, uint32_t m, uint32_t off) {
    u32x4 r;
    r[0] = ((d << 3) & m) | off;
    r[1] = ((d >> 1) & m) | off;
    r[2] = ((d >> 5) & m) | off;
    r[3] = ((d >> 9) & m) | off;
    return r;
}

// Eight bf16 x0..x7 (natural order) -> (x0,x4) (x1,x5) (x2,x6) (x3,x7), one
// byte permute per output dword.
__device__ __forceinline__ u32x4 reorder_x(u32x4 v) {
    u32x4 o;
    o[0] = __builtin_amdgcn_perm(v[2], v[0], 0x05040100u);
    o[1] = __builtin_amdgcn_perm(v[2], v[0], 0x07060302u);
    o[2] = __builtin_amdgcn_perm(v[3], v[1], 0x05040100u);
    o[3] = __builtin_amdgcn_perm(v[3], v[1], 0x07060302u);
    return o;
}

// 4x4 transpose of dwords across the four 16-lane rows of a wave: afterwards
// register t of row j holds what register j of row t held.
__device__ __forceinline__ void transpose_rows(u32x4& v) {
    uint32_t d0 = v[0], d1 = v[1], d2 = v[2], d3 = v[3];
    auto a = __builtin_amdgcn_permlane32_swap(d0, d2, false, false);
    d0 = a[0];
    d2 = a[1];
    auto b = __builtin_amdgcn_permlane32_swap(d1, d3, false, false);
    d1 = b[0];
    d3 = b[1];
    auto c = __builtin_amdgcn_permlane16_swap(d0, d1, false, false);
    d0 = c[0];
    d1 = c[1];
    auto e = __builtin_amdgcn_permlane16_swap(d2, d3, false, false);
    d2 = e[0];
    d3 = e[1];
    v[0] = d0;
    v[1] = d1;
    v[2] = d2;
    v[3] = d3;
}

__device__ __forceinline__ float half_lo(uint32_t w) { return f16_to_f32((uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float half_hi(uint32_t w) { return f16_to_f32((uint16_t)(w >> 16)); }

// ALIGNED: K % 128 == 0 -- every chunk is whole, and a chunk's GPC scales (or
// biases) of one row are one aligned 4 B (G = 64) or 8 B (G = 32) word.
template <int G, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void w4_verify_kernel(W4Args a) {
    constexpr int GPC = kKC / G;        // groups per chunk
    constexpr int SBW = ALIGNED ? GPC / 2 : GPC;  // s/b words per chunk (b32 or b16)
    const int lane = threadIdx.x & 63;
    // wave-uniform work item (readfirstlane keeps it, the matrix and the buffer
    // descriptors in scalar registers)
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const long item = (long)blockIdx.x * (kThreads / 64) + wave;
    if (item >= a.items) return;  // whole wave
    const int ln = lane & 15, j = lane >> 4;
    const int cg = (int)(item % a.ncg);
    const long rest = item / a.ncg;
    const int split = (int)(rest % a.S);
    const int mi = (int)(rest / a.S);
    const W4Mat mat = a.m[mi];
    const int c0 = split * a.cps;
    const int c1 = min(a.nchunks, c0 + a.cps);
    const int K = a.K, N = a.N;
    const uint32_t Kh = (uint32_t)K >> 1;
    const uint32_t KG = (uint32_t)(K / G);

    const rsrc_t rq = make_rsrc(mat.q, (uint32_t)((size_t)N * Kh));
    const rsrc_t rs = make_rsrc(mat.s, (uint32_t)((size_t)N * KG * 2));
    const rsrc_t rb = make_rsrc(mat.b, (uint32_t)((size_t)N * KG * 2));
    const rsrc_t rx = make_rsrc(a.x, (uint32_t)((size_t)a.R * K * 2));

    int ncol[kNT];
    uint32_t qoff[kNT], soff[kNT];
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
        ncol[t] = cg * kWaveCols + t * 16 + ln;
        const bool ok = ncol[t] < N;
        qoff[t] = ok ? (uint32_t)ncol[t] * Kh + 16u * j : kOOB;
        soff[t] = ok ? (uint32_t)ncol[t] * KG * 2u : kOOB;
    }
    const uint32_t xoff = ln < a.R ? ((uint32_t)ln * K + 8u * j) * 2u : kOOB;
    // the mask stays scalar, the or-constant goes to a vector register: gfx9
    // VALU ops read at most one scalar operand, and this lets each decoded pair
    // be one v_and_or_b32
    const uint32_t dm = a.dmask;
    uint32_t doff;
    asm volatile("v_mov_b32 %0, %1" : "=v"(doff) : "s"(a.doff));

    // register ring of kPD chunks
    u32x4 qr[kPD][kNT];
    uint32_t sr[kPD][kNT][SBW], br[kPD][kNT][SBW];
    u32x4 xr[kPD][4];

    // Loads of chunk c into ring slot `slot`.  The chunk's offset is a scalar
    // (soffset); chunks at or past c1 use an out-of-range scalar offset
    // (zeros, no memory traffic), so every slot is written on every path and
    // the ring never has to be copied.
    auto fetch = [&](int c, int slot) {
        const bool live = c < c1;
        const uint32_t kc = (uint32_t)c * kKC;
        const uint32_t sq = live ? (kc >> 1) : kOOB;
        const uint32_t ss = live ? (kc / G) * 2u : kOOB;
        const uint32_t sx = live ? kc * 2u : kOOB;
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
            uint32_t vq = qoff[t];
            if (!ALIGNED && kc + 32u * j >= (uint32_t)K) vq = kOOB;
            qr[slot][t] = bload128(rq, vq, sq);
#pragma unroll
            for (int w = 0; w < SBW; ++w) {
                if (ALIGNED) {
                    sr[slot][t][w] = bload32(rs, soff[t] + 4u * w, ss);
                    br[slot][t][w] = bload32(rb, soff[t] + 4u * w, ss);
                } else {
                    uint32_t so = soff[t] + 2u * w;
                    if (kc + (uint32_t)(w * G) >= (uint32_t)K) so = kOOB;
                    sr[slot][t][w] = bload16(rs, so, ss);
                    br[slot][t][w] = bload16(rb, so, ss);
                }
            }
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) xr[slot][st] = bload128(rx, xoff + 64u * st, sx);
    };

    const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    f32x4 y[kNT];
#pragma unroll
    for (int t = 0; t < kNT; ++t) y[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One chunk: per 32-k step, one MFMA for the group sums of x and one per
    // tile; per group, p += s * acc + (b - 16 s) * xs into a chunk partial p,
    // which is added to y once per chunk.
    auto compute = [&](int c, int slot) {
        const int nst = ALIGNED ? 4 : min(4, (K - c * kKC) >> 5);
#pragma unroll
        for (int t = 0; t < kNT; ++t) transpose_rows(qr[slot][t]);
        f32x4 acc[kNT], part[kNT], xs = {0.f, 0.f, 0.f, 0.f};
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < kNT; ++t) part[t] = zero;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            if (ALIGNED || st < nst) {
                const bf16x8 A = __builtin_bit_cast(bf16x8, reorder_x(xr[slot][st]));
                const bool first = (G == 32) || ((st & 1) == 0);
                xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, ones),
                                                            first ? zero : xs, 0, 0, 0);
#pragma unroll
                for (int t = 0; t < kNT; ++t) {
                    const bf16x8 B =
                        __builtin_bit_cast(bf16x8, decode_nibbles(qr[slot][t][st], dm, doff));
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, first ? zero : acc[t], 0, 0, 0);
                }
                const bool last = (G == 32) || ((st & 1) == 1);
                if (last) {
                    const int gc = (32 * st) / G;  // group within the chunk
#pragma unroll
                    for (int t = 0; t < kNT; ++t) {
                        float sv, bv;
                        if (ALIGNED) {
                            const uint32_t sw = sr[slot][t][gc >> 1], bw = br[slot][t][gc >> 1];
                            sv = (gc & 1) ? half_hi(sw) : half_lo(sw);
                            bv = (gc & 1) ? half_hi(bw) : half_lo(bw);
                        } else {
                            sv = f16_to_f32((uint16_t)sr[slot][t][gc]);
                            bv = f16_to_f32((uint16_t)br[slot][t][gc]);
                        }
                        const float bp = fmaf(-16.f, sv, bv);  // removes the decode offset
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            part[t][i] = fmaf(sv, acc[t][i], part[t][i]);
                            part[t][i] = fmaf(bp, xs[i], part[t][i]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < kNT; ++t) y[t] += part[t];
    };

    // sched_barrier keeps each refill where it is written, so the loads of the
    // other ring slots stay in flight across the compute of this one.
#pragma unroll
    for (int p = 0; p < kPD; ++p) {
        __builtin_amdgcn_sched_barrier(0);
        fetch(c0 + p, p);
    }
    for (int cb = c0; cb < c1; cb += kPD) {
#pragma unroll
        for (int p = 0; p < kPD; ++p) {
            __builtin_amdgcn_sched_barrier(0);
            compute(cb + p, p);
            __builtin_amdgcn_sched_barrier(0);
            fetch(cb + p + kPD, p);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // rows r = 4j + i of columns ncol[t]
    float* out = mat.out + (size_t)split * a.split_stride;
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
        if (ncol[t] < N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * j + i;
                if (r < a.R) out[(size_t)r * N + ncol[t]] = y[t][i];
            }
        }
    }
}

// y[r][n] = sum over s = 0..S-1, ascending, of part[s][r][n].
__global__ void splitk_reduce_kernel(const float* __restrict__ part, int S, int N,
                                     float* __restrict__ y) {
    const int n = blockIdx.x * 256 + threadIdx.x;
    const int r = blockIdx.y;
    if (n >= N) return;
    const size_t stride = (size_t)16 * N;
    float acc = part[(size_t)r * N + n];
    for (int s = 1; s < S; ++s) acc += part[s * stride + (size_t)r * N + n];
    y[(size_t)r * N + n] = acc;
}

// g, u = split sums (ascending s); h = bf16_rne(silu(g) * u).
__global__ void silu_reduce_kernel(const float* __restrict__ pg, const float* __restrict__ pu,
                                   int S, int I, uint16_t* __restrict__ h,
                                   uint16_t* __restrict__ h_copy) {
    const int n = blockIdx.x * 256 + threadIdx.x;
    const int r = blockIdx.y;
    if (n >= I) return;
    const size_t stride = (size_t)16 * I;
    const size_t o = (size_t)r * I + n;
    float g = pg[o], u = pu[o];
    for (int s = 1; s < S; ++s) {
        g += pg[s * stride + o];
        u += pu[s * stride + o];
    }
    const float sg = g / (1.0f + expf(-g));
    const uint16_t hb = f32_to_bf16_rne(sg * u);
    h[o] = hb;
    if (h_copy) h_copy[o] = hb;
}

// Measurement hook: when on, each W4 kernel launch is bracketed by HIP events
// on its own stream, with the launch's algorithmic bytes (weights, x, y).
struct W4Timing {
    std::mutex mu;
    bool on = false;
    struct Rec { hipEvent_t a, b; double bytes; };
    std::vector<Rec> recs;
};
static W4Timing g_timing;

static double w4_algo_bytes(int nmat, int R, int K, int N, int G) {
    const double w = (double)N * K * 0.5 + 4.0 * (double)N * (K / G);
    return nmat * (w + 2.0 * R * K + 4.0 * R * N);
}

static int32_t launch_w4(W4Args args, int nmat, const W4Plan& p, int G, hipStream_t st) {
    args.nchunks = p.nchunks;
    args.cps = p.cps;
    args.S = p.S;
    args.ncg = p.ncg;
    args.items = p.items;
    args.dmask = 0x00780078u;
    args.doff = 0x41804180u;
    const unsigned blocks = (unsigned)((p.items + 3) / 4);
    const bool aligned_k = args.K % kKC == 0;
    hipEvent_t ea = nullptr, eb = nullptr;
    bool timed;
    {
        std::lock_guard<std::mutex> lk(g_timing.mu);
        timed = g_timing.on;
    }
    if (timed) {
        if (hipEventCreate(&ea) != hipSuccess || hipEventCreate(&eb) != hipSuccess)
            return fail(EV_EHIP, "w4 timing: hipEventCreate failed");
        if (hipEventRecord(ea, st) != hipSuccess) return fail(EV_EHIP, "w4 timing: record failed");
    }
    if (G == 64) {
        if (aligned_k)
            hipLaunchKernelGGL((w4_verify_kernel<64, true>), dim3(blocks), dim3(kThreads), 0, st, args);
        else
            hipLaunchKernelGGL((w4_verify_kernel<64, false>), dim3(blocks), dim3(kThreads), 0, st, args);
    } else {
        if (aligned_k)
            hipLaunchKernelGGL((w4_verify_kernel<32, true>), dim3(blocks), dim3(kThreads), 0, st, args);
        else
            hipLaunchKernelGGL((w4_verify_kernel<32, false>), dim3(blocks), dim3(kThreads), 0, st, args);
    }
    int32_t rc = check_hip(hipGetLastError(), "w4_verify_kernel launch");
    if (timed) {
        if (hipEventRecord(eb, st) != hipSuccess) return fail(EV_EHIP, "w4 timing: record failed");
        std::lock_guard<std::mutex> lk(g_timing.mu);
        g_timing.recs.push_back({ea, eb, w4_algo_bytes(nmat, args.R, args.K, args.N, G)});
    }
    return rc;
}

static int32_t check_w4_shape(const char* who, int R, int K, int N, int G) {
    if (R < 1 || R > EV_MAX_LANES) return fail(EV_EINVAL, "%s: R=%d outside 1..16", who, R);
    if ((long long)N * (K / 2) >= (1LL << 31) || (long long)EV_MAX_LANES * K * 2 >= (1LL << 31))
        return fail(EV_EUNSUPPORTED, "%s: N*K/2 must stay below 2^31 bytes", who);
    if (G != 32 && G != 64) return fail(EV_EUNSUPPORTED, "%s: group size %d (32 or 64)", who, G);
    if (K <= 0 || N <= 0) return fail(EV_EINVAL, "%s: K=%d N=%d must be positive", who, K, N);
    if (K % G != 0 || K % 32 != 0)
        return fail(EV_EINVAL, "%s: K=%d must be a multiple of 32 and of G=%d", who, K, G);
    return EV_OK;
}

static int32_t check_w4_ptrs(const char* who, const void* q, const void* s, const void* b) {
    if (!q || !s || !b) return fail(EV_EINVAL, "%s: NULL weight pointer", who);
    if (!aligned(q, 16)) return fail(EV_EINVAL, "%s: q must be 16-byte aligned", who);
    if (!aligned(s, 2) || !aligned(b, 2)) return fail(EV_EINVAL, "%s: scale/bias must be 2-byte aligned", who);
    return EV_OK;
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace ev

using namespace ev;

extern "C" int32_t ev_w4_timing(int32_t enable) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    g_timing.on = enable != 0;
    return EV_OK;
}

extern "C" int32_t ev_w4_timing_read(int64_t* launches, double* total_ms, double* total_bytes) {
    clear_error();
    std::vector<W4Timing::Rec> recs;
    {
        std::lock_guard<std::mutex> lk(g_timing.mu);
        recs.swap(g_timing.recs);
    }
    double ms = 0.0, bytes = 0.0;
    int32_t rc = EV_OK;
    for (auto& r : recs) {
        float t = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
            rc = fail(EV_EHIP, "ev_w4_timing_read: event query failed");
        ms += t;
        bytes += r.bytes;
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    if (launches) *launches = (int64_t)recs.size();
    if (total_ms) *total_ms = ms;
    if (total_bytes) *total_bytes = bytes;
    return rc;
}

extern "C" size_t verify_linear_w4_workspace(int32_t K, int32_t N, int32_t G) {
    if (K <= 0 || N <= 0 || (G != 32 && G != 64)) return 0;
    const W4Plan p = plan_w4(N, K, 1);
    return p.S > 1 ? (size_t)p.S * 16 * (size_t)N * sizeof(float) : 0;
}

extern "C" int32_t verify_linear_w4(const uint16_t* x, int32_t R, int32_t K, const uint8_t* q,
                                    const uint16_t* s, const uint16_t* b, int32_t N, int32_t G,
                                    float* y, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    const char* who = "verify_linear_w4";
    int32_t rc = check_w4_shape(who, R, K, N, G);
    if (rc) return rc;
    if ((rc = check_w4_ptrs(who, q, s, b))) return rc;
    if (!x || !y) return fail(EV_EINVAL, "%s: NULL x or y", who);
    if (!aligned(x, 16)) return fail(EV_EINVAL, "%s: x must be 16-byte aligned", who);
    if (!aligned(y, 4)) return fail(EV_EINVAL, "%s: y must be 4-byte aligned", who);
    const W4Plan p = plan_w4(N, K, 1);
    const size_t need = verify_linear_w4_workspace(K, N, G);
    if (need > 0) {
        if (!ws || ws_bytes < need)
            return fail(EV_EWORKSPACE, "%s: workspace needs %zu bytes, got %zu", who, need,
                        ws ? ws_bytes : (size_t)0);
        if (!aligned(ws, 16)) return fail(EV_EINVAL, "%s: workspace must be 16-byte aligned", who);
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    W4Args a{};
    a.m[0] = W4Mat{q, s, b, p.S > 1 ? reinterpret_cast<float*>(ws) : y};
    a.m[1] = a.m[0];
    a.x = x;
    a.R = R;
    a.K = K;
    a.N = N;
    a.split_stride = p.S > 1 ? (long)16 * N : 0;
    if ((rc = launch_w4(a, 1, p, G, st))) return rc;
    if (p.S > 1) {
        dim3 grid((unsigned)((N + 255) / 256), (unsigned)R);
        hipLaunchKernelGGL(splitk_reduce_kernel, grid, dim3(256), 0, st,
                           reinterpret_cast<const float*>(ws), p.S, N, y);
        if ((rc = check_hip(hipGetLastError(), "splitk_reduce launch"))) return rc;
    }
    return EV_OK;
}

// Workspace layout of the MLP slice: gate partials [S1][16][I] f32, up partials
// [S1][16][I] f32, h [16][I] bf16, down partials [S2][16][H] f32 (if S2 > 1).
struct MlpLayout {
    W4Plan p1, p2;
    size_t off_pu, off_h, off_pd, total;
};

static MlpLayout mlp_layout(int H, int I) {
    MlpLayout L;
    L.p1 = plan_w4(I, H, 2);
    L.p2 = plan_w4(H, I, 1);
    const size_t part1 = align256((size_t)L.p1.S * 16 * I * sizeof(float));
    L.off_pu = part1;
    L.off_h = 2 * part1;
    L.off_pd = L.off_h + align256((size_t)16 * I * sizeof(uint16_t));
    L.total = L.off_pd + (L.p2.S > 1 ? (size_t)L.p2.S * 16 * H * sizeof(float) : 0);
    return L;
}

extern "C" size_t verify_mlp_w4_workspace(int32_t H, int32_t I, int32_t G) {
    if (H <= 0 || I <= 0 || (G != 32 && G != 64)) return 0;
    return mlp_layout(H, I).total;
}

extern "C" int32_t verify_mlp_w4(const uint16_t* x, int32_t R, int32_t H, int32_t I, int32_t G,
                                 const uint8_t* gq, const uint16_t* gs, const uint16_t* gb,
                                 const uint8_t* uq, const uint16_t* us, const uint16_t* ub,
                                 const uint8_t* dq, const uint16_t* ds, const uint16_t* db,
                                 float* y, uint16_t* h_out, void* ws, size_t ws_bytes,
                                 void* stream) {
    clear_error();
    const char* who = "verify_mlp_w4";
    int32_t rc = check_w4_shape(who, R, H, I, G);
    if (rc) return rc;
    if ((rc = check_w4_shape(who, R, I, H, G))) return rc;
    if ((rc = check_w4_ptrs(who, gq, gs, gb)) || (rc = check_w4_ptrs(who, uq, us, ub)) ||
        (rc = check_w4_ptrs(who, dq, ds, db)))
        return rc;
    if (!x || !y) return fail(EV_EINVAL, "%s: NULL x or y", who);
    if (!aligned(x, 16)) return fail(EV_EINVAL, "%s: x must be 16-byte aligned", who);
    if (!aligned(y, 4) || (h_out && !aligned(h_out, 2)))
        return fail(EV_EINVAL, "%s: misaligned y or h", who);
    const MlpLayout L = mlp_layout(H, I);
    if (!ws || ws_bytes < L.total)
        return fail(EV_EWORKSPACE, "%s: workspace needs %zu bytes, got %zu", who, L.total,
                    ws ? ws_bytes : (size_t)0);
    if (!aligned(ws, 256)) return fail(EV_EINVAL, "%s: workspace must be 256-byte aligned", who);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    unsigned char* w = reinterpret_cast<unsigned char*>(ws);
    float* pg = reinterpret_cast<float*>(w);
    float* pu = reinterpret_cast<float*>(w + L.off_pu);
    uint16_t* h = reinterpret_cast<uint16_t*>(w + L.off_h);
    float* pd = reinterpret_cast<float*>(w + L.off_pd);

    // gate and up: one launch, blockIdx.z picks the matrix; always via partials
    W4Args a{};
    a.m[0] = W4Mat{gq, gs, gb, pg};
    a.m[1] = W4Mat{uq, us, ub, pu};
    a.x = x;
    a.R = R;
    a.K = H;
    a.N = I;
    a.split_stride = (long)16 * I;
    if ((rc = launch_w4(a, 2, L.p1, G, st))) return rc;
    {
        dim3 grid((unsigned)((I + 255) / 256), (unsigned)R);
        hipLaunchKernelGGL(silu_reduce_kernel, grid, dim3(256), 0, st, pg, pu, L.p1.S, I, h, h_out);
        if ((rc = check_hip(hipGetLastError(), "silu_reduce launch"))) return rc;
    }
    // down
    W4Args d{};
    d.m[0] = W4Mat{dq, ds, db, L.p2.S > 1 ? pd : y};
    d.m[1] = d.m[0];
    d.x = h;
    d.R = R;
    d.K = I;
    d.N = H;
    d.split_stride = L.p2.S > 1 ? (long)16 * H : 0;
    if ((rc = launch_w4(d, 1, L.p2, G, st))) return rc;
    if (L.p2.S > 1) {
        dim3 grid((unsigned)((H + 255) / 256), (unsigned)R);
        hipLaunchKernelGGL(splitk_reduce_kernel, grid, dim3(256), 0, st, pd, L.p2.S, H, y);
        if ((rc = check_hip(hipGetLastError(), "splitk_reduce launch"))) return rc;
    }
    return EV_OK;
}
