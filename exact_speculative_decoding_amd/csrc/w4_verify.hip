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
// the split of K over workgroups, and therefore every reduction order, is a
// function of (N, K, G) only.
//
// Kernel shape (per workgroup of 4 waves):
//   * 128 output columns (each wave: two 16-column MFMA tiles) over one K-split
//     of up to 14 chunks of 128;
//   * the split's activations for all 16 rows sit in LDS, each 8-element group
//     reordered [0,4,1,5,2,6,3,7] to match the nibble decode below;
//   * each lane streams 16 B of packed nibbles per tile per chunk (one 64 B run
//     per row per wave load), a 4x4 dword transpose across the four 16-lane
//     rows (v_permlane32_swap / v_permlane16_swap) turns them into MFMA B
//     fragments;
//   * nibbles decode exactly into bf16 as 16 + q (bits 0x4180 | q << 3: a shift
//     and an and-or per pair); the offset is removed per group with the group
//     sum of x, so y = sum_g s_g * (acc_g - 16 * xs_g) + b_g * xs_g;
//   * partial sums of K-splits go to a workspace [S][16][N] and are added in
//     ascending split order by a second kernel (fused with SiLU * up for the
//     MLP gate/up pair).
#include <mutex>
#include <vector>

#include "ev_internal.h"

namespace ev {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kNT = 2;                  // 16-column tiles per wave
constexpr int kBN = kWaves * kNT * 16;  // 128 columns per workgroup
constexpr int kKC = 128;                // k per chunk (4 MFMA steps of 32)
constexpr int kMaxCps = 14;             // chunks per split: LDS slab <= 1792 k
constexpr int kXPad = 8;                // bf16 pad per LDS row (bank skew)
constexpr int kTargetBlocks = 512;      // aim: >= 2 workgroups per CU

struct W4Plan {
    int S;        // K-splits
    int cps;      // chunks per split
    int nchunks;  // ceil(K / 128)
};

// Split plan from the column count of the launch and K only (never R).
static W4Plan plan_w4(long ncols, int K) {
    W4Plan p;
    p.nchunks = (K + kKC - 1) / kKC;
    long ncb = (ncols + kBN - 1) / kBN;
    long S = (kTargetBlocks + ncb - 1) / ncb;
    if (S < 1) S = 1;
    long smin = (p.nchunks + kMaxCps - 1) / kMaxCps;
    if (S < smin) S = smin;
    if (S > p.nchunks) S = p.nchunks;
    p.cps = (int)((p.nchunks + S - 1) / S);
    p.S = (p.nchunks + p.cps - 1) / p.cps;
    return p;
}

static size_t w4_lds_bytes(const W4Plan& p, int G) {
    size_t kb = (size_t)p.cps * kKC;
    return 16 * (kb + kXPad) * sizeof(uint16_t) + (kb / G) * 16 * sizeof(float);
}

struct W4Mat {
    const uint8_t* q;
    const uint16_t* s;
    const uint16_t* b;
    float* out;  // split s writes rows at out + s * split_stride
};

struct W4Args {
    W4Mat m[2];  // blockIdx.z selects the matrix (gate/up share one launch)
    const uint16_t* x;
    int R, K, N;
    int nchunks, cps;
    long split_stride;  // floats between consecutive splits' outputs
};

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Eight nibbles q0..q7 (q_i in bits 4i..4i+3) -> four bf16 pairs holding
// 16 + q in the order (q0,q4) (q1,q5) (q2,q6) (q3,q7).  Exact.
__device__ __forceinline__ u32x4 decode_nibbles(uint32_t d) {
    const uint32_t m = 0x00780078u, off = 0x41804180u;
    u32x4 r;
    r[0] = ((d << 3) & m) | off;
    r[1] = ((d >> 1) & m) | off;
    r[2] = ((d >> 5) & m) | off;
    r[3] = ((d >> 9) & m) | off;
    return r;
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

template <int G>
__global__ __launch_bounds__(kThreads) void w4_verify_kernel(W4Args a) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int GPC = kKC / G;  // groups per chunk
    const W4Mat mat = a.m[blockIdx.z];
    const int split = blockIdx.y;
    const int c0 = split * a.cps;
    const int c1 = min(a.nchunks, c0 + a.cps);
    const int k0 = c0 * kKC;
    const int k1 = min(a.K, c1 * kKC);
    const int kb = k1 - k0;
    const int xstride = a.cps * kKC + kXPad;  // LDS row stride (bf16 elements)
    uint16_t* xl = reinterpret_cast<uint16_t*>(smem);
    float* xsl = reinterpret_cast<float*>(smem + (size_t)16 * xstride * sizeof(uint16_t));

    // 1. activations of this split -> LDS (rows >= R are zero)
    const int n8 = kb >> 3;
    for (int idx = threadIdx.x; idx < 16 * n8; idx += kThreads) {
        const int r = idx / n8, c = idx - r * n8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < a.R) v = ld16(a.x + (size_t)r * a.K + k0 + c * 8);
        u32x4 o;
        o[0] = (v[0] & 0xffffu) | (v[2] << 16);
        o[1] = (v[0] >> 16) | (v[2] & 0xffff0000u);
        o[2] = (v[1] & 0xffffu) | (v[3] << 16);
        o[3] = (v[1] >> 16) | (v[3] & 0xffff0000u);
        *reinterpret_cast<u32x4*>(xl + r * xstride + c * 8) = o;
    }
    __syncthreads();

    // 2. group sums of x, one (row, group) per thread, fixed sequential order
    const int ngl = kb / G;
    for (int idx = threadIdx.x; idx < 16 * ngl; idx += kThreads) {
        const int r = idx & 15, g = idx >> 4;
        const uint16_t* p = xl + r * xstride + g * G;
        float sum = 0.f;
#pragma unroll 8
        for (int i = 0; i < G; ++i) sum += bf16_to_f32(p[i]);
        xsl[g * 16 + r] = sum;
    }
    __syncthreads();

    // 3. stream the weights
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int ln = lane & 15, j = lane >> 4;
    const size_t Kh = (size_t)(a.K >> 1);
    const size_t KG = (size_t)(a.K / G);
    const uint8_t* qrow[kNT];
    const uint16_t* srow[kNT];
    const uint16_t* brow[kNT];
    int ncol[kNT];
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
        ncol[t] = blockIdx.x * kBN + wave * (kNT * 16) + t * 16 + ln;
        const size_t nr = (size_t)min(ncol[t], a.N - 1);
        qrow[t] = mat.q + nr * Kh;
        srow[t] = mat.s + nr * KG;
        brow[t] = mat.b + nr * KG;
    }

    f32x4 y[kNT];
#pragma unroll
    for (int t = 0; t < kNT; ++t) y[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // prefetch registers for the next chunk
    u32x4 qn[kNT];
    uint16_t sn[kNT][GPC], bn[kNT][GPC];
    auto fetch = [&](int c) {
        const int kc = c * kKC;
        const int nst = min(4, (a.K - kc) >> 5);
        const int g0 = kc / G;
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
            qn[t] = (j < nst) ? ld16(qrow[t] + (kc >> 1) + 16 * j) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int g = 0; g < GPC; ++g) {
                const bool ok = g * G < (a.K - kc);
                sn[t][g] = ok ? srow[t][g0 + g] : (uint16_t)0;
                bn[t][g] = ok ? brow[t][g0 + g] : (uint16_t)0;
            }
        }
    };

    fetch(c0);
    for (int c = c0; c < c1; ++c) {
        u32x4 qv[kNT];
        float sv[kNT][GPC], bv[kNT][GPC];
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
            qv[t] = qn[t];
#pragma unroll
            for (int g = 0; g < GPC; ++g) {
                sv[t][g] = f16_to_f32(sn[t][g]);
                bv[t][g] = f16_to_f32(bn[t][g]);
            }
        }
        if (c + 1 < c1) fetch(c + 1);

        const int kc = c * kKC;
        const int nst = min(4, (a.K - kc) >> 5);
#pragma unroll
        for (int t = 0; t < kNT; ++t) transpose_rows(qv[t]);

        f32x4 acc[kNT];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            if (st < nst) {
                const u32x4 xa = ld16(xl + ln * xstride + (kc - k0) + 32 * st + 8 * j);
                const bf16x8 A = __builtin_bit_cast(bf16x8, xa);
                const bool first = (G == 32) || ((st & 1) == 0);
#pragma unroll
                for (int t = 0; t < kNT; ++t) {
                    const bf16x8 B = __builtin_bit_cast(bf16x8, decode_nibbles(qv[t][st]));
                    const f32x4 cin = first ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[t];
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, cin, 0, 0, 0);
                }
                const bool last = (G == 32) || ((st & 1) == 1);
                if (last) {
                    const int gc = (32 * st) / G;  // group within the chunk
                    const int gl = (kc - k0) / G + gc;
                    const f32x4 xs4 = *reinterpret_cast<const f32x4*>(xsl + gl * 16 + 4 * j);
#pragma unroll
                    for (int t = 0; t < kNT; ++t) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float d = fmaf(-16.f, xs4[i], acc[t][i]);
                            y[t][i] = fmaf(sv[t][gc], d, y[t][i]);
                            y[t][i] = fmaf(bv[t][gc], xs4[i], y[t][i]);
                        }
                    }
                }
            }
        }
    }

    // 4. rows r = 4j + i of columns ncol[t]
    float* out = mat.out + (size_t)split * a.split_stride;
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
        if (ncol[t] < a.N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * j + i;
                if (r < a.R) out[(size_t)r * a.N + ncol[t]] = y[t][i];
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

static int32_t launch_w4(const W4Args& args, int nmat, const W4Plan& p, int G, long ncols,
                         hipStream_t st) {
    dim3 grid((unsigned)((ncols + kBN - 1) / kBN), (unsigned)p.S, (unsigned)nmat);
    const size_t lds = w4_lds_bytes(p, G);
    hipEvent_t ea = nullptr, eb = nullptr;
    bool timed;
    {
        std::lock_guard<std::mutex> lk(g_timing.mu);
        timed = g_timing.on;
    }
    if (timed) {
        if (hipEventCreate(&ea) != hipSuccess || hipEventCreate(&eb) != hipSuccess)
            return fail(EV_EHIP, "w4 timing: hipEventCreate failed");
        hipEventRecord(ea, st);
    }
    if (G == 64)
        hipLaunchKernelGGL(w4_verify_kernel<64>, grid, dim3(kThreads), lds, st, args);
    else
        hipLaunchKernelGGL(w4_verify_kernel<32>, grid, dim3(kThreads), lds, st, args);
    int32_t rc = check_hip(hipGetLastError(), "w4_verify_kernel launch");
    if (timed) {
        hipEventRecord(eb, st);
        std::lock_guard<std::mutex> lk(g_timing.mu);
        g_timing.recs.push_back({ea, eb, w4_algo_bytes(nmat, args.R, args.K, args.N, G)});
    }
    return rc;
}

static int32_t check_w4_shape(const char* who, int R, int K, int N, int G) {
    if (R < 1 || R > EV_MAX_LANES) return fail(EV_EINVAL, "%s: R=%d outside 1..16", who, R);
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
        hipEventDestroy(r.a);
        hipEventDestroy(r.b);
    }
    if (launches) *launches = (int64_t)recs.size();
    if (total_ms) *total_ms = ms;
    if (total_bytes) *total_bytes = bytes;
    return rc;
}

extern "C" size_t verify_linear_w4_workspace(int32_t K, int32_t N, int32_t G) {
    if (K <= 0 || N <= 0 || (G != 32 && G != 64)) return 0;
    const W4Plan p = plan_w4(N, K);
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
    const W4Plan p = plan_w4(N, K);
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
    a.nchunks = p.nchunks;
    a.cps = p.cps;
    a.split_stride = p.S > 1 ? (long)16 * N : 0;
    if ((rc = launch_w4(a, 1, p, G, N, st))) return rc;
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
    L.p1 = plan_w4(2L * I, H);
    L.p2 = plan_w4(H, I);
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
    a.nchunks = L.p1.nchunks;
    a.cps = L.p1.cps;
    a.split_stride = (long)16 * I;
    if ((rc = launch_w4(a, 2, L.p1, G, I, st))) return rc;
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
    d.nchunks = L.p2.nchunks;
    d.cps = L.p2.cps;
    d.split_stride = L.p2.S > 1 ? (long)16 * H : 0;
    if ((rc = launch_w4(d, 1, L.p2, G, H, st))) return rc;
    if (L.p2.S > 1) {
        dim3 grid((unsigned)((H + 255) / 256), (unsigned)R);
        hipLaunchKernelGGL(splitk_reduce_kernel, grid, dim3(256), 0, st, pd, L.p2.S, H, y);
        if ((rc = check_hip(hipGetLastError(), "splitk_reduce launch"))) return rc;
    }
    return EV_OK;
}
