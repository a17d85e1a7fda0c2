// Keyed Gumbel-max sampler and the accept rule on gfx950.
//
// TensorFold README, exactness paragraph (restated by 650 Group, "TensorFold:
// the contract is what it does not change"): the token at position p is the
// argmax over the top-k/top-p candidates of logit/T + g(seed, p, token), with g
// Gumbel noise from a hash of seed, position and token id -- an exact draw that
// depends only on that row's logits and its position.  Temperature 0 is greedy
// (README options table).
//
// Two launches per call, neither depending on R except through the grid's row
// dimension (each row is processed by its own workgroups, identically):
//   topk_chunk_kernel   grid (ceil(V/4096), R) x 256: each workgroup selects
//                       the top-kk of its 4096 logits under (logit desc, id asc)
//                       as 64-bit order keys: each wave takes its own top-kk
//                       by kk rounds of a DPP wave maximum, and the four lists
//                       are merged by counting larger keys;
//   merge_sample_kernel grid R x 64: one wave merges the chunk lists into the
//                       row's top-kk, then top-p and the keyed argmax in fp64.
// The selection involves no arithmetic, so it is exact; the fp64 stage follows
// the same fixed order for every row.
#include "ev_internal.h"

namespace ev {

constexpr int kChunk = 4096;         // logits per top-k workgroup
constexpr int kSThreads = 256;
constexpr int kPer = kChunk / kSThreads;
constexpr int kMaxChunks = 64;       // V <= 64 * 4096 = 262144 (one merge lane per chunk)
constexpr unsigned long long kGamma = 0x9E3779B97F4A7C15ull;

// SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014).
__device__ __forceinline__ unsigned long long mix64(unsigned long long z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// g(seed, p, id): row key = output p+1 of the stream started at mix64(seed);
// token hash = output id+1 of the stream started at the row key; uniform from
// the top 52 bits plus a half; Gumbel by inversion, all in fp64.
__device__ __forceinline__ double keyed_gumbel(unsigned long long seed, long long pos, int id) {
    const unsigned long long row = mix64(mix64(seed) + (unsigned long long)(pos + 1) * kGamma);
    const unsigned long long h = mix64(row + (unsigned long long)((long long)id + 1) * kGamma);
    const double u = ((double)(h >> 12) + 0.5) * 0x1p-52;
    return -log(-log(u));
}

// Sorts 16 keys descending in registers (a fixed bitonic network).
__device__ __forceinline__ void sort16_desc(unsigned long long (&k)[kPer]) {
    static_assert(kPer == 16, "network for 16 keys");
#pragma unroll
    for (int size = 2; size <= 16; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int j = i ^ stride;
                if (j > i) {
                    const bool desc = (i & size) == 0;  // direction of this bitonic block
                    const unsigned long long a = k[i], b = k[j];
                    const bool sw = desc ? (a < b) : (a > b);
                    k[i] = sw ? b : a;
                    k[j] = sw ? a : b;
                }
            }
}

// Maximum of a 32-bit value over the wave (DPP steps as in wave_max_u64),
// returned to every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    uint32_t o;
    o = __builtin_amdgcn_update_dpp(v, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v = o > v ? o : v;
    o = __builtin_amdgcn_update_dpp(v, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v = o > v ? o : v;
    o = __builtin_amdgcn_update_dpp(v, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v = o > v ? o : v;
    o = __builtin_amdgcn_update_dpp(v, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v = o > v ? o : v;
    o = __builtin_amdgcn_update_dpp(v, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v = o > v ? o : v;
    o = __builtin_amdgcn_update_dpp(v, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    v = o > v ? o : v;
    return __builtin_amdgcn_readlane(v, 63);
}
// The wave's largest 64-bit key: the largest high word, then the largest low
// word among the lanes that hold it (the lexicographic order of the pair).
__device__ __forceinline__ unsigned long long wave_max_key(unsigned long long k) {
    const uint32_t hi = (uint32_t)(k >> 32);
    const uint32_t mh = wave_max_u32(hi);
    const uint32_t ml = wave_max_u32(hi == mh ? (uint32_t)k : 0u);
    return ((unsigned long long)mh << 32) | ml;
}
// Entries of the descending list l[0..n) greater than e.
__device__ __forceinline__ int count_greater(const unsigned long long* l, int n, unsigned long long e) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (l[mid] > e)
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo;
}

// The chunk's top-kk keys in order.  Every thread sorts its 16 keys once and
// keeps keys 1..15 in LDS.  Each wave then takes its own top-kk in kk rounds
// of a wave maximum over the threads' heads (no barrier; the lane that held
// the winner reads its next key).  The chunk's top-kk lies in the union of
// the four wave lists, and a candidate's place is the number of larger keys
// in the four lists (binary search in the other three): keys are unique, so
// the places of the chunk's top-kk are 0..kk-1 and every other candidate's
// place is kk or more.
// Candidates a row keeps: the top_k largest, 2 when greedy (the argmax and
// the runner-up for the gap), never more than V; always within 1..64, the
// bound of the kernels' lists (validated parameters are inside it anyway).
__host__ __device__ inline int sample_kk_of(double T, int top_k, int V) {
    int k = T == 0.0 ? 2 : top_k;
    k = k < 1 ? 1 : (k > EV_MAX_TOPK ? EV_MAX_TOPK : k);
    return k < V ? k : V;
}

__global__ __launch_bounds__(kSThreads) void topk_chunk_kernel(const float* __restrict__ logits,
                                                               int V, int kk, int nchunk,
                                                               const ev_sampling* __restrict__ sd,
                                                               unsigned long long* __restrict__ out) {
    if (sd) kk = sample_kk_of(sd->temperature, sd->top_k, V);  // parameters kept on the device
    constexpr int kW = kSThreads / 64;
    __shared__ unsigned long long rest[kPer - 1][kSThreads];  // thread t's keys 1..15 in column t
    __shared__ unsigned long long wl[kW][EV_MAX_TOPK];       // each wave's top-kk, in order
    __shared__ unsigned long long sel[EV_MAX_TOPK];          // the chunk's top-kk, in order
    const int r = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
    const int base = chunk * kChunk;
    const float* row = logits + (size_t)r * V;
    unsigned long long keys[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int idx = base + i * kSThreads + tid;
        keys[i] = idx < V ? order_key(row[idx], idx) : 0ull;
    }
    sort16_desc(keys);
#pragma unroll
    for (int i = 1; i < kPer; ++i) rest[i - 1][tid] = keys[i];
    if (tid < kk) sel[tid] = 0ull;  // places past the chunk's real keys stay 0
    const int wave = tid >> 6, lane = tid & 63;
    unsigned long long head = keys[0];
    int at = 0;
    for (int round = 0; round < kk; ++round) {
        const unsigned long long w = wave_max_key(head);
        if (lane == 0) wl[wave][round] = w;
        if (w != 0ull && head == w) {  // keys are unique: one lane
            ++at;
            head = at < kPer ? rest[at - 1][tid] : 0ull;
        }
    }
    __syncthreads();
    if (tid < kW * kk) {
        const int v = tid / kk, i = tid - v * kk;
        const unsigned long long e = wl[v][i];
        if (e != 0ull) {
            int place = i;
#pragma unroll
            for (int u = 0; u < kW; ++u)
                if (u != v) place += count_greater(wl[u], kk, e);
            if (place < kk) sel[place] = e;
        }
    }
    __syncthreads();
    unsigned long long* dst = out + ((size_t)r * nchunk + chunk) * kk;
    if (tid < kk) dst[tid] = sel[tid];
}

struct SampleArgs {
    const unsigned long long* cand;  // [R][nchunk][kk]
    const long long* positions;
    int nchunk, kk, V;
    double T, top_p;
    unsigned long long seed;
    const ev_sampling* sd;  // when non-NULL, T, top_k, top_p and seed are read here
    int* tokens;
    double* gap;
};

__global__ __launch_bounds__(64) void merge_sample_kernel(SampleArgs a) {
    if (a.sd) {
        const ev_sampling s = *a.sd;
        a.T = s.temperature;
        a.top_p = s.top_p;
        a.seed = s.seed;
        a.kk = sample_kk_of(s.temperature, s.top_k, a.V);
    }
    __shared__ unsigned long long lists[kMaxChunks * EV_MAX_TOPK];  // [chunk][kk], each in order
    const int r = blockIdx.x, lane = threadIdx.x;
    const int n = a.nchunk * a.kk;  // <= 64 * 64
    const unsigned long long* src = a.cand + (size_t)r * n;
    for (int i = lane; i < n; i += 64) lists[i] = src[i];
    __syncthreads();
    // k-way merge: lane c follows list c; a round takes the maximum of the
    // heads, and the lane that held it advances (keys are unique)
    int at = 0;
    unsigned long long head = lane < a.nchunk ? lists[lane * a.kk] : 0ull;
    unsigned long long mine = 0ull;  // candidate j ends up in lane j
    for (int round = 0; round < a.kk; ++round) {
        const unsigned long long win = wave_max_u64(head);
        if (lane == round) mine = win;
        if (win != 0ull && head == win) {
            ++at;
            head = at < a.kk ? lists[lane * a.kk + at] : 0ull;
        }
    }
    const int ncand = a.kk < a.V ? a.kk : a.V;
    const float l = key_logit(mine);
    const int id = key_id(mine);

    if (a.T == 0.0) {  // greedy: candidates 0 and 1 of the exact order
        const double l0 = (double)__shfl(l, 0, 64), l1 = (double)__shfl(l, 1, 64);
        const int id0 = __shfl(id, 0, 64);
        if (lane == 0) {
            a.tokens[r] = id0;
            if (a.gap) a.gap[r] = ncand > 1 ? l0 - l1 : __builtin_huge_val();
        }
        return;
    }

    // top-p: e_j = exp((l_j - l_0) / T), Z summed in candidate order; keep j
    // while the mass before it is below top_p * Z.  Every lane runs the same
    // sequential loop on the shuffled values, so all lanes agree.
    const double m = (double)__shfl(l, 0, 64);
    const double e = lane < ncand ? exp(((double)l - m) / a.T) : 0.0;
    double Z = 0.0;
    for (int jj = 0; jj < ncand; ++jj) Z += __shfl(e, jj, 64);
    const double thr = a.top_p * Z;
    int kept = 0;
    double before = 0.0;
    for (int jj = 0; jj < ncand; ++jj) {
        if (jj > 0 && !(before < thr)) break;
        kept = jj + 1;
        before += __shfl(e, jj, 64);
    }

    // perturbed scores and the argmax (lower id on equal scores)
    const long long pos = a.positions[r];
    double z = -__builtin_huge_val();
    if (lane < kept) z = (double)l / a.T + keyed_gumbel(a.seed, pos, id);
    double bz = z;
    int bid = lane < kept ? id : 0x7fffffff;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double oz = __shfl_xor(bz, off, 64);
        const int oid = __shfl_xor(bid, off, 64);
        if (oz > bz || (oz == bz && oid < bid)) {
            bz = oz;
            bid = oid;
        }
    }
    // second best: the best score among the other kept candidates
    double sz = (lane < kept && id != bid) ? z : -__builtin_huge_val();
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double oz = __shfl_xor(sz, off, 64);
        sz = oz > sz ? oz : sz;
    }
    if (lane == 0) {
        a.tokens[r] = bid;
        if (a.gap) a.gap[r] = kept > 1 ? bz - sz : __builtin_huge_val();
    }
}

// n_accept = leading i < D with draft[i] == sampled[i]; n_commit = min(a+1, R).
__global__ __launch_bounds__(64) void accept_kernel(const int* __restrict__ sampled, int R,
                                                    const int* __restrict__ draft, int D,
                                                    int* __restrict__ n_accept,
                                                    int* __restrict__ n_commit) {
    const int i = threadIdx.x;
    const bool mism = i < D && draft[i] != sampled[i];
    const unsigned long long mask = __ballot(mism);
    const int acc = mask ? (__ffsll((long long)mask) - 1) : D;
    if (i == 0) {
        *n_accept = acc;
        *n_commit = acc + 1 < R ? acc + 1 : R;
    }
}

static int sample_nchunk(int V) { return (V + kChunk - 1) / kChunk; }

}  // namespace ev

using namespace ev;

namespace ev {
int32_t check_sampling(const char* who, const ev_sampling& s) {
    if (!(s.temperature >= 0.0) || !(s.temperature < __builtin_huge_val()))
        return fail(EV_EINVAL, "%s: temperature must be finite and >= 0", who);
    if (s.temperature > 0.0) {
        if (s.top_k < 1) return fail(EV_EINVAL, "%s: top_k=%d", who, s.top_k);
        if (s.top_k > EV_MAX_TOPK) return fail(EV_EUNSUPPORTED, "%s: top_k=%d above 64", who, s.top_k);
        if (!(s.top_p > 0.0 && s.top_p <= 1.0)) return fail(EV_EINVAL, "%s: top_p outside (0,1]", who);
    }
    return EV_OK;
}
}  // namespace ev

extern "C" size_t keyed_sample_workspace(int32_t V) {
    if (V <= 0) return 0;
    return (size_t)EV_MAX_LANES * sample_nchunk(V) * EV_MAX_TOPK * sizeof(unsigned long long);
}

// Checks the shapes and pointers of a keyed sample (the sampling parameters
// are checked by the caller).
static int32_t check_sample_args(const char* who, const float* logits, int32_t R, int32_t V,
                                 const int64_t* positions, int32_t* tokens, double* gap, void* ws,
                                 size_t ws_bytes) {
    if (R < 1 || R > EV_MAX_LANES) return fail(EV_EINVAL, "%s: R=%d outside 1..16", who, R);
    if (V < 1) return fail(EV_EINVAL, "%s: V=%d", who, V);
    if (V > kMaxChunks * kChunk) return fail(EV_EUNSUPPORTED, "%s: V=%d above %d", who, V, kMaxChunks * kChunk);
    if (!logits || !positions || !tokens) return fail(EV_EINVAL, "%s: NULL pointer", who);
    if (!aligned(logits, 4) || !aligned(positions, 8) || !aligned(tokens, 4) || (gap && !aligned(gap, 8)))
        return fail(EV_EINVAL, "%s: misaligned pointer", who);
    const size_t need = keyed_sample_workspace(V);
    if (!ws || ws_bytes < need)
        return fail(EV_EWORKSPACE, "%s: workspace needs %zu bytes, got %zu", who, need, ws ? ws_bytes : (size_t)0);
    if (!aligned(ws, 8)) return fail(EV_EINVAL, "%s: workspace must be 8-byte aligned", who);
    return EV_OK;
}

namespace ev {
// The two launches of a keyed sample.  `sd` (device, may be NULL): when
// given, the kernels read the sampling parameters there instead of from `s`
// (the verify step keeps them in its workspace, so that one captured step
// serves every seed and temperature).
int32_t launch_keyed_sample(const float* logits, int R, int V, const long long* positions, const ev_sampling& s,
                            const ev_sampling* sd, int32_t* tokens, double* gap, void* ws, hipStream_t st) {
    const int nchunk = sample_nchunk(V);
    const int kk = sample_kk_of(s.temperature, s.top_k, V);
    unsigned long long* cand = reinterpret_cast<unsigned long long*>(ws);
    hipLaunchKernelGGL(topk_chunk_kernel, dim3(nchunk, R), dim3(kSThreads), 0, st, logits, V, kk, nchunk, sd,
                       cand);
    int32_t rc = check_hip(hipGetLastError(), "topk_chunk launch");
    if (rc) return rc;
    SampleArgs a{cand, positions, nchunk, kk, V, s.temperature, s.top_p, (unsigned long long)s.seed, sd,
                 tokens, gap};
    hipLaunchKernelGGL(merge_sample_kernel, dim3(R), dim3(64), 0, st, a);
    return check_hip(hipGetLastError(), "merge_sample launch");
}
}  // namespace ev

extern "C" int32_t keyed_sample(const float* logits, int32_t R, int32_t V, const int64_t* positions,
                                ev_sampling s, int32_t* tokens, double* gap, void* ws,
                                size_t ws_bytes, void* stream) {
    clear_error();
    const char* who = "keyed_sample";
    int32_t rc;
    if ((rc = check_sample_args(who, logits, R, V, positions, tokens, gap, ws, ws_bytes))) return rc;
    if ((rc = check_sampling(who, s))) return rc;
    return launch_keyed_sample(logits, R, V, reinterpret_cast<const long long*>(positions), s, nullptr, tokens,
                               gap, ws, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int32_t accept_prefix(const int32_t* sampled, int32_t R, const int32_t* draft, int32_t D,
                                 int32_t* n_accept, int32_t* n_commit, void* stream) {
    clear_error();
    const char* who = "accept_prefix";
    if (R < 1 || R > EV_MAX_LANES) return fail(EV_EINVAL, "%s: R=%d outside 1..16", who, R);
    if (D < 0 || D > R) return fail(EV_EINVAL, "%s: D=%d outside 0..R", who, D);
    if (!sampled || !n_accept || !n_commit || (D > 0 && !draft))
        return fail(EV_EINVAL, "%s: NULL pointer", who);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(accept_kernel, dim3(1), dim3(64), 0, st, sampled, R, draft, D, n_accept,
                       n_commit);
    return check_hip(hipGetLastError(), "accept launch");
}
