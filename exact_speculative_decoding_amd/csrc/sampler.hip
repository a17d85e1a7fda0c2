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
//                       as 64-bit order keys: the keys at or above a lower
//                       bound of the kk-th are placed by counting larger keys;
//   merge_sample_kernel grid R x 256: the workgroup merges the chunk lists
//                       into the row's top-kk the same way, then one wave
//                       takes top-p and the keyed argmax in fp64.
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

// Sorts 16 keys descending in registers (a fixed bitonic network); the
// selection rounds need each thread's keys in order.
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

// Lane src's value, the same in every lane (v_readlane: no LDS round trip;
// src must be the same in every lane).
__device__ __forceinline__ int lane_i32(int v, int src) { return __builtin_amdgcn_readlane(v, src); }
__device__ __forceinline__ float lane_f32(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}
__device__ __forceinline__ double lane_f64(double v, int src) {
    const unsigned long long b = __builtin_bit_cast(unsigned long long, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, src);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), src);
    return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}
// Order key of a double (larger key, larger value; -0 folded onto +0, so equal
// values have equal keys); 0 is below every key of a non-NaN value.
__device__ __forceinline__ unsigned long long f64_order_key(double v) {
    const unsigned long long b = v == 0.0 ? 0ull : __builtin_bit_cast(unsigned long long, v);
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// Inclusive prefix sum of v over the wave's lanes.
__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    return v;
}

// Selection by rank: cand[0..n) holds distinct keys; the key with exactly
// `rank` larger keys among them goes to out[rank] when rank < kk.  nthreads
// threads share the candidates (every thread reads every candidate: LDS
// broadcasts).  The caller syncs before (cand complete) and after (out).
__device__ __forceinline__ int rank_of(const unsigned long long* cand, int n, unsigned long long e) {
    int rank = 0;
    int i = 0;
    for (; i + 8 <= n; i += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) rank += cand[i + u] > e ? 1 : 0;
    }
    for (; i < n; ++i) rank += cand[i] > e ? 1 : 0;
    return rank;
}
__device__ __forceinline__ void place_by_rank(const unsigned long long* cand, int n, int kk,
                                              unsigned long long* out, int nthreads) {
    for (int j = threadIdx.x; j < n; j += nthreads) {
        const unsigned long long e = cand[j];
        const int rank = rank_of(cand, n, e);
        if (rank < kk) out[rank] = e;
    }
}
// The kk-th largest nonzero key of sample[0..S) (keys distinct except 0), or
// 0 when the sample holds fewer than kk nonzero keys: written to *t by the
// thread that holds it.  The caller zeroes *t and syncs before and after.
__device__ __forceinline__ void kth_of_sample(const unsigned long long* sample, int S, int kk,
                                              unsigned long long* t, int nthreads) {
    for (int j = threadIdx.x; j < S; j += nthreads) {
        const unsigned long long e = sample[j];
        if (e != 0ull && rank_of(sample, S, e) == kk - 1) *t = e;
    }
}
constexpr int kRankCap = 256;  // candidates ranked directly; more fall back to selection rounds
constexpr int kRoundsMax = 2;  // kk up to this (greedy) always selects in rounds: two are cheaper

// The chunk's top-kk keys in order.  Every thread sorts its 16 keys once.
// The kk-th largest of the maxima of groups of adjacent threads is a lower
// bound t of the chunk's kk-th largest key (kk distinct keys are at or above
// it; t = 0 when fewer than kk groups hold a key).  The keys >= t (the chunk's top-kk
// among them, usually a few more) are gathered in LDS and each is placed by
// the number of larger ones.  When more than kRankCap keys reach t (ties,
// short chunks), the selection runs in kk rounds instead: each wave takes its
// own top-kk by a wave maximum over the threads' heads, and a candidate's
// place is the number of larger keys in the four wave lists (binary search):
// keys are unique, so the places of the chunk's top-kk are 0..kk-1.
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
                                                               unsigned long long* __restrict__ out,
                                                               int* __restrict__ acc_count) {
    if (acc_count && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *acc_count = 0;
    if (sd) kk = sample_kk_of(sd->temperature, sd->top_k, V);  // parameters kept on the device
    constexpr int kW = kSThreads / 64;
    __shared__ unsigned long long rest[kPer - 1][kSThreads];  // thread t's keys 1..15 in column t
    __shared__ unsigned long long wl[kW][EV_MAX_TOPK];       // each wave's top-kk, in order
    __shared__ unsigned long long sel[EV_MAX_TOPK];          // the chunk's top-kk, in order
    __shared__ unsigned long long cand[kRankCap];            // the keys >= t
    __shared__ unsigned long long smax[kSThreads];           // the threads' maxima
    __shared__ unsigned long long s_t;
    __shared__ int wsum[kW];
    const int r = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
    const int base = chunk * kChunk;
    const float* row = logits + (size_t)r * V;
    // all sixteen loads issued before the first use: the index is clamped
    // and the key masked, rather than the load made conditional (a
    // conditional load waits for each one in turn)
    unsigned long long keys[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int idx = base + i * kSThreads + tid;
        const float v = row[idx < V ? idx : V - 1];
        keys[i] = order_key(v, idx) & (0ull - (unsigned long long)(idx < V));
    }
    if (tid < kk) sel[tid] = 0ull;  // places past the chunk's real keys stay 0
    const int wave = tid >> 6, lane = tid & 63;

    if (kk > kRoundsMax) {
        // the lower bound t: the kk-th largest maximum of groups of gs adjacent
        // threads (no sort here: only the thread's maximum and its keys >= t,
        // in any order, are needed)
        const int gs = kk <= 32 ? 4 : 2;  // at least 2 kk groups
        unsigned long long gm = keys[0];
#pragma unroll
        for (int i = 1; i < kPer; ++i) gm = keys[i] > gm ? keys[i] : gm;
        for (int off = 1; off < gs; off <<= 1) {
            const unsigned long long o = __shfl_xor(gm, off, 64);
            gm = o > gm ? o : gm;
        }
        if ((lane & (gs - 1)) == 0) smax[tid / gs] = gm;
        if (tid == 0) s_t = 0ull;
        __syncthreads();
        kth_of_sample(smax, kSThreads / gs, kk, &s_t, kSThreads);
        __syncthreads();
        const unsigned long long t = s_t;
        // the thread's keys >= t (key 0 pads past V)
        int c = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) c += (keys[i] >= t && keys[i] != 0ull) ? 1 : 0;
        const int incl = wave_incl_scan(c);
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int off0 = 0, n = 0;
#pragma unroll
        for (int v = 0; v < kW; ++v) {
            off0 += v < wave ? wsum[v] : 0;
            n += wsum[v];
        }
        if (n <= kRankCap) {
            int o = off0 + incl - c;
#pragma unroll
            for (int i = 0; i < kPer; ++i)
                if (keys[i] >= t && keys[i] != 0ull) cand[o++] = keys[i];
            __syncthreads();
            place_by_rank(cand, n, kk, sel, kSThreads);
            __syncthreads();
            unsigned long long* dst = out + ((size_t)r * nchunk + chunk) * kk;
            if (tid < kk) dst[tid] = sel[tid];
            return;
        }
    }

    // selection rounds: the thread's keys sorted, 1..15 in LDS (its own
    // column); its current key and the one after it (read ahead, so that a
    // win does not wait for LDS); nxt is key at of the sorted 16
    sort16_desc(keys);
#pragma unroll
    for (int i = 1; i < kPer; ++i) rest[i - 1][tid] = keys[i];
    unsigned long long head = keys[0], nxt = keys[1];
    int at = 1;
    for (int round = 0; round < kk; ++round) {
        const unsigned long long w = wave_max_u64(head);
        if (lane == 0) wl[wave][round] = w;
        if (w != 0ull && head == w) {  // keys are unique: one lane
            head = nxt;
            ++at;
            nxt = at < kPer ? rest[at - 1][tid] : 0ull;
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
    FusedAccept acc;  // acc.count == NULL: no accept here
    int R;
};

// The accept prefix by the last of the R merge workgroups to store its token
// (wave 0, after its lane 0 stored the row's token): each workgroup makes its
// token visible device-wide before it counts itself; the one that completes
// the count sees every row's token, compares the drafts as accept_kernel
// does, and clears the count for the next step.
__device__ __forceinline__ void fused_accept(const SampleArgs& a) {
    if (!a.acc.count) return;
    const int lane = threadIdx.x & 63;
    int last = 0;
    if (lane == 0) {
        __threadfence();
        last = atomicAdd(a.acc.count, 1) == a.R - 1;
    }
    if (!__shfl(last, 0, 64)) return;
    __threadfence();
    const int i = lane;
    const bool mism = i < a.acc.D && a.acc.draft[i] != a.tokens[i];
    const unsigned long long mask = __ballot(mism);
    const int n = mask ? (__ffsll((long long)mask) - 1) : a.acc.D;
    if (lane == 0) {
        *a.acc.n_accept = n;
        *a.acc.n_commit = n + 1 < a.R ? n + 1 : a.R;
        *a.acc.count = 0;
    }
}

// k-way merge of sorted lists in kk rounds by one wave (lane c follows list
// c, `has` for c < nchunk): a round takes the maximum of the heads, the lane
// that held it advances (keys are unique), and lane j keeps round j's key.
// Each lane also holds the entry after its head, read ahead.
__device__ __forceinline__ void merge_rounds(const unsigned long long* mylist, bool has, int kk,
                                             unsigned long long& mine) {
    const int lane = threadIdx.x & 63;
    int at = 0;
    unsigned long long head = has ? mylist[0] : 0ull;
    unsigned long long nxt = has && kk > 1 ? mylist[1] : 0ull;
    for (int round = 0; round < kk; ++round) {
        const unsigned long long win = wave_max_u64(head);
        if (lane == round) mine = win;
        if (win != 0ull && head == win) {
            ++at;
            head = nxt;
            nxt = at + 1 < kk ? mylist[at + 1] : 0ull;
        }
    }
}

constexpr int kMThreads = 256;  // merge workgroup: four waves select, wave 0 samples
__global__ __launch_bounds__(kMThreads) void merge_sample_kernel(SampleArgs a) {
    if (a.sd) {
        const ev_sampling s = *a.sd;
        a.T = s.temperature;
        a.top_p = s.top_p;
        a.seed = s.seed;
        a.kk = sample_kk_of(s.temperature, s.top_k, a.V);
    }
    __shared__ unsigned long long lists[kMaxChunks * EV_MAX_TOPK];  // [chunk][kk], each in order
    __shared__ unsigned long long cand[kRankCap];                   // the sample, then the keys >= t
    __shared__ unsigned long long top[EV_MAX_TOPK];
    __shared__ unsigned long long s_t;
    __shared__ int s_nc;
    const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int n = a.nchunk * a.kk;  // <= 64 * 64
    const unsigned long long* src = a.cand + (size_t)r * n;
    // the lists into LDS, up to sixteen loads in flight per thread
    {
        unsigned long long v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int i = kMThreads * u + tid;
            v[u] = i < n ? src[i] : 0ull;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int i = kMThreads * u + tid;
            if (i < n) lists[i] = v[u];
        }
    }
    // The row's top-kk from the chunk lists.  The kk-th largest of a sample
    // -- the first ms = ceil(kk / nchunk) keys of every list -- is a lower
    // bound t of the row's kk-th key (t = 0 when the sample holds fewer than
    // kk keys): the keys >= t are gathered and each is placed by the number
    // of larger ones.  With more than kRankCap of them, wave 0 merges the
    // lists in kk rounds instead: a round takes the maximum of the lists'
    // heads and the lane that held it advances (keys are unique).
    const bool has = tid < a.nchunk;
    const unsigned long long* mylist = lists + (has ? tid : 0) * a.kk;
    unsigned long long mine = 0ull;  // candidate j ends up in lane j of wave 0
    if (a.kk <= kRoundsMax) {
        __syncthreads();
        if (tid >= 64) return;
        merge_rounds(mylist, has, a.kk, mine);
    } else {
        const int ms = (a.kk + a.nchunk - 1) / a.nchunk;
        const int S = a.nchunk * ms;  // < kk + nchunk <= 128
        if (tid < a.kk) top[tid] = 0ull;
        if (tid == 0) s_t = 0ull;
        __syncthreads();
        if (tid < S) cand[tid] = lists[(tid / ms) * a.kk + tid % ms];
        __syncthreads();
        kth_of_sample(cand, S, a.kk, &s_t, kMThreads);
        __syncthreads();
        const unsigned long long t = s_t;
        // wave 0: lane c counts list c's keys >= t (a prefix: binary search; key
        // 0 pads) and copies them after the lists before it
        int c = 0, incl = 0;
        if (tid < 64) {
            if (has) {
                int lo = 0, hi = a.kk;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    const unsigned long long e = mylist[mid];
                    if (e >= t && e != 0ull)
                        lo = mid + 1;
                    else
                        hi = mid;
                }
                c = lo;
            }
            incl = wave_incl_scan(c);
            if (tid == 63) s_nc = incl;
        }
        __syncthreads();
        const int nc = s_nc;
        if (nc <= kRankCap) {
            if (tid < 64 && incl <= kRankCap)
                for (int i = 0; i < c; ++i) cand[incl - c + i] = mylist[i];
            __syncthreads();
            place_by_rank(cand, nc, a.kk, top, kMThreads);
            __syncthreads();
            if (tid >= 64) return;
            if (lane < a.kk) mine = top[lane];
        } else {
            if (tid >= 64) return;
            merge_rounds(mylist, has, a.kk, mine);
        }
    }
    const int ncand = a.kk < a.V ? a.kk : a.V;
    const float l = key_logit(mine);
    const int id = key_id(mine);

    if (a.T == 0.0) {  // greedy: candidates 0 and 1 of the exact order
        const double l0 = (double)lane_f32(l, 0), l1 = (double)lane_f32(l, 1);
        const int id0 = lane_i32(id, 0);
        if (lane == 0) {
            a.tokens[r] = id0;
            if (a.gap) a.gap[r] = ncand > 1 ? l0 - l1 : __builtin_huge_val();
        }
        fused_accept(a);
        return;
    }

    // top-p: e_j = exp((l_j - l_0) / T), Z summed in candidate order (every
    // lane runs the same sequential sum on values read from lane j); lane j
    // keeps the mass before it, P_j.  Candidate j is kept while P_j < top_p Z
    // (j = 0 always): the masses are >= 0, so P_j grows with j and the kept
    // candidates are 0 and the lanes j >= 1 with P_j < top_p Z.
    const double m = (double)lane_f32(l, 0);
    const double e = lane < ncand ? exp(((double)l - m) / a.T) : 0.0;
    double Z = 0.0, P = 0.0;
    for (int jj = 0; jj < ncand; ++jj) {
        if (lane == jj) P = Z;
        Z += lane_f64(e, jj);
    }
    const double thr = a.top_p * Z;
    const int kept = 1 + __popcll(__ballot(lane >= 1 && lane < ncand && P < thr));

    // perturbed scores (one per lane) and the argmax under (score desc, id
    // asc): a wave maximum of the scores' order keys (-0 folded onto +0, so
    // equal scores have equal keys), the lowest id among the lanes that hold
    // it; then the best score among the other kept candidates (from the
    // lowest lane that holds it)
    const long long pos = a.positions[r];
    double z = -__builtin_huge_val();
    if (lane < kept) z = (double)l / a.T + keyed_gumbel(a.seed, pos, id);
    const unsigned long long kz = lane < kept ? f64_order_key(z) : 0ull;
    const unsigned long long kb = wave_max_u64(kz);
    const unsigned long long tie = __ballot(kz == kb);
    int bl = __builtin_ctzll(tie);
    if (__popcll(tie) > 1) {  // equal best scores: the lowest id
        const unsigned long long mi = wave_max_u64(kz == kb ? (unsigned long long)(0xffffffffu - (uint32_t)id) : 0ull);
        bl = __builtin_ctzll(__ballot(kz == kb && (unsigned long long)(0xffffffffu - (uint32_t)id) == mi));
    }
    const int bid = lane_i32(id, bl);
    const double bz = lane_f64(z, bl);
    const unsigned long long k2 = id != bid ? kz : 0ull;
    const unsigned long long ks = wave_max_u64(k2);
    const double sz = ks ? lane_f64(z, __builtin_ctzll(__ballot(k2 == ks))) : -__builtin_huge_val();
    if (lane == 0) {
        a.tokens[r] = bid;
        if (a.gap) a.gap[r] = kept > 1 ? bz - sz : __builtin_huge_val();
    }
    fused_accept(a);
}

// ---- top-p over the whole vocabulary (top_k == 0) ------------------------------
// The nucleus is cut on fixed-point masses, which add to the same total in any
// order: with the tokens ordered (logit desc, id asc) and m the largest logit,
// token j's mass is e_j = nearest(exp((l_j - m) / T) * 2^40), Z = sum e_j, and
// thr = max(1, trunc(fl(top_p * fl(Z)))); token j is kept iff the mass of the
// tokens before it is below thr.  The last kept token is found by a
// most-significant-digit-first select on the 64-bit order keys: six passes of
// 11, 11, 11, 11, 11 and 9 bits, each a histogram of integer masses over the
// keys that share the digits chosen so far (integer additions, so the
// histogram is the same whatever order the atomics land in); a pass picks the
// largest digit at which the mass of the keys above, plus that digit's, first
// reaches thr.  Then the keyed argmax over the tokens whose key is at least
// that last kept key.
constexpr int kTpPasses = 6;
constexpr int kTpBuckets = 2048;
constexpr double kTpScale = 1099511627776.0;  // 2^40
__device__ __forceinline__ int tp_shift(int d) { return d < 5 ? 53 - 11 * d : 0; }
__device__ __forceinline__ int tp_bits(int d) { return d < 5 ? 11 : 9; }

struct TpArgs {
    const float* logits;
    int V, nchunk;
    const long long* positions;
    double T, top_p;
    unsigned long long seed;
    const ev_sampling* sd;          // when non-NULL, T, top_p and seed are read here
    unsigned long long* cmax;       // [R][kMaxChunks] chunk maxima (order keys)
    unsigned long long* hist;       // [R][kTpPasses][kTpBuckets] fixed-point masses
    double* best;                   // [R][kMaxChunks][4]: z1, z2, id1 (as double), unused
    int* tokens;
    double* gap;
};

__device__ __forceinline__ void tp_params(const TpArgs& a, double& T, double& top_p, unsigned long long& seed) {
    if (a.sd) {
        const ev_sampling s = *a.sd;
        T = s.temperature;
        top_p = s.top_p;
        seed = s.seed;
    } else {
        T = a.T;
        top_p = a.top_p;
        seed = a.seed;
    }
}

// The row's largest order key (every wave computes it; no barrier needed).
__device__ __forceinline__ unsigned long long tp_row_max(const TpArgs& a, int r) {
    const int lane = threadIdx.x & 63;
    unsigned long long k = lane < a.nchunk ? a.cmax[(size_t)r * kMaxChunks + lane] : 0ull;
    return wave_max_u64(k);
}

// Chunk maxima; chunk 0 of each row also clears the row's histograms.
__global__ __launch_bounds__(kSThreads) void tp_max_kernel(TpArgs a) {
    __shared__ unsigned long long red[kSThreads / 64];
    const int r = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
    const float* row = a.logits + (size_t)r * a.V;
    unsigned long long k = 0ull;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {  // clamped index: the loads are all in flight at once
        const int idx = chunk * kChunk + i * kSThreads + tid;
        const float v = row[idx < a.V ? idx : a.V - 1];
        const unsigned long long o = order_key(v, idx) & (0ull - (unsigned long long)(idx < a.V));
        k = o > k ? o : k;
    }
    k = wave_max_u64(k);
    if ((tid & 63) == 0) red[tid >> 6] = k;
    __syncthreads();
    if (tid == 0) {
        unsigned long long m = red[0];
        for (int w = 1; w < kSThreads / 64; ++w) m = red[w] > m ? red[w] : m;
        a.cmax[(size_t)r * kMaxChunks + chunk] = m;
    }
    if (chunk == 0) {
        unsigned long long* h = a.hist + (size_t)r * kTpPasses * kTpBuckets;
        for (int i = tid; i < kTpPasses * kTpBuckets; i += kSThreads) h[i] = 0ull;
    }
}

// Block-wide inclusive prefix sum of one integer per thread, in thread order.
__device__ __forceinline__ unsigned long long tp_block_scan(unsigned long long v, unsigned long long* sh) {
    const int tid = threadIdx.x;
    sh[tid] = v;
    __syncthreads();
    for (int off = 1; off < kSThreads; off <<= 1) {
        const unsigned long long add = tid >= off ? sh[tid - off] : 0ull;
        __syncthreads();
        sh[tid] += add;
        __syncthreads();
    }
    const unsigned long long out = sh[tid];
    __syncthreads();
    return out;
}

// One pass's choice: the largest digit b at which A + (mass of digits >= b)
// reaches thr; *A becomes A + (mass of digits > b).  Digits descend with the
// thread index (thread t holds digits 2047 - 8t .. 2040 - 8t).
__device__ int tp_select(const unsigned long long* h, unsigned long long* A, unsigned long long thr,
                         unsigned long long* sh, int* win) {
    const int tid = threadIdx.x;
    constexpr int per = kTpBuckets / kSThreads;
    unsigned long long v[per], tot = 0ull;
#pragma unroll
    for (int i = 0; i < per; ++i) {
        v[i] = h[kTpBuckets - 1 - (per * tid + i)];
        tot += v[i];
    }
    const unsigned long long incl = tp_block_scan(tot, sh);
    unsigned long long run = *A + incl - tot;  // mass of the digits above this thread's
    int mine = -1;
    unsigned long long above = 0ull;
#pragma unroll
    for (int i = 0; i < per; ++i) {
        if (mine < 0 && run + v[i] >= thr) {
            mine = kTpBuckets - 1 - (per * tid + i);
            above = run;
        }
        run += v[i];
    }
    if (tid == 0) *win = kSThreads;
    __syncthreads();
    if (mine >= 0) atomicMin(win, tid);
    __syncthreads();
    const int w = *win;
    __syncthreads();
    if (tid == w) {
        sh[0] = above;
        sh[1] = (unsigned long long)mine;
    }
    __syncthreads();
    const int digit = w < kSThreads ? (int)sh[1] : 0;  // a winner always exists for a consistent histogram
    if (w < kSThreads) *A = sh[0];
    __syncthreads();
    return digit;
}

// Z, thr and the digits of passes < d: the key prefix and the mass above it.
__device__ void tp_prefix(const TpArgs& a, int r, int d, double top_p, unsigned long long* prefix,
                          unsigned long long* thr_out, unsigned long long* sh, int* win) {
    const unsigned long long* h = a.hist + (size_t)r * kTpPasses * kTpBuckets;
    const int tid = threadIdx.x;
    unsigned long long z = 0ull;
    for (int i = tid; i < kTpBuckets; i += kSThreads) z += h[i];
    const unsigned long long Z = tp_block_scan(z, sh);  // the last thread holds the total
    if (tid == kSThreads - 1) sh[kSThreads] = Z;
    __syncthreads();
    const unsigned long long Zt = sh[kSThreads];
    __syncthreads();
    unsigned long long thr = (unsigned long long)(top_p * (double)Zt);
    if (thr < 1ull) thr = 1ull;
    unsigned long long A = 0ull, pre = 0ull;
    for (int p = 0; p < d; ++p) {
        const int b = tp_select(h + (size_t)p * kTpBuckets, &A, thr, sh, win);
        pre |= (unsigned long long)b << tp_shift(p);
    }
    *prefix = pre;
    *thr_out = thr;
}

// Pass d: the fixed-point masses of the keys that match the prefix, by digit d.
__global__ __launch_bounds__(kSThreads) void tp_hist_kernel(TpArgs a, int d) {
    __shared__ unsigned long long sh[kSThreads + 1];
    __shared__ unsigned long long lh[kTpBuckets];
    __shared__ int win;
    const int r = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
    double T, top_p;
    unsigned long long seed;
    tp_params(a, T, top_p, seed);
    const double m = (double)key_logit(tp_row_max(a, r));
    unsigned long long pre = 0ull, thr = 0ull;
    if (d > 0) tp_prefix(a, r, d, top_p, &pre, &thr, sh, &win);
    for (int i = tid; i < kTpBuckets; i += kSThreads) lh[i] = 0ull;
    __syncthreads();
    const int hi = d > 0 ? tp_shift(d - 1) : 64;  // bits at and above hi are fixed
    const float* row = a.logits + (size_t)r * a.V;
    for (int i = 0; i < kPer; ++i) {
        const int idx = chunk * kChunk + i * kSThreads + tid;
        if (idx >= a.V) continue;
        const float l = row[idx];
        const unsigned long long k = order_key(l, idx);
        if (hi < 64 && (k >> hi) != (pre >> hi)) continue;
        const int digit = (int)((k >> tp_shift(d)) & ((1ull << tp_bits(d)) - 1ull));
        const unsigned long long e = (unsigned long long)rint(exp(((double)l - m) / T) * kTpScale);
        if (e) atomicAdd(&lh[digit], e);
    }
    __syncthreads();
    unsigned long long* h = a.hist + ((size_t)r * kTpPasses + d) * kTpBuckets;
    for (int i = tid; i < kTpBuckets; i += kSThreads)
        if (lh[i]) atomicAdd(&h[i], lh[i]);
}

// The keyed argmax over the kept tokens (keys >= the last kept key), per
// chunk: the best and second-best perturbed scores (lower id on equal scores).
__global__ __launch_bounds__(kSThreads) void tp_pick_kernel(TpArgs a) {
    __shared__ unsigned long long sh[kSThreads + 1];
    __shared__ double zs[kSThreads / 64];
    __shared__ int ids[kSThreads / 64];
    __shared__ int win;
    const int r = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    double T, top_p;
    unsigned long long seed;
    tp_params(a, T, top_p, seed);
    unsigned long long kstar = 0ull, thr = 0ull;
    tp_prefix(a, r, kTpPasses, top_p, &kstar, &thr, sh, &win);
    const long long pos = a.positions[r];
    const float* row = a.logits + (size_t)r * a.V;
    double z[kPer];
    int id[kPer];
    double bz = -__builtin_huge_val();
    int bid = 0x7fffffff;
    for (int i = 0; i < kPer; ++i) {
        const int idx = chunk * kChunk + i * kSThreads + tid;
        z[i] = -__builtin_huge_val();
        id[i] = 0x7fffffff;
        if (idx >= a.V) continue;
        const float l = row[idx];
        if (order_key(l, idx) < kstar) continue;
        z[i] = (double)l / T + keyed_gumbel(seed, pos, idx);
        id[i] = idx;
        if (z[i] > bz || (z[i] == bz && idx < bid)) {
            bz = z[i];
            bid = idx;
        }
    }
    // the chunk's best (z desc, id asc)
    for (int off = 32; off >= 1; off >>= 1) {
        const double oz = __shfl_xor(bz, off, 64);
        const int oid = __shfl_xor(bid, off, 64);
        if (oz > bz || (oz == bz && oid < bid)) {
            bz = oz;
            bid = oid;
        }
    }
    if (lane == 0) {
        zs[w] = bz;
        ids[w] = bid;
    }
    __syncthreads();
    double cz = zs[0];
    int cid = ids[0];
    for (int u = 1; u < kSThreads / 64; ++u)
        if (zs[u] > cz || (zs[u] == cz && ids[u] < cid)) {
            cz = zs[u];
            cid = ids[u];
        }
    __syncthreads();
    // the best score among the chunk's other kept tokens
    double sz = -__builtin_huge_val();
    for (int i = 0; i < kPer; ++i)
        if (id[i] != 0x7fffffff && id[i] != cid) sz = z[i] > sz ? z[i] : sz;
    for (int off = 32; off >= 1; off >>= 1) {
        const double oz = __shfl_xor(sz, off, 64);
        sz = oz > sz ? oz : sz;
    }
    if (lane == 0) zs[w] = sz;
    __syncthreads();
    if (tid == 0) {
        double s2 = zs[0];
        for (int u = 1; u < kSThreads / 64; ++u) s2 = zs[u] > s2 ? zs[u] : s2;
        double* o = a.best + ((size_t)r * kMaxChunks + chunk) * 4;
        o[0] = cz;
        o[1] = s2;
        o[2] = (double)cid;
    }
}

// The row's token: the best of the chunks' bests (lower id on equal scores);
// gap = best - the best score among all other kept tokens.
__global__ __launch_bounds__(64) void tp_merge_kernel(TpArgs a) {
    const int r = blockIdx.x, lane = threadIdx.x;
    double z1 = -__builtin_huge_val(), z2 = -__builtin_huge_val();
    int id1 = 0x7fffffff;
    if (lane < a.nchunk) {
        const double* o = a.best + ((size_t)r * kMaxChunks + lane) * 4;
        z1 = o[0];
        z2 = o[1];
        id1 = (int)o[2];
    }
    double bz = z1;
    int bid = id1;
    for (int off = 32; off >= 1; off >>= 1) {
        const double oz = __shfl_xor(bz, off, 64);
        const int oid = __shfl_xor(bid, off, 64);
        if (oz > bz || (oz == bz && oid < bid)) {
            bz = oz;
            bid = oid;
        }
    }
    // second: the other chunks' bests and every chunk's second best
    double sz = id1 == bid ? z2 : (z1 > z2 ? z1 : z2);
    for (int off = 32; off >= 1; off >>= 1) {
        const double oz = __shfl_xor(sz, off, 64);
        sz = oz > sz ? oz : sz;
    }
    if (lane == 0) {
        a.tokens[r] = bid;
        if (a.gap) a.gap[r] = sz == -__builtin_huge_val() ? __builtin_huge_val() : bz - sz;
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
        if (s.top_k < 0) return fail(EV_EINVAL, "%s: top_k=%d", who, s.top_k);
        if (s.top_k > EV_MAX_TOPK) return fail(EV_EUNSUPPORTED, "%s: top_k=%d above 64", who, s.top_k);
        if (!(s.top_p > 0.0 && s.top_p <= 1.0)) return fail(EV_EINVAL, "%s: top_p outside (0,1]", who);
    }
    return EV_OK;
}
}  // namespace ev

// Workspace: the top-k candidate lists [16][nchunk][64], then for top-p over
// the whole vocabulary the chunk maxima [16][64], the select histograms
// [16][6][2048] and the chunks' best scores [16][64][4].
static size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }
static size_t tp_off_cmax(int V) { return al256((size_t)EV_MAX_LANES * sample_nchunk(V) * EV_MAX_TOPK * 8); }
static size_t tp_off_hist() { return al256((size_t)EV_MAX_LANES * kMaxChunks * 8); }
static size_t tp_off_best() { return al256((size_t)EV_MAX_LANES * kTpPasses * kTpBuckets * 8); }

extern "C" size_t keyed_sample_workspace(int32_t V) {
    if (V <= 0) return 0;
    return tp_off_cmax(V) + tp_off_hist() + tp_off_best() + (size_t)EV_MAX_LANES * kMaxChunks * 4 * sizeof(double);
}

// Checks the shapes and pointers of a keyed sample (the sampling parameters
// are checked by the caller).
static int32_t check_sample_args(const char* who, const float* logits, int32_t R, int32_t V,
                                 const int64_t* positions, int32_t* tokens, double* gap) {
    if (R < 1 || R > EV_MAX_LANES) return fail(EV_EINVAL, "%s: R=%d outside 1..16", who, R);
    if (V < 1) return fail(EV_EINVAL, "%s: V=%d", who, V);
    if (V > kMaxChunks * kChunk) return fail(EV_EUNSUPPORTED, "%s: V=%d above %d", who, V, kMaxChunks * kChunk);
    if (!logits || !positions || !tokens) return fail(EV_EINVAL, "%s: NULL pointer", who);
    if (!aligned(logits, 4) || !aligned(positions, 8) || !aligned(tokens, 4) || (gap && !aligned(gap, 8)))
        return fail(EV_EINVAL, "%s: misaligned pointer", who);
    return EV_OK;
}

static int32_t check_sample_ws(const char* who, int32_t V, void* ws, size_t ws_bytes) {
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
                            const ev_sampling* sd, int32_t* tokens, double* gap, void* ws, hipStream_t st,
                            const FusedAccept* acc) {
    const int nchunk = sample_nchunk(V);
    if (s.temperature > 0.0 && s.top_k == 0) {  // top-p over the whole vocabulary
        unsigned char* b = reinterpret_cast<unsigned char*>(ws);
        const size_t oc = tp_off_cmax(V), oh = oc + tp_off_hist(), ob = oh + tp_off_best();
        TpArgs a{logits, V, nchunk, positions, s.temperature, s.top_p, (unsigned long long)s.seed, sd,
                 reinterpret_cast<unsigned long long*>(b + oc), reinterpret_cast<unsigned long long*>(b + oh),
                 reinterpret_cast<double*>(b + ob), tokens, gap};
        const dim3 grid(nchunk, R);
        hipLaunchKernelGGL(tp_max_kernel, grid, dim3(kSThreads), 0, st, a);
        for (int d = 0; d < kTpPasses; ++d) hipLaunchKernelGGL(tp_hist_kernel, grid, dim3(kSThreads), 0, st, a, d);
        hipLaunchKernelGGL(tp_pick_kernel, grid, dim3(kSThreads), 0, st, a);
        hipLaunchKernelGGL(tp_merge_kernel, dim3(R), dim3(64), 0, st, a);
        if (acc)  // here the accept prefix stays a launch of its own
            hipLaunchKernelGGL(accept_kernel, dim3(1), dim3(64), 0, st, tokens, R, acc->draft, acc->D,
                               acc->n_accept, acc->n_commit);
        return check_hip(hipGetLastError(), "top-p launches");
    }
    const int kk = sample_kk_of(s.temperature, s.top_k, V);
    unsigned long long* cand = reinterpret_cast<unsigned long long*>(ws);
    hipLaunchKernelGGL(topk_chunk_kernel, dim3(nchunk, R), dim3(kSThreads), 0, st, logits, V, kk, nchunk, sd,
                       cand, acc ? acc->count : nullptr);
    int32_t rc = check_hip(hipGetLastError(), "topk_chunk launch");
    if (rc) return rc;
    SampleArgs a{cand, positions, nchunk, kk, V, s.temperature, s.top_p, (unsigned long long)s.seed, sd,
                 tokens, gap, acc ? *acc : FusedAccept{}, R};
    hipLaunchKernelGGL(merge_sample_kernel, dim3(R), dim3(kMThreads), 0, st, a);
    return check_hip(hipGetLastError(), "merge_sample launch");
}
}  // namespace ev

extern "C" int32_t keyed_sample(const float* logits, int32_t R, int32_t V, const int64_t* positions,
                                ev_sampling s, int32_t* tokens, double* gap, void* ws,
                                size_t ws_bytes, void* stream) {
    clear_error();
    const char* who = "keyed_sample";
    int32_t rc;
    if ((rc = check_sample_args(who, logits, R, V, positions, tokens, gap))) return rc;
    if ((rc = check_sampling(who, s))) return rc;
    if ((rc = check_sample_ws(who, V, ws, ws_bytes))) return rc;
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
