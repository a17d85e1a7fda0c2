// MoE verify layer on gfx950: per-lane top-k routing, grouping of the lanes by
// expert, one grouped W4 pass over the touched experts, and a combine in rank
// order.
//
// Each lane (row) of the verify pass is routed on its own: pi = softmax of its
// router logits, the top experts by pi (lower expert id on ties), weights
// renormalised over the selected experts, output = sum over the selected
// experts in rank order of weight * SiLU-gated MLP of that expert.  The pages'
// MoE models (Nemotron 30B-A3B in the TensorFold README's model notes and the
// blog's "The numbers") run their verify rows through this layer; row
// exactness ([README] exactness paragraph) requires that a lane's output not
// depend on which other lanes share an expert.  That holds here because
//   * routing, grouping order and the combine are per lane;
//   * an expert's pass pads its lanes to the 16 rows of the MFMA tile, and an
//     MFMA output row depends only on its own input row;
//   * the split plans of gate/up and down follow from (H, I) only.
//
// Launches (all on the caller's stream, none depending on R except grids):
//   moe_route_kernel    1 x 1024: routing of all lanes (a wave each), then per
//                       expert its lanes in ascending order, the list of
//                       touched experts in ascending id, and each (lane,
//                       rank)'s place;
//   w4_pair_kernel      grouped: h = bf16(silu(gate) * up) per expert row, gate
//                       and up of every touched expert in one paired pass;
//   w4_verify_kernel    grouped: down of every touched expert;
//   moe_combine_kernel  per lane: split sums, then the weighted sum in rank order.
#include "w4_kernel.h"

namespace ev {

constexpr int kMoeMaxE = 256;   // experts
constexpr int kMoeMaxTop = 8;   // experts per lane

struct MoeTables {
    int* ids;     // [16][kMoeMaxTop] selected experts per lane, in rank order
    float* w;     // [16][kMoeMaxTop] their renormalised weights
    int* pos;     // [16][kMoeMaxTop] 16 * group + tile row of (lane, rank)
    int* gcount;  // [1] touched experts
    int* gexp;    // [gmax] expert of each group, ascending
    int* gcnt;    // [gmax] lanes of each group
    int* grows;   // [gmax][16] lane of each tile row (0 past gcnt)
    int* ids_out;    // optional caller copies [R][top]
    float* w_out;
};

// One workgroup of 16 waves.  Wave r routes lane r; experts are then grouped
// through a 16-bit mask per expert of the lanes that chose it (a lane picks an
// expert at most once): its popcount is the group's lane count, the lanes
// below r give lane r's row in the group, and a ballot scan over the experts
// numbers the touched ones in ascending id.
constexpr int kRouteThreads = 1024;
__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(const float* __restrict__ rho, int R, int E,
                                                                  int top, MoeTables t) {
    __shared__ int sids[16][kMoeMaxTop];
    __shared__ unsigned smask[kMoeMaxE];
    __shared__ int sgid[kMoeMaxE];
    __shared__ int swave[kMoeMaxE / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < E) smask[tid] = 0u;
    __syncthreads();

    // wave r: keys of lane r's E logits, `top` rounds of a wave max
    if (wave < R) {
        const int r = wave;
        unsigned long long key[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // clamped index, masked key: the four loads in flight together
            const int e = lane + 64 * i;
            const float v = rho[(size_t)r * E + (e < E ? e : E - 1)];
            key[i] = order_key(v, e) & (0ull - (unsigned long long)(e < E));
        }
        float lsel[kMoeMaxTop];
        int isel[kMoeMaxTop];
#pragma unroll
        for (int j = 0; j < kMoeMaxTop; ++j) {
            lsel[j] = 0.f;
            isel[j] = 0;
            if (j < top) {
                unsigned long long mine = key[0];
#pragma unroll
                for (int i = 1; i < 4; ++i) mine = key[i] > mine ? key[i] : mine;
                const unsigned long long best = wave_max_u64(mine);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (key[i] == best) key[i] = 0ull;  // keys are unique (the id is in them)
                lsel[j] = key_logit(best);
                isel[j] = key_id(best);
            }
        }
        if (lane == 0) {
            // pi_j / sum of the selected pi = e^(l_j - l_0) / sum of the same
            float ev[kMoeMaxTop], sum = 0.f;
#pragma unroll
            for (int j = 0; j < kMoeMaxTop; ++j) {
                ev[j] = j < top ? expf(lsel[j] - lsel[0]) : 0.f;
                sum += ev[j];
            }
#pragma unroll
            for (int j = 0; j < kMoeMaxTop; ++j) {
                if (j < top) {
                    const float wj = ev[j] / sum;
                    sids[r][j] = isel[j];
                    atomicOr(&smask[isel[j]], 1u << r);
                    t.ids[r * kMoeMaxTop + j] = isel[j];
                    t.w[r * kMoeMaxTop + j] = wj;
                    if (t.ids_out) t.ids_out[r * top + j] = isel[j];
                    if (t.w_out) t.w_out[r * top + j] = wj;
                }
            }
        }
    }
    __syncthreads();

    // thread e: touched or not; the touched experts' group ids in ascending e
    const unsigned msk = tid < E ? smask[tid] : 0u;
    const bool touched = msk != 0u;
    const unsigned long long bal = __ballot(touched);
    if (tid < E && lane == 0) swave[wave] = __popcll(bal);
    __syncthreads();
    if (tid < E) {
        int g = __popcll(bal & ((1ull << lane) - 1ull));
        for (int v = 0; v < wave; ++v) g += swave[v];
        sgid[tid] = touched ? g : -1;
        if (tid == E - 1) t.gcount[0] = g + (touched ? 1 : 0);
        if (touched) {
            t.gexp[g] = tid;
            t.gcnt[g] = __popc(msk);
            unsigned rest = msk;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                t.grows[16 * g + m] = rest ? __ffs(rest) - 1 : 0;  // lanes in ascending order, then 0
                rest &= rest - 1u;
            }
        }
    }
    __syncthreads();

    // (lane r, rank j): row 16 g + (lanes below r in the group)
    if (wave < R && lane < top) {
        const int r = wave, e = sids[r][lane];
        t.pos[r * kMoeMaxTop + lane] = 16 * sgid[e] + __popc(smask[e] & ((1u << r) - 1u));
    }
}

// y[r][n] = sum over ranks j = 0..top-1, in order, of w[r][j] * e_j[n], with
// e_j the down projection of lane r in its j-th expert (its split partials
// added in ascending split order).  One thread per 4 consecutive n.
__global__ __launch_bounds__(64) void moe_combine_kernel(const float* __restrict__ pd, int S, int H,
                                                         long gstride, int gmax,
                                                         const int* __restrict__ pos,
                                                         const float* __restrict__ w, int top,
                                                         float* __restrict__ y) {
    const int n4 = (blockIdx.x * 64 + threadIdx.x) * 4;
    const int r = blockIdx.y;
    if (n4 >= H) return;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < top; ++j) {
        const int p = pos[r * kMoeMaxTop + j];
        if ((unsigned)(p >> 4) >= (unsigned)gmax) continue;  // cannot happen: every (lane, rank) is placed
        const float* b = pd + (size_t)(p >> 4) * gstride + (size_t)(p & 15) * H + n4;
        f32x4 v = *reinterpret_cast<const f32x4*>(b);
        for (int s = 1; s < S; ++s) v += *reinterpret_cast<const f32x4*>(b + (size_t)s * 16 * H);
        acc += w[r * kMoeMaxTop + j] * v;
    }
    *reinterpret_cast<f32x4*>(y + (size_t)r * H + n4) = acc;
}

// Workspace: routing tables, then h [gmax][16][I] bf16 and down partials
// [gmax][S2][16][H]; gmax = min(E, 16 top) groups at most.  A function of
// (H, I, E, top) only.
struct MoeLayout {
    W4Plan p1, p2;
    int gmax;
    size_t off_w, off_pos, off_gcount, off_gexp, off_gcnt, off_grows, off_h, off_pd, total;
};
static MoeLayout moe_layout(int H, int I, int E, int top) {
    MoeLayout L;
    L.p1 = plan_w4_pair(I, H);
    L.p2 = plan_w4(H, I, 1);
    L.gmax = E < 16 * top ? E : 16 * top;
    const size_t tab = align256(sizeof(int) * 16 * kMoeMaxTop);
    L.off_w = tab;
    L.off_pos = 2 * tab;
    L.off_gcount = 3 * tab;
    L.off_gexp = L.off_gcount + 256;
    L.off_gcnt = L.off_gexp + align256(sizeof(int) * L.gmax);
    L.off_grows = L.off_gcnt + align256(sizeof(int) * L.gmax);
    L.off_h = L.off_grows + align256(sizeof(int) * 16 * L.gmax);
    L.off_pd = L.off_h + align256((size_t)L.gmax * 16 * I * sizeof(uint16_t));
    L.total = L.off_pd + align256((size_t)L.gmax * L.p2.S * 16 * H * sizeof(float));
    return L;
}

static int32_t check_moe_dims(const char* who, int H, int I, int E, int top, int G) {
    int32_t rc;
    if ((rc = check_w4_dims(who, H, I, G)) || (rc = check_w4_dims(who, I, H, G))) return rc;
    if (E < 1 || E > kMoeMaxE) return fail(EV_EUNSUPPORTED, "%s: E=%d experts (1..%d)", who, E, kMoeMaxE);
    if (top < 1 || top > kMoeMaxTop || top > E)
        return fail(EV_EUNSUPPORTED, "%s: top=%d experts per lane (1..%d, <= E)", who, top, kMoeMaxTop);
    return EV_OK;
}

}  // namespace ev

using namespace ev;

extern "C" size_t verify_moe_w4_workspace(int32_t H, int32_t I, int32_t E, int32_t top, int32_t G) {
    if (H <= 0 || I <= 0 || E < 1 || E > kMoeMaxE || top < 1 || top > kMoeMaxTop || top > E ||
        (G != 32 && G != 64))
        return 0;
    return moe_layout(H, I, E, top).total;
}

extern "C" int32_t verify_moe_w4(const uint16_t* x, const float* router, int32_t R, int32_t H, int32_t I,
                                 int32_t E, int32_t top, int32_t G, const void* w_gate, const void* w_up,
                                 const void* w_down, float* y, int32_t* expert_ids, float* expert_w,
                                 void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    const char* who = "verify_moe_w4";
    int32_t rc;
    if ((rc = check_lanes(who, R)) || (rc = check_moe_dims(who, H, I, E, top, G))) return rc;
    if (!x || !router || !w_gate || !w_up || !w_down || !y) return fail(EV_EINVAL, "%s: NULL pointer", who);
    if (!aligned(x, 16) || !aligned(router, 4) || !aligned(w_gate, 16) || !aligned(w_up, 16) ||
        !aligned(w_down, 16) || !aligned(y, 16) || (expert_ids && !aligned(expert_ids, 4)) ||
        (expert_w && !aligned(expert_w, 4)))
        return fail(EV_EINVAL, "%s: misaligned pointer (x, weights, y 16 B; router, ids, w 4 B)", who);
    const MoeLayout L = moe_layout(H, I, E, top);
    if ((rc = check_ws(who, ws, ws_bytes, L.total))) return rc;
    const size_t hbytes = (size_t)L.gmax * 16 * I * sizeof(uint16_t);
    if (hbytes >= (1ull << 31)) return fail(EV_EUNSUPPORTED, "%s: expert activations exceed 2^31 bytes", who);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    unsigned char* b = reinterpret_cast<unsigned char*>(ws);
    MoeTables t;
    t.ids = reinterpret_cast<int*>(b);
    t.w = reinterpret_cast<float*>(b + L.off_w);
    t.pos = reinterpret_cast<int*>(b + L.off_pos);
    t.gcount = reinterpret_cast<int*>(b + L.off_gcount);
    t.gexp = reinterpret_cast<int*>(b + L.off_gexp);
    t.gcnt = reinterpret_cast<int*>(b + L.off_gcnt);
    t.grows = reinterpret_cast<int*>(b + L.off_grows);
    t.ids_out = expert_ids;
    t.w_out = expert_w;
    uint16_t* h = reinterpret_cast<uint16_t*>(b + L.off_h);
    float* pd = reinterpret_cast<float*>(b + L.off_pd);
    // groups launched: at most the distinct experts R lanes can touch
    const int ng = E < top * R ? E : top * R;

    hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(kRouteThreads), 0, st, router, R, E, top, t);
    if ((rc = check_hip(hipGetLastError(), "moe_route launch"))) return rc;

    W4Args a{};
    a.w[0] = reinterpret_cast<const uint8_t*>(w_gate);
    a.w[1] = reinterpret_cast<const uint8_t*>(w_up);
    a.x = x;
    a.R = R;
    a.N = I;
    a.h = h;
    a.hgstride = (long)16 * I;
    a.gcount = t.gcount;
    a.gexp = t.gexp;
    a.gcnt = t.gcnt;
    a.grows = t.grows;
    a.wstride = (long)w4_blob_bytes(I, H, G);
    a.xbytes = (uint32_t)((size_t)R * H * sizeof(uint16_t));
    if ((rc = launch_w4_pair(a, L.p1, H, G, st, ng))) return rc;

    W4Args d{};
    d.w[0] = d.w[1] = reinterpret_cast<const uint8_t*>(w_down);
    d.out[0] = d.out[1] = pd;
    d.x = h;
    d.R = 16;
    d.N = H;
    d.split_stride = (long)16 * H;
    d.gcount = t.gcount;
    d.gexp = t.gexp;
    d.gcnt = t.gcnt;
    d.grows = nullptr;  // the rows of group g are h rows 16 g + r
    d.wstride = (long)w4_blob_bytes(H, I, G);
    d.ogstride = (long)L.p2.S * 16 * H;
    d.xbytes = (uint32_t)((size_t)ng * 16 * I * sizeof(uint16_t));
    if ((rc = launch_w4(d, 1, L.p2, I, G, st, ng))) return rc;

    dim3 grid((unsigned)((H / 4 + 63) / 64), (unsigned)R);
    hipLaunchKernelGGL(moe_combine_kernel, grid, dim3(64), 0, st, pd, L.p2.S, H, (long)L.p2.S * 16 * H, ng, t.pos,
                       t.w, top, y);
    return check_hip(hipGetLastError(), "moe_combine launch");
}
