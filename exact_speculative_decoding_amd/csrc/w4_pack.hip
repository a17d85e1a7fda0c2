// Exact repacking of W4 weights (once, at load) into the layout of
// w4_layout.h.  Pure data movement: every output value is a copy of an input
// value or a padding zero.
#include "w4_kernel.h"  // the layout, and the argument checks of the entry points

namespace ev {

// The 8 codes q0..q7 of a standard dword (q_i in bits 4i..4i+3) with the
// even-k codes moved to the low half and the odd-k codes to the high half:
// nibbles, low to high, q0 q2 q4 q6 q1 q3 q5 q7.  q_{2m} and q_{2m+1} then sit
// exactly 16 bits apart, so one shift and mask places both in a bf16 pair.
__device__ __forceinline__ uint32_t nibble_split(uint32_t w) {
    uint32_t e = w & 0x0F0F0F0Fu, o = (w >> 4) & 0x0F0F0F0Fu;
    e = (e | (e >> 4)) & 0x00FF00FFu;
    o = (o | (o >> 4)) & 0x00FF00FFu;
    e = (e | (e >> 8)) & 0x0000FFFFu;
    o = (o | (o >> 8)) & 0x0000FFFFu;
    return e | (o << 16);
}

// One thread per (tile, chunk, lane): 16 B of codes, plus (for the lanes of
// row group j == 0) the row's (scale, bias) pairs of the chunk.
__global__ void w4_pack_kernel(const uint8_t* __restrict__ q, const uint16_t* __restrict__ s,
                               const uint16_t* __restrict__ b, int N, int K, int G,
                               uint8_t* __restrict__ out) {
    const int NC = w4_chunks(K);
    const long total = (long)w4_tiles(N) * NC * 64;
    const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const int L = (int)(gid & 63);
    const long tc = gid >> 6;
    const int c = (int)(tc % NC);
    const long tile = tc / NC;
    const int ln = L & 15, j = L >> 4;
    const long n = tile * 16 + ln;
    const int GPC = kKC / G;
    uint8_t* dst = out + w4_tc_offset(tile, c, w4_tiles(N), G);
    const size_t Kh = (size_t)K / 2;
    u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int k = kKC * c + 32 * t + 8 * j;
        if (n < N && k < K) w[t] = nibble_split(*reinterpret_cast<const uint32_t*>(q + (size_t)n * Kh + k / 2));
    }
    *reinterpret_cast<u32x4*>(dst + 16 * L) = w;
    if (j == 0) {
        const int KG = K / G;
        for (int g = 0; g < GPC; ++g) {
            const int kg = kKC * c + g * G;
            uint32_t v = 0u;
            if (n < N && kg < K) {
                const size_t o = (size_t)n * KG + kg / G;
                v = (uint32_t)s[o] | ((uint32_t)b[o] << 16);
            }
            *reinterpret_cast<uint32_t*>(dst + 1024 + 4 * (ln * GPC + g)) = v;
        }
    }
}

// NVFP4 packing, one thread per (tile, chunk, lane): dword t of lane (ln, j)
// holds the 8 E2M1 codes of row 16 tile + ln at k = 128 c + 32 t + 4 j + {0..3}
// (bytes 0, 1) and + 16 + {0..3} (bytes 2, 3), low nibble first -- the B
// fragments of the step's two 16 x 16 x 16 MFMA; lanes of row group j == 0
// copy the row's 8 E4M3 block scales of the chunk after the 1 KB of codes.
__device__ __forceinline__ uint32_t fp4_code(const uint8_t* q, size_t Kh, long n, int k) {
    const uint8_t b = q[(size_t)n * Kh + k / 2];
    return (k & 1) ? (uint32_t)(b >> 4) : (uint32_t)(b & 15);
}

__global__ void nvfp4_pack_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s, int N, int K,
                                  uint8_t* __restrict__ out) {
    const int NC = w4_chunks(K);
    const long total = (long)w4_tiles(N) * NC * 64;
    const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const int L = (int)(gid & 63);
    const long tc = gid >> 6;
    const int c = (int)(tc % NC);
    const long tile = tc / NC;
    const int ln = L & 15, j = L >> 4;
    const long n = tile * 16 + ln;
    uint8_t* dst = out + w4_tc_offset(tile, c, w4_tiles(N), 64);
    const size_t Kh = (size_t)K / 2;
    u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t v = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int k = kKC * c + 32 * t + 4 * j + (e & 3) + 16 * (e >> 2);
            if (n < N && k < K) v |= fp4_code(q, Kh, n, k) << (4 * e);
        }
        w[t] = v;
    }
    *reinterpret_cast<u32x4*>(dst + 16 * L) = w;
    if (j == 0) {
        const int KB = K / 16;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int kb = kKC * c + 16 * b;
            dst[1024 + 8 * ln + b] = (n < N && kb < K) ? s[(size_t)n * KB + kb / 16] : (uint8_t)0;
        }
    }
}

int32_t check_w4_dims(const char* who, int K, int N, int G) {
    if (G != 32 && G != 64) return fail(EV_EUNSUPPORTED, "%s: group size %d (32 or 64)", who, G);
    if (K <= 0 || N <= 0) return fail(EV_EINVAL, "%s: K=%d N=%d must be positive", who, K, N);
    if (K % G != 0 || K % 32 != 0)
        return fail(EV_EINVAL, "%s: K=%d must be a multiple of 32 and of G=%d", who, K, G);
    if (w4_blob_bytes(N, K, G) >= (1ull << 31))
        return fail(EV_EUNSUPPORTED, "%s: packed weights of %zu bytes exceed 2^31", who,
                    w4_blob_bytes(N, K, G));
    return EV_OK;
}

}  // namespace ev

using namespace ev;

extern "C" size_t w4_packed_bytes(int32_t N, int32_t K, int32_t G) {
    if (N <= 0 || K <= 0 || (G != 32 && G != 64)) return 0;
    return w4_blob_bytes(N, K, G);
}

extern "C" int32_t w4_pack(const uint8_t* q, const uint16_t* s, const uint16_t* b, int32_t N, int32_t K,
                           int32_t G, void* packed, size_t packed_bytes, void* stream) {
    clear_error();
    const char* who = "w4_pack";
    int32_t rc = check_w4_dims(who, K, N, G);
    if (rc) return rc;
    if (!q || !s || !b || !packed) return fail(EV_EINVAL, "%s: NULL pointer", who);
    if (!aligned(q, 4) || !aligned(s, 2) || !aligned(b, 2) || !aligned(packed, 16))
        return fail(EV_EINVAL, "%s: misaligned pointer (q 4 B, s/b 2 B, packed 16 B)", who);
    if (packed_bytes < w4_blob_bytes(N, K, G))
        return fail(EV_EINVAL, "%s: packed buffer needs %zu bytes, got %zu", who, w4_blob_bytes(N, K, G),
                    packed_bytes);
    const long total = (long)w4_tiles(N) * w4_chunks(K) * 64;
    hipLaunchKernelGGL(w4_pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), q, s, b, N, K, G,
                       reinterpret_cast<uint8_t*>(packed));
    return check_hip(hipGetLastError(), "w4_pack launch");
}

extern "C" size_t nvfp4_packed_bytes(int32_t N, int32_t K) {
    if (N <= 0 || K <= 0) return 0;
    return w4_blob_bytes(N, K, 64);
}

extern "C" int32_t nvfp4_pack(const uint8_t* q, const uint8_t* s, int32_t N, int32_t K, void* packed,
                              size_t packed_bytes, void* stream) {
    clear_error();
    const char* who = "nvfp4_pack";
    int32_t rc = check_w4_dims(who, K, N, 32);  // K a multiple of 32
    if (rc) return rc;
    if (!q || !s || !packed) return fail(EV_EINVAL, "%s: NULL pointer", who);
    if (!aligned(packed, 16)) return fail(EV_EINVAL, "%s: misaligned packed buffer (16 B)", who);
    if (packed_bytes < w4_blob_bytes(N, K, 64))
        return fail(EV_EINVAL, "%s: packed buffer needs %zu bytes, got %zu", who, w4_blob_bytes(N, K, 64),
                    packed_bytes);
    const long total = (long)w4_tiles(N) * w4_chunks(K) * 64;
    hipLaunchKernelGGL(nvfp4_pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), q, s, N, K, reinterpret_cast<uint8_t*>(packed));
    return check_hip(hipGetLastError(), "nvfp4_pack launch");
}

// ---- the linear on standard-layout weights ---------------------------------
// The matrix is packed into the front of the workspace (w4_pack, an exact
// byte permutation), then the packed launches run on the rest: the same
// arithmetic as verify_linear_w4 on a matrix packed once at load, at the
// cost of streaming the weights twice per call.
static size_t std_pack_bytes(int32_t K, int32_t N, int32_t G) { return (w4_blob_bytes(N, K, G) + 255) & ~(size_t)255; }

extern "C" size_t verify_linear_w4_standard_workspace(int32_t K, int32_t N, int32_t G) {
    if (K <= 0 || N <= 0 || (G != 32 && G != 64) || K % G != 0 || K % 32 != 0) return 0;
    return std_pack_bytes(K, N, G) + verify_linear_w4_workspace(K, N, G);
}

extern "C" int32_t verify_linear_w4_standard(const uint16_t* x, int32_t R, int32_t K, const uint8_t* q,
                                             const uint16_t* scale_f16, const uint16_t* bias_f16, int32_t N,
                                             int32_t G, float* y, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    const char* who = "verify_linear_w4_standard";
    int32_t rc;
    // every check of both steps before either launches
    if ((rc = check_lanes(who, R)) || (rc = check_w4_dims(who, K, N, G))) return rc;
    if (!x || !q || !scale_f16 || !bias_f16 || !y) return fail(EV_EINVAL, "%s: NULL pointer", who);
    if (!aligned(x, 16) || !aligned(q, 4) || !aligned(scale_f16, 2) || !aligned(bias_f16, 2) || !aligned(y, 4))
        return fail(EV_EINVAL, "%s: misaligned pointer (x 16 B, q 4 B, scale/bias 2 B, y 4 B)", who);
    const size_t pack = std_pack_bytes(K, N, G);
    if ((rc = check_ws(who, ws, ws_bytes, pack + verify_linear_w4_workspace(K, N, G)))) return rc;
    unsigned char* wsb = reinterpret_cast<unsigned char*>(ws);
    if ((rc = w4_pack(q, scale_f16, bias_f16, N, K, G, wsb, pack, stream))) return rc;
    return verify_linear_w4(x, R, K, wsb, N, G, y, wsb + pack, ws_bytes - pack, stream);
}
