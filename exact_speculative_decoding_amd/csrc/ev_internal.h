// Internal helpers of libexactverify (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "exactverify.h"

namespace ev {

// Set the thread-local error message and return `code`.
int32_t fail(int32_t code, const char* fmt, ...);
// Clear the error message (called at the start of every entry point).
void clear_error();
// Check the result of a launch / runtime call.
int32_t check_hip(hipError_t e, const char* what);

// Sampling parameters as keyed_sample accepts them (EV_OK or the error code).
int32_t check_sampling(const char* who, const ev_sampling& s);

// The launches of keyed_sample on checked arguments; with `sd` (device) the
// kernels read the sampling parameters there rather than from `s`, which then
// only has to give a valid top-k for the launch's candidate count bound.
// The accept prefix folded into the top-k sampler's last workgroup (the verify
// step): n_accept = leading i < D with draft[i] == tokens[i], n_commit =
// min(n_accept + 1, R); `count` is a device int the sampler's first kernel
// clears and its last workgroup to finish restores to zero.
struct FusedAccept {
    int* count;
    const int32_t* draft;
    int D;
    int32_t* n_accept;
    int32_t* n_commit;
};
int32_t launch_keyed_sample(const float* logits, int R, int V, const long long* positions, const ev_sampling& s,
                            const ev_sampling* sd, int32_t* tokens, double* gap, void* ws, hipStream_t st,
                            const FusedAccept* acc = nullptr);

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---- device helpers -------------------------------------------------------

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even fp32 -> bf16 bits; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// fp32 -> fp16 bits, round to nearest even (the hardware conversion).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// fp32 -> fp16 bits for a cache entry: clamped to the finite range (+-65504)
// first, then rounded to nearest even, so that no entry is ever infinite (an
// infinite value in a slot that a row masks out with weight 0 would turn the
// row's sum into NaN).
__device__ __forceinline__ uint16_t f32_to_f16_sat(float v) {
    const float c = fabsf(v) > 65504.f ? copysignf(65504.f, v) : v;
    return f32_to_f16_bits(c);
}

// fp16 bits -> fp32 (exact) via the hardware conversion.
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    _Float16 v = __builtin_bit_cast(_Float16, h);
    return (float)v;
}

// Order key of (value l, index id): a larger key comes earlier in the order
// (l desc, id asc).  -0 and +0 compare equal as values, so -0 is folded onto
// +0.  Key 0 is below every real key.
__device__ __forceinline__ unsigned long long order_key(float l, int id) {
    uint32_t u = __float_as_uint(l);
    if ((u & 0x7fffffffu) == 0u) u = 0u;
    const uint32_t ok = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)ok << 32) | (unsigned long long)(~(uint32_t)id);
}
__device__ __forceinline__ float key_logit(unsigned long long k) {
    const uint32_t ok = (uint32_t)(k >> 32);
    const uint32_t u = (ok & 0x80000000u) ? (ok & 0x7fffffffu) : ~ok;
    return __uint_as_float(u);
}
__device__ __forceinline__ int key_id(unsigned long long k) { return (int)(~(uint32_t)k); }

// Maximum of v over the 64 lanes of the wave, returned to every lane.  DPP
// moves (VALU, no LDS round trip): prefix maxima within each row of 16 lanes
// (row_shr 1, 2, 4, 8), then rows 0..1 and 2..3 via row_bcast15, then all via
// row_bcast31, so lane 63 holds the maximum; max is exact in any order.
__device__ __forceinline__ unsigned long long dpp_max_step(unsigned long long v, int ctrl_sel) {
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    uint32_t olo, ohi;
    // lanes without a source keep their own value (bound_ctrl off)
    switch (ctrl_sel) {
        case 0: olo = __builtin_amdgcn_update_dpp(lo, lo, 0x111, 0xf, 0xf, false);
                ohi = __builtin_amdgcn_update_dpp(hi, hi, 0x111, 0xf, 0xf, false); break;  // row_shr:1
        case 1: olo = __builtin_amdgcn_update_dpp(lo, lo, 0x112, 0xf, 0xf, false);
                ohi = __builtin_amdgcn_update_dpp(hi, hi, 0x112, 0xf, 0xf, false); break;  // row_shr:2
        case 2: olo = __builtin_amdgcn_update_dpp(lo, lo, 0x114, 0xf, 0xf, false);
                ohi = __builtin_amdgcn_update_dpp(hi, hi, 0x114, 0xf, 0xf, false); break;  // row_shr:4
        case 3: olo = __builtin_amdgcn_update_dpp(lo, lo, 0x118, 0xf, 0xf, false);
                ohi = __builtin_amdgcn_update_dpp(hi, hi, 0x118, 0xf, 0xf, false); break;  // row_shr:8
        case 4: olo = __builtin_amdgcn_update_dpp(lo, lo, 0x142, 0xa, 0xf, false);
                ohi = __builtin_amdgcn_update_dpp(hi, hi, 0x142, 0xa, 0xf, false); break;  // row_bcast:15
        default: olo = __builtin_amdgcn_update_dpp(lo, lo, 0x143, 0xc, 0xf, false);
                 ohi = __builtin_amdgcn_update_dpp(hi, hi, 0x143, 0xc, 0xf, false); break;  // row_bcast:31
    }
    const unsigned long long o = ((unsigned long long)ohi << 32) | olo;
    return o > v ? o : v;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
    for (int k = 0; k < 6; ++k) v = dpp_max_step(v, k);
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 63);
    return ((unsigned long long)hi << 32) | lo;
}

}  // namespace ev
