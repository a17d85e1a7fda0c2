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

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

}  // namespace ev
