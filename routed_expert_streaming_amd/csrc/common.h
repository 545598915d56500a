// Shared helpers of the HIP library: error reporting, numeric formats and wave
// reductions for gfx950 (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Thread-local error state behind moe_last_hip_error / moe_last_error_message.
int fail(int status, const char *fmt, ...);
int fail_hip(hipError_t err, const char *what);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace moe

#define MOE_TRY_HIP(expr)                                   \
    do {                                                    \
        hipError_t _e = (expr);                             \
        if (_e != hipSuccess) return moe::fail_hip(_e, #expr); \
    } while (0)

// Launch then check the launch status.
#define MOE_LAUNCH_CHECK(what)                               \
    do {                                                     \
        hipError_t _e = hipGetLastError();                   \
        if (_e != hipSuccess) return moe::fail_hip(_e, what); \
    } while (0)

// ------------------------------------------------------------------ device helpers
typedef __bf16 moe_bf16x2 __attribute__((ext_vector_type(2)));

typedef unsigned int moe_u32x4 __attribute__((ext_vector_type(4)));

// Build-time tuning knobs of the weight-streaming kernels (defaults are the
// tuned values; see the build script for how to override them).
#ifndef MOE_STREAM_NT
#define MOE_STREAM_NT 0  // 1: weight loads marked non-temporal
#endif

// Global-address-space views: loads through them compile to global_load (not
// flat_load, which would also count against the LDS wait counter and make every
// LDS wait drain the weight stream).
typedef __attribute__((address_space(1))) const moe_u32x4 moe_gu32x4;
typedef __attribute__((address_space(1))) const uint32_t moe_gu32;

// Weight loads: every weight byte is read once per launch.
__device__ __forceinline__ uint4 load_stream_u4(const void *p) {
    const moe_gu32x4 *g = (const moe_gu32x4 *)p;
#if MOE_STREAM_NT
    const moe_u32x4 v = __builtin_nontemporal_load(g);
#else
    const moe_u32x4 v = *g;
#endif
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t load_stream_u32(const void *p) {
    const moe_gu32 *g = (const moe_gu32 *)p;
#if MOE_STREAM_NT
    return __builtin_nontemporal_load(g);
#else
    return *g;
#endif
}
__device__ __forceinline__ uint32_t load_stream_u8(const void *p) {
    typedef __attribute__((address_space(1))) const uint8_t moe_gu8;
    const moe_gu8 *g = (const moe_gu8 *)p;
#if MOE_STREAM_NT
    return __builtin_nontemporal_load(g);
#else
    return *g;
#endif
}
// Plain global loads of small operands (activations, tables).
__device__ __forceinline__ uint4 load_global_u4(const void *p) {
    const moe_u32x4 v = *(const moe_gu32x4 *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float fp16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// acc + a.lo*b.lo + a.hi*b.hi with bf16 pairs packed in 32-bit words.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(moe_bf16x2, a), __builtin_bit_cast(moe_bf16x2, b),
                                           acc, false);
}

// Butterfly sum over groups of W consecutive lanes (W a power of two <= 64).  The
// order is fixed, so results are reproducible; every lane of the group gets the sum.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = W / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        unsigned long long w = __shfl_xor(v, o, 64);
        v = w > v ? w : v;
    }
    return v;
}
