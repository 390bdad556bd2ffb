// Device helpers shared by the decode, combine and merge kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace mla {

// ---- number formats -------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(uint32_t(h) << 16);
}

// float32 -> bfloat16 with round-to-nearest-even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

// Two float32 -> packed bfloat16 (a in the low half), round-to-nearest-even,
// in one hardware conversion (v_cvt_pk_bf16_f32).  The output paths use it;
// the cache write keeps f32_to_bf16, whose result on every input is fixed
// by its definition above.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// OCP E4M3FN code -> float32 from the bit fields: bias 7, subnormals
// m * 2^-9, S.1111.111 = NaN, no infinities.
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t c) {
    const uint32_t sign = (c & 0x80u) << 24;
    const uint32_t e = (c >> 3) & 0xfu;
    const uint32_t m = c & 0x7u;
    float mag;
    if (e == 0) {
        mag = float(m) * 0.001953125f;  // m * 2^-9
    } else if (e == 0xfu && m == 0x7u) {
        return __uint_as_float(0x7fc00000u);
    } else {
        mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
    }
    return __uint_as_float(__float_as_uint(mag) | sign);
}

// ---- sharding ---------------------------------------------------------------

__device__ __forceinline__ int32_t dev_local_len(int32_t L, int32_t s, int32_t n) {
    return L > s ? (L - s + n - 1) / n : 0;
}

// floor(g / n) for 0 <= g < 2^31 and 1 <= n <= 4096, given inv = 1.0 / n in
// float64.  g * inv lies within 2^-21 of g / n, and a quotient that is not an
// integer is at least 1/n >= 2^-12 below the next integer, so truncating
// g * inv + 2^-20 gives the exact floor (a handful of instructions instead of
// an integer division by a runtime divisor).
__device__ __forceinline__ int32_t div_by(int32_t g, double inv) {
    return int32_t(fma(double(g), inv, 0x1p-20));
}

__device__ __forceinline__ void raise_error(uint32_t* err, uint32_t bit) {
    atomicOr(err, bit);
}

// ---- wave reductions ------------------------------------------------------

template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, W));
    return v;
}

template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, W);
    return v;
}

}  // namespace mla
