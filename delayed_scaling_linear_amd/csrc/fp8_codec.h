// OCP FP8 encode shared by the kernels that write FP8 codes (the cast and
// the FP8-output epilogue of the matrix product).
//
// "Accelerating PyTorch Training Workloads with FP8 -- Part 2" (section on
// PyTorch-native FP8 data types) gives the two formats, float8_e4m3fn (max
// 448, no infinities) and float8_e5m2 (max 57344).  A value is multiplied by
// its tensor's scale in fp32, clamped to +-max (saturation: v_med3_f32) and
// converted by the hardware OCP converter (v_cvt_pk_fp8_f32 /
// v_cvt_pk_bf8_f32, round to nearest even).  A NaN product becomes
// 0x7F | (sign(x) ^ sign(scale)); the clamp alone would not keep it NaN.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8dsl.h"

namespace fp8dsl {

template <int FMT>
struct Fp8Traits;
template <>
struct Fp8Traits<FP8_E4M3> {
    static constexpr float kMax = 448.0f;
    template <bool HI>
    __device__ static __forceinline__ int cvt(float a, float b, int old) {
        return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
    }
};
template <>
struct Fp8Traits<FP8_E5M2> {
    static constexpr float kMax = 57344.0f;
    template <bool HI>
    __device__ static __forceinline__ int cvt(float a, float b, int old) {
        return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
    }
};

// Four scaled, clamped values -> one word of four codes (byte i = value i).
template <int FMT>
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d, float s) {
    using T = Fp8Traits<FMT>;
    a = __builtin_amdgcn_fmed3f(a * s, -T::kMax, T::kMax);
    b = __builtin_amdgcn_fmed3f(b * s, -T::kMax, T::kMax);
    c = __builtin_amdgcn_fmed3f(c * s, -T::kMax, T::kMax);
    d = __builtin_amdgcn_fmed3f(d * s, -T::kMax, T::kMax);
    // The first convert fills the low half and keeps the high half of its
    // third operand, which the second convert then overwrites: any register
    // serves, and a's (dead after) saves a move of zero.
    int w = T::template cvt<false>(a, b, (int)__float_as_uint(a));
    w = T::template cvt<true>(c, d, w);
    return (uint32_t)w;
}

// Rare path: a NaN product gets 0x7F | (sign(x) ^ sign(s)).  Callers run it
// only where a NaN source was seen (or everywhere, when the scale is 0, inf
// or NaN).
__device__ __forceinline__ uint32_t patch_nan4(uint32_t w, const float x[4], float s) {
    const uint32_t sbits = __float_as_uint(s);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float v = x[i] * s;
        if (v != v) {
            const uint32_t code = 0x7Fu | (((__float_as_uint(x[i]) ^ sbits) >> 24) & 0x80u);
            w = (w & ~(0xFFu << (8 * i))) | (code << (8 * i));
        }
    }
    return w;
}

}  // namespace fp8dsl
