// Device-side helpers shared by the KDA kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// bfloat16 bits -> float (exact widening)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

template <typename TI>
__device__ __forceinline__ float ld_in(const TI* p, int64_t i);

template <>
__device__ __forceinline__ float ld_in<float>(const float* p, int64_t i) {
    return p[i];
}

template <>
__device__ __forceinline__ float ld_in<uint16_t>(const uint16_t* p, int64_t i) {
    return bf16_to_f32(p[i]);
}

// exp(x) through the hardware base-2 exponential (v_exp_f32).
__device__ __forceinline__ float fast_exp(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// Fused input prologue: beta from its logit, g from the raw gate input.  Both use the hardware
// base-2 exponential and logarithm (about 1e-7 relative error), which keeps them small enough
// for the register budget of the kernels they are inlined into.
__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + fast_exp(-x)); }

__device__ __forceinline__ float gate_from_raw(float a, float scale) {
    // -scale * softplus(a), softplus(a) = log(1 + e^a) written so that it cannot overflow:
    // max(a, 0) + log(1 + e^-|a|)
    const float t = 1.f + fast_exp(-fabsf(a));
    return -scale * (fmaxf(a, 0.f) + __builtin_amdgcn_logf(t) * 0.6931471805599453f);
}

}  // namespace kda
