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

// Buffer descriptor for `bytes` bytes at `base`; loads past the end return 0.  Both are
// wave-uniform where it is used; reading them through readfirstlane tells the compiler so (a
// descriptor it cannot prove uniform is wrapped in a per-lane loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    void* up = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(up, 0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Element i of a descriptor over storage type TI, as float (0 past the descriptor's end).
template <typename TI>
__device__ __forceinline__ float ld_buf(__amdgpu_buffer_rsrc_t r, int i);

template <>
__device__ __forceinline__ float ld_buf<float>(__amdgpu_buffer_rsrc_t r, int i) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, 0));
}

template <>
__device__ __forceinline__ float ld_buf<uint16_t>(__amdgpu_buffer_rsrc_t r, int i) {
    return bf16_to_f32((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, i * 2, 0, 0));
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
