// KDA chunked prefill, fp32 arithmetic throughout (any supported shape; q/k/v/beta stored as
// fp32 or bfloat16): the reference-precision path.  The chunk equations and their derivation
// are in kda_chunk_f32.h.
//
// One workgroup per (sequence, head, block of 16 value columns); value columns never interact,
// so blocks of them are independent chains.
#include "kda_chunk_f32.h"

namespace kda {
namespace {

constexpr int kThreads = 256;

template <int DK, int DV, int C, typename TI>
__global__ __launch_bounds__(kThreads) void chunk_f32_kernel(PrefillArgs a) {
    extern __shared__ float lds[];
    constexpr int NVB = DV / kF32BV;
    const int vb = blockIdx.x % NVB;
    const int h = (blockIdx.x / NVB) % a.H;
    const int64_t n = blockIdx.x / NVB / a.H;
    f32_chain<DK, DV, C, kThreads, TI>(a, n, h, vb, lds);
}

template <int DK, int DV, int C>
hipError_t launch_shape(const PrefillArgs& a, hipStream_t s) {
    constexpr size_t bytes = F32Lds<DK, C>::kBytes;
    const dim3 grid(static_cast<unsigned>(a.N * a.H * (DV / kF32BV)));
    const bool timed = timing_on();
    if (timed) timed_begin(kKernelChunkF32, s);
    if (a.bf16) {
        auto fn = chunk_f32_kernel<DK, DV, C, uint16_t>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(fn, grid, dim3(kThreads), bytes, s, a);
    } else {
        auto fn = chunk_f32_kernel<DK, DV, C, float>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(fn, grid, dim3(kThreads), bytes, s, a);
    }
    hipError_t e = hipGetLastError();
    if (timed) timed_end(s);
    return e;
}

constexpr size_t kLdsLimit = 160 * 1024;

template <int DK, int C>
constexpr bool fits() {
    return F32Lds<DK, C>::kBytes <= kLdsLimit;
}

}  // namespace

bool chunk_f32_supported(int dk, int dv, int chunk) {
    const bool okd = (dk == 16 || dk == 32 || dk == 64 || dk == 128) && (dv == 16 || dv == 32 || dv == 64 || dv == 128);
    if (!okd) return false;
    if (chunk == 16) return true;
    if (chunk == 32) return true;
    if (chunk == 64) return dk <= 64;
    return false;
}

hipError_t launch_chunk_f32(const PrefillArgs& a, hipStream_t s) {
    if (a.N * a.H == 0) return hipSuccess;
#define KDA_F32(DK_, DV_, C_) \
    if (a.dk == DK_ && a.dv == DV_ && a.chunk == C_) return launch_shape<DK_, DV_, C_>(a, s);
#define KDA_F32_DV(DK_, C_) KDA_F32(DK_, 16, C_) KDA_F32(DK_, 32, C_) KDA_F32(DK_, 64, C_) KDA_F32(DK_, 128, C_)
    KDA_F32_DV(16, 16) KDA_F32_DV(32, 16) KDA_F32_DV(64, 16) KDA_F32_DV(128, 16)
    KDA_F32_DV(16, 32) KDA_F32_DV(32, 32) KDA_F32_DV(64, 32) KDA_F32_DV(128, 32)
    KDA_F32_DV(16, 64) KDA_F32_DV(32, 64) KDA_F32_DV(64, 64)
#undef KDA_F32_DV
#undef KDA_F32
    static_assert(fits<128, 32>() && fits<64, 64>(), "LDS budget");
    return hipErrorInvalidValue;
}

}  // namespace kda
