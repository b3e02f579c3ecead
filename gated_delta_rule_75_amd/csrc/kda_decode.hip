// KDA single-token decode step (HBM-bound).
//
// One new token per sequence and head ("The decode wall" and "KDA: trade the
// cache for a fixed-size state" in "Kimi K3, explained": the read touches the
// d_k x d_v state once per token, whatever the context length).  With the
// state S in R^{d_k x d_v} and alpha = exp(g):
//     S' = (I - beta k k^T) Diag(alpha) S + beta k v^T,   o = S'^T q.
// Because Diag(alpha) only scales rows, both reductions can use the OLD state:
//     u = S^T (alpha * k),  p = S^T (alpha * q),  delta = beta (v - u),
//     o = p + (k . q) delta,  S' = alpha * S + k delta^T,
// so every state element is read once and written once.
//
// Work decomposition: one workgroup per (sequence, head).  A thread owns 4
// consecutive value columns (one 16-byte vector) of RPT rows; a wave covers
// whole consecutive rows, so each load/store instruction moves contiguous
// memory.  The column reductions over key rows go through registers, then a
// small LDS table.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

template <int DK, int DV>
struct DecodeShape {
    static constexpr int kColThreads = DV / 4;                       // threads per row
    static constexpr int kThreads = (kColThreads * DK) < 256 ? kColThreads * DK : 256;
    static constexpr int kRowGroups = kThreads / kColThreads;
    static constexpr int kRowsPerThread = DK / kRowGroups;
    static_assert(DV % 4 == 0, "value width must be a multiple of 4");
    static_assert(DK % kRowGroups == 0, "rows must split evenly");
};

template <int DK, int DV, typename TI>
__global__ __launch_bounds__(256) void decode_kernel(
    const TI* __restrict__ q, const TI* __restrict__ k, const TI* __restrict__ v, const float* __restrict__ g,
    const TI* __restrict__ beta, const float* s_in, float* s_out, float* __restrict__ o) {
    using Sh = DecodeShape<DK, DV>;
    constexpr int CT = Sh::kColThreads, RG = Sh::kRowGroups, RPT = Sh::kRowsPerThread;
    const int64_t nh = blockIdx.x;  // sequence * H + head
    const int tid = threadIdx.x;
    const int c4 = tid % CT;  // owns columns 4*c4 .. 4*c4+3
    const int rg = tid / CT;  // owns rows rg, rg + RG, ...

    __shared__ float s_ak[DK], s_aq[DK], s_k[DK], s_a[DK];
    __shared__ float s_u[RG][DV], s_p[RG][DV];
    __shared__ float s_kq;

    const floatx4* Sin = reinterpret_cast<const floatx4*>(s_in + nh * (int64_t)DK * DV);
    floatx4* Sout = reinterpret_cast<floatx4*>(s_out + nh * (int64_t)DK * DV);

    // issue the state loads first: they are the bulk of the traffic
    floatx4 st[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) st[i] = __builtin_nontemporal_load(&Sin[(rg + i * RG) * CT + c4]);

    for (int i = tid; i < DK; i += Sh::kThreads) {
        const float a = expf(g[nh * DK + i]);
        const float kk = ld_in(k, nh * DK + i);
        const float qq = ld_in(q, nh * DK + i);
        s_a[i] = a;
        s_k[i] = kk;
        s_ak[i] = a * kk;
        s_aq[i] = a * qq;
    }
    if (tid < 64) {  // k . q, one wave
        float acc = 0.f;
        for (int i = tid; i < DK; i += 64) acc += ld_in(k, nh * DK + i) * ld_in(q, nh * DK + i);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
        if (tid == 0) s_kq = acc;
    }
    __syncthreads();

    float u[4] = {0.f, 0.f, 0.f, 0.f}, p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + i * RG;
        const float ak = s_ak[r], aq = s_aq[r];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u[j] += ak * st[i][j];
            p[j] += aq * st[i][j];
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        s_u[rg][4 * c4 + j] = u[j];
        s_p[rg][4 * c4 + j] = p[j];
    }
    __syncthreads();

    float d[4];
    const float b = ld_in(beta, nh);
    const float kq = s_kq;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = 4 * c4 + j;
        float uu = 0.f, pp = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            uu += s_u[r][col];
            pp += s_p[r][col];
        }
        d[j] = b * (ld_in(v, nh * DV + col) - uu);
        if (rg == 0) o[nh * DV + col] = pp + kq * d[j];
    }

#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + i * RG;
        const float a = s_a[r], kk = s_k[r];
        floatx4 ns;
#pragma unroll
        for (int j = 0; j < 4; ++j) ns[j] = a * st[i][j] + kk * d[j];
        __builtin_nontemporal_store(ns, &Sout[r * CT + c4]);
    }
}

template <int DK, int DV>
hipError_t launch_shape(const DecodeArgs& a, hipStream_t s) {
    using Sh = DecodeShape<DK, DV>;
    const dim3 grid(static_cast<unsigned>(a.N * a.H));
    const bool timed = timing_on();
    if (timed) timed_begin(kKernelDecode, s);
    if (a.bf16) {
        hipLaunchKernelGGL((decode_kernel<DK, DV, uint16_t>), grid, dim3(Sh::kThreads), 0, s,
                           static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                           static_cast<const uint16_t*>(a.v), a.g, static_cast<const uint16_t*>(a.beta), a.s_in,
                           a.s_out, a.o);
    } else {
        hipLaunchKernelGGL((decode_kernel<DK, DV, float>), grid, dim3(Sh::kThreads), 0, s,
                           static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                           static_cast<const float*>(a.v), a.g, static_cast<const float*>(a.beta), a.s_in,
                           a.s_out, a.o);
    }
    hipError_t e = hipGetLastError();
    if (timed) timed_end(s);
    return e;
}

}  // namespace

bool decode_supported(int dk, int dv) {
    const bool okk = dk == 16 || dk == 32 || dk == 64 || dk == 128;
    const bool okv = dv == 16 || dv == 32 || dv == 64 || dv == 128;
    return okk && okv;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    if (a.N * a.H == 0) return hipSuccess;
#define KDA_DEC(DK_, DV_) \
    if (a.dk == DK_ && a.dv == DV_) return launch_shape<DK_, DV_>(a, s);
#define KDA_DEC_ROW(DK_) KDA_DEC(DK_, 16) KDA_DEC(DK_, 32) KDA_DEC(DK_, 64) KDA_DEC(DK_, 128)
    KDA_DEC_ROW(16)
    KDA_DEC_ROW(32)
    KDA_DEC_ROW(64)
    KDA_DEC_ROW(128)
#undef KDA_DEC_ROW
#undef KDA_DEC
    return hipErrorInvalidValue;
}

}  // namespace kda
