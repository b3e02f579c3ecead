// KDA chunked backward: gradients of the chunked prefill with respect to q, k, v, g = log(alpha),
// beta and the initial state, given dL/do and dL/dS_T.  fp32 accumulation throughout.
//
// "Kimi K3, explained" says that training runs the recurrence in chunks ("How is KDA trained
// efficiently if it is a recurrence?", "Training in chunks") and gives no gradient equations.  The
// ones used here are the derivative of the chunk equations of the forward pass (the same as the
// fp32 forward kernel's).  For a chunk of L tokens (rows r, s; G the in-chunk cumulative
// log-decay, E(r,s,c) = exp(G_rc - G_sc) for s <= r, S0 the state entering the chunk):
//   P[r,s] = sum_c k_rc k_sc E(r,s,c)  (s < r)        A = Diag(beta) P,   T = (I + A)^{-1}
//   M[r,s] = sum_c q_rc k_sc E(r,s,c)  (s <= r)
//   K+ = K exp(G),  Q+ = Q exp(G),  K' = K exp(G_last - G),  gamma = exp(G_last)
//   W = T Diag(beta) K+,  U = T Diag(beta) V,  D = U - W S0
//   O = Q+ S0 + M D,      S1 = Diag(gamma) S0 + K'^T D
// Backwards, with dS1 the gradient reaching the chunk's final state and dO its outputs' gradient:
//   dD = K' dS1 + M^T dO          dS0 = Diag(gamma) dS1 + Q+^T dO - W^T dD     (chain over chunks)
//   dK' = D dS1^T   dQ+ = dO S0^T   dW = -dD S0^T   dgamma = rowsum(dS1 * S0)   dM = tril(dO D^T)
//   dT = dD (beta V)^T + dW (beta K+)^T,  dA = -T^T dT T^T (strictly lower part)
//   dV = beta (T^T dD),  dK+ = beta (T^T dW),  dbeta = rowsum(V T^T dD + K+ T^T dW + dA P)
//   dP = Diag(beta) dA, and dP, dM back through the pairwise products into dK, dQ and dG
//   dG collects every exp(G) factor; dg is its suffix sum over the chunk's rows.
//
// Five launches:
//   factors     (chunk, head)          P, M, T, W, U, Q+, K', gamma into the workspace
//   fwd_chain   (sequence, head, vb)   states entering each chunk and D, chunk by chunk
//   rev_chain   (sequence, head, vb)   dS leaving each chunk and dD, chunks in reverse; dS0
//   grad_state  (chunk, head)          dK', dQ+, dW, dM, dgamma (products over the value axis)
//   grad_chunk  (chunk, head)          dq, dk, dv, dg, dbeta
// The two chains are sequential over chunks and split by 16 value columns (columns of S and dS
// never interact); the three per-chunk kernels are fully parallel.  Every product is a 16x16
// tile on the matrix cores: fp32 steps (v_mfma_f32_16x16x4f32), or, for bfloat16 storage at
// d = 128, chunk 64, split-bf16 steps in the two chains and grad_state (see SplitShape).  The
// pairwise products P, M and their gradients are included: the decay exp(G_r - G_s) of a pair is
// split at a 16-row block boundary m,
// exp(G_r - G_m) exp(G_m - G_s), and the two factors scale the two operands.  Across blocks both
// exponents are <= 0.  Inside a block one factor can exceed 1; where a block's 16-token decay
// exceeds e^64 those pairs take their own exponentials on the vector ALUs instead.
#include <cstdlib>
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves
constexpr int kBV = 16;        // value columns per chain workgroup
constexpr int kWarm = 3;       // chunks between a chain's L2 warm-up of a record and its use

// acc += A (16 x 4KS) * B (4KS x 16) with A(r, k) = A[r * ar + k * ak] and B(k, c) = B[k * bk + c * bc].
// Result layout: acc[e] is row 4 * (lane >> 4) + e, column lane & 15.
template <int KS>
__device__ __forceinline__ floatx4 mma(const float* A, int ar, int ak, const float* B, int bk, int bc, floatx4 acc,
                                       int lane) {
    const int r = lane & 15, kq = lane >> 4;
    const float* pa = A + r * ar + kq * ak;
    const float* pb = B + kq * bk + r * bc;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[4 * ks * ak], pb[4 * ks * bk], acc, 0, 0, 0);
    return acc;
}

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// f(e) for e = tid, tid + S kThreads, tid + 2 S kThreads, ... below N (S = 1, or 2 for element pairs
// at even e = S tid + ...), unrolled over a static trip count so that the compiler can issue the
// loop's memory operations together instead of one iteration at a time.
template <int N, int S = 1, typename F>
__device__ __forceinline__ void for_each_elem(int tid, F&& f) {
    constexpr int IT = (N + S * kThreads - 1) / (S * kThreads);
#pragma unroll
    for (int m = 0; m < IT; ++m) {
        const int e = S * tid + S * kThreads * m;
        if (IT * S * kThreads == N || e < N) f(e);
    }
}

// f(i) for i = w, w + 4, w + 8, ... below N (w = this wave, one of 4), unrolled over a static trip
// count like for_each_elem.
template <int N, typename F>
__device__ __forceinline__ void for_each_wave(int w, F&& f) {
    constexpr int IT = (N + 3) / 4;
#pragma unroll
    for (int m = 0; m < IT; ++m) {
        const int i = w + 4 * m;
        if (4 * IT == N || i < N) f(i);
    }
}

// acc += A (16 x 16 KS) * B (16 KS x 16) with both operands contiguous along k in LDS:
// A(r, k) = A[r * ar + k] and B(k, c) = Bt[c * bc + k], ar and bc multiples of 4.  Lane (r, kq) feeds
// k = 16 s + 4 kq + i at the i-th of the four steps of group s (any assignment of k to steps gives the
// same sum), so each group takes one 16-byte LDS read per operand; even and odd groups go to two
// accumulators.
template <int KS>
__device__ __forceinline__ floatx4 mma_k4(const float* A, int ar, const float* Bt, int bc, floatx4 acc, int lane) {
    const int r = lane & 15, kq = lane >> 4;
    const float* pa = A + r * ar + 4 * kq;
    const float* pb = Bt + r * bc + 4 * kq;
    floatx4 acc1 = zero4();
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const float4 a4 = *reinterpret_cast<const float4*>(pa + 16 * s);
        const float4 b4 = *reinterpret_cast<const float4*>(pb + 16 * s);
        floatx4& x = (s & 1) ? acc1 : acc;
        x = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.x, b4.x, x, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.y, b4.y, x, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.z, b4.z, x, 0, 0, 0);
        x = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.w, b4.w, x, 0, 0, 0);
    }
    return acc + acc1;
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations (lgkmcnt) but not for
// its outstanding global loads and stores, so loads issued one step ahead stay in flight across it
// (a __syncthreads() fence would drain them).  No kernel here reads global memory that another
// workgroup thread wrote in the same launch.  The empty asm statements keep the compiler from
// moving memory operations across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // gfx9 encoding: vmcnt/expcnt at max, lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// sum over the 16 lanes that share (lane >> 4)
__device__ __forceinline__ float sum16(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    return x;
}

// Split-bf16 operands (bfloat16 storage at d_k = d_v = 128, chunk 64): an fp32 value x is kept as
// hi = bf16(x) and lo = bf16(x - hi), so x = hi + lo to within 2^-18 of |x|, and a product takes
// three bf16 matrix-core steps (hi hi + hi lo + lo hi; lo lo is below 2^-18 of the product), with
// fp32 accumulation and fp32's exponent range.  A 32-deep contraction is then one 16x16x32 step
// where the fp32 16x16x4 form needs eight steps of twice the cost.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void split4(float4 x, bf16x4& hi, bf16x4& lo) {
    const float v[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hi[i] = (__bf16)v[i];
        lo[i] = (__bf16)(v[i] - (float)hi[i]);
    }
}

__device__ __forceinline__ floatx4 mfma_split(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, floatx4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
}

template <int DK, int DV, int C, typename TI>
struct SplitShape {
    static constexpr bool value = std::is_same<TI, uint16_t>::value && DK == 128 && DV == 128 && C == 64;
};

// Elements i and i + 1 (i even) of an n-element chain operand array at rec + off, split: bf16 hi in
// the array's first half and bf16 lo in its second half (the bytes of n floats), one 4-byte store
// for each.
__device__ __forceinline__ void put_pair(float* rec, int64_t off, int n, int i, float x0, float x1) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 hi, lo;
    hi[0] = (__bf16)x0;
    hi[1] = (__bf16)x1;
    lo[0] = (__bf16)(x0 - (float)hi[0]);
    lo[1] = (__bf16)(x1 - (float)hi[1]);
    bf16x2* p = reinterpret_cast<bf16x2*>(rec + off);
    p[i >> 1] = hi;
    p[(n + i) >> 1] = lo;
}

// A 16x32 bf16 operand fragment from LDS holding bf16 pairs packed in floats (row stride ldf
// floats): rows row0 + (lane & 15), k = 32 ks + 8 (lane >> 4) .. +7.
__device__ __forceinline__ bf16x8 frag16(const float* base, int row0, int ldf, int ks, int lane) {
    return *reinterpret_cast<const bf16x8*>(base + (row0 + (lane & 15)) * ldf + 16 * ks + 4 * (lane >> 4));
}

// Workspace record of one (chunk slot, head), in floats.
template <int DK, int DV, int C>
struct Rec {
    // the forward chain's operands (W, U, K'^T), then the reverse chain's (K', Q+^T, W^T, M^T): each
    // stored with the contraction index contiguous, as the chains consume it
    static constexpr int64_t W = 0;                       // [C][DK]  T Diag(beta) K+
    static constexpr int64_t U = W + C * DK;              // [C][DV]  T Diag(beta) V
    static constexpr int64_t KdT = U + C * DV;            // [DK][C]  K'^T
    static constexpr int64_t Kd = KdT + DK * C;           // [C][DK]  K'
    static constexpr int64_t QpT = Kd + C * DK;           // [DK][C]  Q+^T
    static constexpr int64_t WT = QpT + DK * C;           // [DK][C]  W^T
    static constexpr int64_t MT = WT + DK * C;            // [C][C]   M^T
    static constexpr int64_t T = MT + C * C;              // [C][C]
    static constexpr int64_t P = T + C * C;               // [C][C]   strictly lower
    static constexpr int64_t gam = P + C * C;             // [DK]
    static constexpr int64_t S0 = gam + DK;               // [DK][DV] state entering the chunk
    static constexpr int64_t dS1 = S0 + DK * DV;          // [DK][DV] gradient of the state leaving it
    static constexpr int64_t D = dS1 + DK * DV;           // [C][DV]
    static constexpr int64_t dD = D + C * DV;             // [C][DV]
    static constexpr int64_t dKd = dD + C * DV;           // [C][DK]
    static constexpr int64_t dQp = dKd + C * DK;          // [C][DK]
    static constexpr int64_t dW = dQp + C * DK;           // [C][DK]
    static constexpr int64_t dM = dW + C * DK;            // [C][C]
    static constexpr int64_t dgam = dM + C * C;           // [DK]
    static constexpr int64_t kFloats = (dgam + DK + 63) / 64 * 64;  // records stay 256-byte aligned
};

// Sequences (device cu_seqlens) and chunk slots.  One pass over every chunk (wlen = 0): sequence n
// owns slots base(n) .. base(n) + chunks - 1.  A window (wlen > 0): only chunks wlo .. wlo + wlen - 1
// of every sequence, sequence n owning slots n * wlen .. n * wlen + wlen - 1 (slot = base(n) + c).
template <int C>
struct Map {
    const int32_t* cu;
    int64_t N;
    int64_t wlo, wlen;
    __device__ __forceinline__ int64_t base(int64_t n) const { return wlen ? n * wlen - wlo : (int64_t)cu[n] / C + n; }
    // this launch's chunks [c0, c1) of sequence n
    __device__ __forceinline__ void range(int64_t n, int64_t& c0, int64_t& c1) const {
        const int64_t nck = ((int64_t)cu[n + 1] - cu[n] + C - 1) / C;
        c0 = wlen ? (wlo < nck ? wlo : nck) : 0;
        c1 = wlen ? (wlo + wlen < nck ? wlo + wlen : nck) : nck;
    }
    __device__ __forceinline__ bool locate(int64_t slot, int64_t& n, int64_t& c, int64_t& t0, int& L) const {
        if (wlen) {
            n = slot / wlen;
            c = wlo + slot % wlen;
            if (n >= N) return false;
        } else {
            if (N <= 0 || base(0) > slot) return false;
            int64_t lo = 0, hi = N - 1;
            while (lo < hi) {
                const int64_t mid = (lo + hi + 1) >> 1;
                if (base(mid) <= slot) lo = mid; else hi = mid - 1;
            }
            n = lo;
            c = slot - base(n);
        }
        const int64_t bos = cu[n], eos = cu[n + 1];
        t0 = bos + c * C;
        if (t0 >= eos) return false;
        L = (int)(eos - t0 < C ? eos - t0 : C);
        return true;
    }
};

// Unconditional loads: where a row may lie past the chunk end, the row index is clamped to the last
// valid row and the value replaced by zero after the load.  A branch around the load would make
// the wave wait for the load before the branches merge, which serialises every prefetch.
__device__ __forceinline__ float gate_at(const float* g, int gate_head, int64_t t, int H, int h, int DK, int c) {
    return gate_head ? g[t * H + h] : g[(t * H + h) * (int64_t)DK + c];
}

// Inclusive prefix sum over the 64 lanes of a wave, in lane order: within each row of 16 lanes by
// DPP right shifts of 1, 2, 4 and 8 (lanes shifted in from outside the row add 0), then rows 1 and
// 3 add the last lane of the row before them (DPP row_bcast:15) and rows 2 and 3 add lane 31 (DPP
// row_bcast:31); rows left out by the row mask add 0.
__device__ __forceinline__ float wave_prefix64(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xA, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xC, 0xF, false));
    return x;
}

// ------------------------------------------------------------------------------------------
// factors: one workgroup per (chunk slot, head), under 80 KB of LDS (two per CU).  Key channels
// are visited in tiles of 32, each tile's cumulative log-decay recomputed there by a prefix sum over
// the rows (one lane per row, wave_prefix64).
//   pass 1: P and M.  Pairs (r, s) in different 16-row blocks i > j use the matrix cores with the
//           decay split at m, the last row of block j: exp(G_r - G_s) = exp(G_r - G_m) exp(G_m - G_s),
//           both exponents <= 0, applied to the operands as they are loaded.  Pairs inside a block
//           take the exponential of their own difference on the vector ALUs.
//   then T = (I + Diag(beta) P)^{-1};
//   pass 2: Q+, K', gamma and W = T (beta K+) per channel tile;  pass 3: U = T (beta V) per value tile.
// ------------------------------------------------------------------------------------------
template <int DK, int DV, int C>
struct FactorsLds {
    static constexpr int LC = C + 1, CT = 32, LT = CT + 1;
    static constexpr size_t kFloats = 3 * (size_t)C * LC + 3 * (size_t)C * LT + C + 4;
    static constexpr size_t kBytes = kFloats * sizeof(float);
};

template <int DK, int DV, int C, typename TI>
__global__ __launch_bounds__(kThreads, 2) void factors_kernel(BwdArgs a, Map<C> mp) {
    using R = Rec<DK, DV, C>;
    constexpr bool SPLIT = SplitShape<DK, DV, C, TI>::value;  // chain operands stored as bf16 hi and lo
    using Lds = FactorsLds<DK, DV, C>;
    constexpr int LC = Lds::LC, LT = Lds::LT, NR = C / 16;
    constexpr int CT = DK < Lds::CT ? DK : Lds::CT;  // channels per tile
    constexpr int VT = DV < Lds::CT ? DV : Lds::CT;  // value columns per tile
    extern __shared__ float lds[];
    float* sP = lds;            // [C][LC]
    float* sM = sP + C * LC;    // [C][LC]  M, then A = Diag(beta) P
    float* sT = sM + C * LC;    // [C][LC]
    float* tK = sT + C * LC;    // [C][LT]  k, then beta K+
    float* tQ = tK + C * LT;    // [C][LT]  q, then beta V
    float* tG = tQ + C * LT;    // [C][LT]  g, then G
    float* sB = tG + C * LT;    // [C]
    int* sFlag = reinterpret_cast<int*>(sB + C);  // a block of the current tile decays by more than e^64

    const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
    const int64_t slot = blockIdx.x;
    int64_t n, c, t0;
    int L;
    if (!mp.locate(slot, n, c, t0, L)) return;  // uniform over the workgroup
    const int H = a.H;
    const TI* q = static_cast<const TI*>(a.q);
    const TI* k = static_cast<const TI*>(a.k);
    const TI* v = static_cast<const TI*>(a.v);
    const TI* beta = static_cast<const TI*>(a.beta);
    float* rec = a.ws + (slot * H + h) * R::kFloats;
    if (tid < C) sB[tid] = tid < L ? ld_in<TI>(beta, (t0 + tid) * H + h) : 0.f;
    // descriptors over this chunk's rows of k, q, g and v: rows past the chunk end read 0, so the
    // tile loads need no clamping or selects (and no branch, which would serialise them)
    const int64_t tok0 = t0 * H + h;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + tok0 * DK, (uint32_t)((((int64_t)L - 1) * H * DK + DK) * sizeof(TI)));
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(q + tok0 * DK, (uint32_t)((((int64_t)L - 1) * H * DK + DK) * sizeof(TI)));
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + tok0 * DV, (uint32_t)((((int64_t)L - 1) * H * DV + DV) * sizeof(TI)));
    const __amdgpu_buffer_rsrc_t grs =
        a.gate_head ? make_rsrc(a.g + tok0, (uint32_t)((((int64_t)L - 1) * H + 1) * 4))
                    : make_rsrc(a.g + tok0 * DK, (uint32_t)((((int64_t)L - 1) * H * DK + DK) * 4));

    // Channel tiles c0 .. c0 + CT - 1 of k, q and g (rows >= L are zero) and value tiles of v go
    // through registers one tile ahead of their use: the tile sequence is the channel tiles of
    // pass 1, the same tiles again for pass 2, then the value tiles of pass 3.  Element m of a
    // thread is row (tid + kThreads m) / CT, column (tid + kThreads m) % CT.
    constexpr int EPT = (C * CT + kThreads - 1) / kThreads, NCTILE = DK / CT;
    struct TileRegs {
        float k[EPT], q[EPT], g[EPT];
    } tr;
    constexpr int VPT = (C * VT + kThreads - 1) / kThreads;
    float vr[VPT];
    auto fetch_tile = [&](int c0) {
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int e = tid + kThreads * m, r = e / CT, cc = e % CT;
            const int o = r * H * DK + c0 + cc;  // past the descriptors' ends (r >= L) the loads read 0
            tr.k[m] = ld_buf<TI>(krs, o);
            tr.q[m] = ld_buf<TI>(qrs, o);
            tr.g[m] = ld_buf<float>(grs, a.gate_head ? r * H : o);
        }
    };
    auto fetch_value = [&](int j0) {
#pragma unroll
        for (int m = 0; m < VPT; ++m) {
            const int e = tid + kThreads * m, r = e / VT, j = e % VT;
            vr[m] = ld_buf<TI>(vrs, r * H * DV + j0 + j);
        }
    };
    // registers -> tK, tQ, tG (raw g), then G = tril(ones) g into tG
    auto put_tile = [&]() {
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int e = tid + kThreads * m, r = e / CT, cc = e % CT;
            if (EPT * kThreads == C * CT || e < C * CT) {
                tK[r * LT + cc] = tr.k[m];
                tQ[r * LT + cc] = tr.q[m];
                tG[r * LT + cc] = tr.g[m];
            }
        }
        lds_barrier();
        // G = tril(ones) g, a prefix sum over the rows: wave w scans columns w, w + 4, ... with one
        // lane per row (each wave reads and writes only its own columns)
        static_assert(C <= 64, "one lane per chunk row");
        for_each_wave<CT>(w, [&](int j) {
            const float x = wave_prefix64(lane < C ? tG[lane * LT + j] : 0.f);
            if (lane < C) tG[lane * LT + j] = x;
        });
        lds_barrier();
    };
    fetch_tile(0);

    // ---- pass 1: P and M
    constexpr int NPAIR = NR * (NR - 1) / 2, PPW = (NPAIR + 3) / 4;  // off-diagonal block pairs
    floatx4 accP[PPW > 0 ? PPW : 1], accM[PPW > 0 ? PPW : 1];
    int pi[PPW > 0 ? PPW : 1], pj[PPW > 0 ? PPW : 1];
#pragma unroll
    for (int m = 0; m < PPW; ++m) {
        accP[m] = accM[m] = zero4();
        int t = w + 4 * m, i = 1;
        while (t >= i) { t -= i; ++i; }  // pair index -> (i, j), j < i
        pi[m] = i;
        pj[m] = t;
    }
    constexpr int NDIAG = NR * 136, DPT = (NDIAG + kThreads - 1) / kThreads;  // pairs s <= r inside a block
    float dp[DPT], dm[DPT];
    int dr[DPT], ds[DPT];
#pragma unroll
    for (int m = 0; m < DPT; ++m) {
        dp[m] = dm[m] = 0.f;
        int t = tid + kThreads * m;
        const int blk = t / 136;
        t %= 136;
        int rr = 0;
        while (t > rr) { t -= rr + 1; ++rr; }
        dr[m] = 16 * blk + rr;
        ds[m] = 16 * blk + t;
    }
    // pairs inside block w, on the matrix cores as the pairs across blocks but split at the block's
    // own last row: the row factor exp(G_r - G_m) is then >= 1, bounded by exp(D) with D the block's
    // 16-token decay.  A tile where D > 64 for some block and channel takes the exact per-pair
    // exponentials instead (vector ALUs, pairs spread over the workgroup).
    floatx4 accPd = zero4(), accMd = zero4();
    bool any_exact = false;
    if (tid == 0) *sFlag = 0;
#pragma unroll
    for (int ti = 0; ti < NCTILE; ++ti) {
        put_tile();
        fetch_tile(ti + 1 < NCTILE ? (ti + 1) * CT : 0);  // the last one is pass 2's first tile
        if (tid < NR * CT) {
            const int b = tid / CT, cc = tid % CT;
            const float D = (b > 0 ? tG[(16 * b - 1) * LT + cc] : 0.f) - tG[(16 * b + 15) * LT + cc];
            if (D > 64.f) *sFlag = 1;  // benign race: every writer stores 1
        }
        lds_barrier();
        const bool exact = *sFlag != 0;
        any_exact |= exact;
        if (!exact && w < NR) {
            const int ra = 16 * w + lr, mj = 16 * w + 15;
#pragma unroll 4
            for (int ks = 0; ks < CT / 4; ++ks) {
                const int cc = 4 * ks + lg;
                const float gm = tG[mj * LT + cc];
                const float ea = fast_exp(tG[ra * LT + cc] - gm);
                const float bb = tK[ra * LT + cc] * fast_exp(gm - tG[ra * LT + cc]);
                accPd = __builtin_amdgcn_mfma_f32_16x16x4f32(tK[ra * LT + cc] * ea, bb, accPd, 0, 0, 0);
                accMd = __builtin_amdgcn_mfma_f32_16x16x4f32(tQ[ra * LT + cc] * ea, bb, accMd, 0, 0, 0);
            }
        }
#pragma unroll
        for (int m = 0; m < PPW; ++m) {
            if (w + 4 * m < NPAIR) {
                const int ra = 16 * pi[m] + lr, sb = 16 * pj[m] + lr, mj = 16 * pj[m] + 15;
#pragma unroll 4
                for (int ks = 0; ks < CT / 4; ++ks) {
                    const int cc = 4 * ks + lg;
                    const float gm = tG[mj * LT + cc];
                    const float ea = fast_exp(tG[ra * LT + cc] - gm);
                    const float bb = tK[sb * LT + cc] * fast_exp(gm - tG[sb * LT + cc]);
                    accP[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(tK[ra * LT + cc] * ea, bb, accP[m], 0, 0, 0);
                    accM[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(tQ[ra * LT + cc] * ea, bb, accM[m], 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int m = 0; m < DPT; ++m) {
            if (exact && tid + kThreads * m < NDIAG) {
                const float* kr = tK + dr[m] * LT;
                const float* qr = tQ + dr[m] * LT;
                const float* gr = tG + dr[m] * LT;
                const float* ks = tK + ds[m] * LT;
                const float* gs = tG + ds[m] * LT;
#pragma unroll 8
                for (int cc = 0; cc < CT; ++cc) {
                    const float e = fast_exp(gr[cc] - gs[cc]) * ks[cc];
                    dp[m] += kr[cc] * e;
                    dm[m] += qr[cc] * e;
                }
            }
        }
        lds_barrier();  // the tile is restaged next
        if (tid == 0) *sFlag = 0;
    }
    // P, M into LDS: zero above the blocks' diagonal, then the two kinds of pairs
    for_each_elem<C * C>(tid, [&](int e) {
        const int r = e / C, s2 = e % C;
        if (s2 / 16 > r / 16) {
            sP[r * LC + s2] = 0.f;
            sM[r * LC + s2] = 0.f;
        } else if (s2 / 16 == r / 16 && s2 > r) {
            sP[r * LC + s2] = 0.f;
            sM[r * LC + s2] = 0.f;
        }
    });
    if (w < NR)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * w + 4 * lg + e, s2 = 16 * w + lr;
            sP[r * LC + s2] = s2 < r ? accPd[e] : 0.f;
            sM[r * LC + s2] = s2 <= r ? accMd[e] : 0.f;
        }
    if (any_exact) {  // uniform: every thread read the same flags
        lds_barrier();
#pragma unroll
        for (int m = 0; m < DPT; ++m)
            if (tid + kThreads * m < NDIAG) {
                sP[dr[m] * LC + ds[m]] += ds[m] < dr[m] ? dp[m] : 0.f;
                sM[dr[m] * LC + ds[m]] += dm[m];
            }
    }
#pragma unroll
    for (int m = 0; m < PPW; ++m)
        if (w + 4 * m < NPAIR)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * pi[m] + 4 * lg + e, s2 = 16 * pj[m] + lr;
                sP[r * LC + s2] = accP[m][e];
                sM[r * LC + s2] = accM[m][e];
            }
    lds_barrier();
    if constexpr (SPLIT) {
        for_each_elem<C * C, 2>(tid, [&](int e) {  // element pairs along a row
            const int r = e / C, s2 = e % C;
            put_pair(rec, R::MT, C * C, e, sM[s2 * LC + r], sM[(s2 + 1) * LC + r]);  // M^T[r][s2] = M[s2][r]
            *reinterpret_cast<float2*>(rec + R::P + e) = make_float2(sP[r * LC + s2], sP[r * LC + s2 + 1]);
        });
    } else {
        for_each_elem<C * C>(tid, [&](int e) {
            const int r = e / C, s2 = e % C;
            rec[R::MT + e] = sM[s2 * LC + r];  // M^T[r][s2] = M[s2][r]
            rec[R::P + e] = sP[r * LC + s2];
        });
    }
    lds_barrier();
    // A = Diag(beta) P into M's buffer; T zeroed
    float* sA = sM;
    for_each_elem<C * C>(tid, [&](int e) {
        const int r = e / C, s2 = e % C;
        sA[r * LC + s2] = sB[r] * sP[r * LC + s2];
        sT[r * LC + s2] = 0.f;
    });
    lds_barrier();

    // T = (I + A)^{-1}, unit lower triangular.  Diagonal 16x16 blocks by forward substitution (lane =
    // column, the block's rows in registers); then the blocks below the diagonal, nearest first:
    // T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj.
    if (w < NR && lane < 16) {
        const int j = lane, o = 16 * w;
        float tc[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            float acc = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < rr; ++s2) acc += sA[(o + rr) * LC + o + s2] * tc[s2];
            tc[rr] = rr < j ? 0.f : (rr == j ? 1.f : -acc);
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) sT[(o + rr) * LC + o + j] = tc[rr];
    }
    lds_barrier();
    float* sXs = sP + w * 16 * 17;  // per-wave 16x16 scratch (P is in the record already)
    for (int dist = 1; dist < NR; ++dist) {
        const int j = w, i = w + dist;
        if (i < NR) {
            floatx4 acc = zero4();
            for (int m = j; m < i; ++m)
                acc = mma<4>(sA + 16 * i * LC + 16 * m, LC, 1, sT + 16 * m * LC + 16 * j, LC, 1, acc, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) sXs[(4 * lg + e) * 17 + lr] = acc[e];
        }
        lds_barrier();
        if (i < NR) {
            const floatx4 t = mma<4>(sT + 16 * i * LC + 16 * i, LC, 1, sXs, 17, 1, zero4(), lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) sT[(16 * i + 4 * lg + e) * LC + 16 * j + lr] = -t[e];
        }
        lds_barrier();
    }
    for_each_elem<C * C>(tid, [&](int e) { rec[R::T + e] = sT[(e / C) * LC + e % C]; });

    // ---- pass 2: Q+^T, K', K'^T, gamma and W = T (beta K+), channel tile by channel tile
#pragma unroll
    for (int ti = 0; ti < NCTILE; ++ti) {
        const int c0 = ti * CT;
        put_tile();
        if (ti + 1 < NCTILE)
            fetch_tile((ti + 1) * CT);
        else
            fetch_value(0);
        if constexpr (SPLIT) {
            for_each_elem<C * CT, 2>(tid, [&](int e) {  // channel-major, token pairs
                const int cc = e / C, r = e % C;
                const float g0 = tG[r * LT + cc], g1 = tG[(r + 1) * LT + cc], gl = tG[(C - 1) * LT + cc];
                put_pair(rec, R::QpT, DK * C, (c0 + cc) * C + r, tQ[r * LT + cc] * fast_exp(g0),
                         tQ[(r + 1) * LT + cc] * fast_exp(g1));
                put_pair(rec, R::KdT, DK * C, (c0 + cc) * C + r, tK[r * LT + cc] * fast_exp(gl - g0),
                         tK[(r + 1) * LT + cc] * fast_exp(gl - g1));
            });
        } else {
            for_each_elem<C * CT>(tid, [&](int e) {  // channel-major outputs (token index fastest)
                const int cc = e / C, r = e % C;
                const float g = tG[r * LT + cc], gl = tG[(C - 1) * LT + cc];
                rec[R::QpT + (c0 + cc) * C + r] = tQ[r * LT + cc] * fast_exp(g);
                rec[R::KdT + (c0 + cc) * C + r] = tK[r * LT + cc] * fast_exp(gl - g);
            });
        }
        lds_barrier();
        if constexpr (SPLIT) {
            for_each_elem<C * CT, 2>(tid, [&](int e) {  // token-major, channel pairs
                const int r = e / CT, cc = e % CT;
                const float g0 = tG[r * LT + cc], g1 = tG[r * LT + cc + 1];
                const float gl0 = tG[(C - 1) * LT + cc], gl1 = tG[(C - 1) * LT + cc + 1];
                const float k0 = tK[r * LT + cc], k1 = tK[r * LT + cc + 1];
                put_pair(rec, R::Kd, C * DK, r * DK + c0 + cc, k0 * fast_exp(gl0 - g0), k1 * fast_exp(gl1 - g1));
                tK[r * LT + cc] = sB[r] * k0 * fast_exp(g0);
                tK[r * LT + cc + 1] = sB[r] * k1 * fast_exp(g1);
            });
        } else {
            for_each_elem<C * CT>(tid, [&](int e) {  // token-major outputs; K becomes beta K+ in place
                const int r = e / CT, cc = e % CT;
                const float g = tG[r * LT + cc], gl = tG[(C - 1) * LT + cc], kk = tK[r * LT + cc];
                rec[R::Kd + r * DK + c0 + cc] = kk * fast_exp(gl - g);
                tK[r * LT + cc] = sB[r] * kk * fast_exp(g);
            });
        }
        if (tid < CT) rec[R::gam + c0 + tid] = fast_exp(tG[(C - 1) * LT + tid]);
        lds_barrier();
        for_each_wave<NR * (CT / 16)>(w, [&](int t) {
            const int rb = t % NR, cb = t / NR;
            const floatx4 acc = mma<C / 4>(sT + 16 * rb * LC, LC, 1, tK + 16 * cb, LT, 1, zero4(), lane);
            if constexpr (SPLIT) {
                // W: the lanes of a column pair swap half their rows, so each writes two rows of a
                // column pair
                const bool odd = lr & 1;
                const float r0 = __shfl_xor(odd ? acc[0] : acc[2], 1), r1 = __shfl_xor(odd ? acc[1] : acc[3], 1);
                const int row = 16 * rb + 4 * lg + (odd ? 2 : 0), col = c0 + 16 * cb + (lr & ~1);
                put_pair(rec, R::W, C * DK, row * DK + col, odd ? r0 : acc[0], odd ? acc[2] : r0);
                put_pair(rec, R::W, C * DK, (row + 1) * DK + col, odd ? r1 : acc[1], odd ? acc[3] : r1);
                bf16x4 hi, lo;
                split4(make_float4(acc[0], acc[1], acc[2], acc[3]), hi, lo);
                const int64_t i = (int64_t)(c0 + 16 * cb + lr) * C + 16 * rb + 4 * lg;
                bf16x4* p = reinterpret_cast<bf16x4*>(rec + R::WT);
                p[i >> 2] = hi;
                p[(DK * C + i) >> 2] = lo;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) rec[R::W + (16 * rb + 4 * lg + e) * DK + c0 + 16 * cb + lr] = acc[e];
                *reinterpret_cast<float4*>(rec + R::WT + (int64_t)(c0 + 16 * cb + lr) * C + 16 * rb + 4 * lg) =
                    make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
        });
        lds_barrier();
    }
    // ---- pass 3: U = T (beta V), value tile by value tile (beta V staged in q's buffer)
#pragma unroll
    for (int j0 = 0; j0 < DV; j0 += VT) {
#pragma unroll
        for (int m = 0; m < VPT; ++m) {
            const int e = tid + kThreads * m, r = e / VT, j = e % VT;
            if (VPT * kThreads == C * VT || e < C * VT) tQ[r * LT + j] = sB[r] * vr[m];
        }
        fetch_value(j0 + VT < DV ? j0 + VT : j0);
        lds_barrier();
        for_each_wave<NR * (VT / 16)>(w, [&](int t) {
            const int rb = t % NR, cb = t / NR;
            const floatx4 acc = mma<C / 4>(sT + 16 * rb * LC, LC, 1, tQ + 16 * cb, LT, 1, zero4(), lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) rec[R::U + (16 * rb + 4 * lg + e) * DV + j0 + 16 * cb + lr] = acc[e];
        });
        lds_barrier();
    }
}

// ------------------------------------------------------------------------------------------
// Chain operands: the next chunk's record rows are loaded into registers while the current chunk
// computes from LDS, then written to LDS for the next step.  rows x cols floats (cols a multiple
// of 4) go to an LDS array with row stride ld.
// ------------------------------------------------------------------------------------------
template <int ROWS, int COLS>
struct Stage {
    static constexpr int kVec = ROWS * COLS / 4;
    static constexpr int kPer = (kVec + kThreads - 1) / kThreads;
    float4 r[kPer];
    // src: row-major with row stride src_ld floats (16-byte aligned rows)
    __device__ __forceinline__ void load(const float* src, int64_t src_ld) {
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int e = threadIdx.x + m * kThreads;
            if (kVec % kThreads == 0 || e < kVec) {
                const int row = e / (COLS / 4), c4 = e % (COLS / 4);
                r[m] = *reinterpret_cast<const float4*>(src + row * src_ld + 4 * c4);
            }
        }
    }
    __device__ __forceinline__ void store(float* dst, int ld) const {
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int e = threadIdx.x + m * kThreads;
            if (kVec % kThreads == 0 || e < kVec) {
                const int row = e / (COLS / 4), c4 = e % (COLS / 4);
                float* p = dst + row * ld + 4 * c4;  // 16-byte aligned: ld is a multiple of 4
                p[0] = r[m].x;
                p[1] = r[m].y;
                p[2] = r[m].z;
                p[3] = r[m].w;
            }
        }
    }
};

// Warm L2 with floats [off, off + n) of a record ahead of its use: the nvb chain workgroups of a
// sequence-head read the same record, so value block vb touches every nvb-th 128-byte line of the
// range, with 4-byte direct-to-LDS loads into a dummy slot (no registers are written and nothing
// waits on them).  Unconditional (lanes past the end repeat the last line), so the compiler's
// load counting for the operand prefetch stays exact.
template <int64_t N>
__device__ __forceinline__ void warm_range(const float* rec, int64_t off, int vb, int nvb,
                                           __attribute__((address_space(3))) void* dummy) {
    constexpr int64_t kLines = (N * 4 + 127) / 128;
    const int64_t per = (kLines + nvb - 1) / nvb;
#pragma unroll
    for (int m = 0; m < (int)((kLines + kThreads - 1) / kThreads); ++m) {
        int64_t i = threadIdx.x + (int64_t)kThreads * m;
        if (i >= per) i = per - 1;
        int64_t line = vb + (int64_t)nvb * i;
        if (line >= kLines) line = kLines - 1;
        __builtin_amdgcn_global_load_lds(rec + off + line * 32, dummy, 4, 0, 0);
    }
}

// Chain workgroup -> (sequence-head, value block).  Workgroups are dealt to the 8 XCDs round-robin;
// when the sequence-heads divide into 8, the value blocks of one sequence-head go to one XCD so that
// they share its L2 (each reads the same per-chunk record).
template <int NVB>
__device__ __forceinline__ void chain_unit(int64_t gid, int64_t nh_total, int64_t& nh, int& vb) {
    if ((nh_total & 7) == 0) {
        const int64_t xcd = gid & 7, u = gid >> 3;
        vb = (int)(u % NVB);
        nh = xcd + 8 * (u / NVB);
    } else {
        vb = (int)(gid % NVB);
        nh = gid / NVB;
    }
}

// ------------------------------------------------------------------------------------------
// fwd_chain: one workgroup per (sequence, head, 16 value columns); states entering each chunk.
// Every product reads both operands contiguous along its contraction index (mma_k4): the state
// block and D are kept transposed in LDS ([value column][contraction index]).
// ------------------------------------------------------------------------------------------
template <int DK, int DV, int C>
__global__ __launch_bounds__(kThreads) void fwd_chain_kernel(BwdArgs a, Map<C> mp) {
    using R = Rec<DK, DV, C>;
    constexpr int NVB = DV / kBV, LW = DK + 4, LT = C + 4;
    __shared__ __attribute__((aligned(16))) float sW[C * LW];    // W: A of W S
    __shared__ __attribute__((aligned(16))) float sKT[DK * LT];  // K'^T: A of K'^T D
    __shared__ __attribute__((aligned(16))) float sU[C * kBV];
    __shared__ __attribute__((aligned(16))) float sg[DK];
    __shared__ __attribute__((aligned(16))) float sSt[kBV * LW];  // state block [column][key channel]
    __shared__ __attribute__((aligned(16))) float sDt[kBV * LT];  // D [column][token]
    __shared__ __attribute__((aligned(16))) float sDummy[64];     // sink of the L2 warm-up loads
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
    int64_t nh;
    int vb;
    chain_unit<NVB>(blockIdx.x, mp.N * a.H, nh, vb);
    auto* dummy = reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(&sDummy[0]));
    const int h = (int)(nh % a.H);
    const int64_t n = nh / a.H;
    const int H = a.H;
    for (int e = tid; e < DK * kBV; e += kThreads) {
        const int i = e / kBV, j = e % kBV;
        sSt[j * LW + i] = a.s0 ? a.s0[((n * H + h) * DK + i) * (int64_t)DV + vb * kBV + j] : 0.f;
    }
    const int64_t slot0 = mp.base(n);
    int64_t c0, c1;
    mp.range(n, c0, c1);
    float* s_fin = a.s_fin ? a.s_fin + ((n * H + h) * DK) * (int64_t)DV + vb * kBV : nullptr;
    if (c0 >= c1) {  // uniform: no chunk here, the state passes through (each thread its own elements)
        if (s_fin)
            for (int e = tid; e < DK * kBV; e += kThreads) s_fin[(e / kBV) * DV + e % kBV] = sSt[(e % kBV) * LW + e / kBV];
        return;
    }
    Stage<C, DK> pW;
    Stage<DK, C> pK;
    Stage<C, kBV> pU;
    Stage<1, DK> pg;
    auto fetch = [&](int64_t c) {
        const float* rec = a.ws + ((slot0 + c) * H + h) * R::kFloats;
        pW.load(rec + R::W, DK);
        pK.load(rec + R::KdT, C);
        pU.load(rec + R::U + vb * kBV, DV);
        pg.load(rec + R::gam, DK);
    };
    fetch(c0);
    for (int64_t c = c0; c < c1; ++c) {
        float* rec = a.ws + ((slot0 + c) * H + h) * R::kFloats;
        lds_barrier();  // the previous chunk is done with the LDS operands; sSt is its final state
        pW.store(sW, LW);
        pK.store(sKT, LT);
        pU.store(sU, kBV);
        pg.store(sg, DK);
        for_each_elem<DK * kBV>(tid, [&](int e) {
            rec[R::S0 + (e / kBV) * DV + vb * kBV + e % kBV] = sSt[(e % kBV) * LW + e / kBV];
        });
        lds_barrier();
        // D = U - W S (rows 16 w .. 16 w + 15 per wave)
        for_each_wave<C / 16>(w, [&](int rb) {
            const floatx4 acc = mma_k4<DK / 16>(sW + 16 * rb * LW, LW, sSt, LW, zero4(), lane);
            float4 dv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * lg + e;
                const float d = sU[r * kBV + lr] - acc[e];
                (&dv.x)[e] = d;
                rec[R::D + r * DV + vb * kBV + lr] = d;
            }
            *reinterpret_cast<float4*>(sDt + lr * LT + 16 * rb + 4 * lg) = dv;
        });
        lds_barrier();
        // the next chunk's operands and the L2 warm-up are requested here, after D: issued before
        // it, their loads held up the product that the next barrier waits for
        fetch(c + 1 < c1 ? c + 1 : c);
        {  // W, U and K'^T (one contiguous range) of the chunk kWarm ahead
            const float* wrec = a.ws + ((slot0 + (c + kWarm < c1 ? c + kWarm : c1 - 1)) * H + h) * R::kFloats;
            warm_range<R::Kd>(wrec, 0, vb, NVB, dummy);
        }
        // S <- Diag(gamma) S + K'^T D
        for_each_wave<DK / 16>(w, [&](int cb) {
            const int i0 = 16 * cb + 4 * lg;
            const float4 s4 = *reinterpret_cast<const float4*>(sSt + lr * LW + i0);
            floatx4 acc = {sg[i0] * s4.x, sg[i0 + 1] * s4.y, sg[i0 + 2] * s4.z, sg[i0 + 3] * s4.w};
            acc = mma_k4<C / 16>(sKT + 16 * cb * LT, LT, sDt, LT, acc, lane);
            *reinterpret_cast<float4*>(sSt + lr * LW + i0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        });
    }
    if (s_fin) {  // the state after the last chunk (a checkpoint for a later window)
        lds_barrier();
        for (int e = tid; e < DK * kBV; e += kThreads) s_fin[(e / kBV) * DV + e % kBV] = sSt[(e % kBV) * LW + e / kBV];
    }
}

// ------------------------------------------------------------------------------------------
// fwd_chain with split-bf16 operands (bfloat16 storage at d = 128, chunk 64).  W and K'^T arrive as
// bf16 hi and lo from the factors kernel and are staged as they are; the state block is kept in
// fp32 (for gamma * S and the stored S0) and, beside it, as bf16 hi and lo for the product W S; D
// likewise for K'^T D.
// ------------------------------------------------------------------------------------------
template <int DK, int DV, int C>
__global__ __launch_bounds__(kThreads) void fwd_chain_split_kernel(BwdArgs a, Map<C> mp) {
    using R = Rec<DK, DV, C>;
    static_assert(DK == 128 && DV == 128 && C == 64, "split-bf16 chains cover the d = 128, chunk 64 shape");
    // row strides in floats; the bf16 arrays hold packed pairs (k + 8 bf16 per row)
    constexpr int NVB = DV / kBV, NR = C / 16, LW = DK + 4, LWh = DK / 2 + 4, LTh = C / 2 + 4;
    __shared__ __attribute__((aligned(16))) float sW[2][C * LWh];    // W hi, lo [token][channel]: A of W S
    __shared__ __attribute__((aligned(16))) float sKT[2][DK * LTh];  // K'^T hi, lo [channel][token]: A of K'^T D
    __shared__ __attribute__((aligned(16))) float sU[C * kBV];
    __shared__ __attribute__((aligned(16))) float sg[DK];
    __shared__ __attribute__((aligned(16))) float sSt[kBV * LW];     // state block, fp32 [column][channel]
    __shared__ __attribute__((aligned(16))) float sSh[2][kBV * LWh]; // its hi, lo: B of W S
    __shared__ __attribute__((aligned(16))) float sDh[2][kBV * LTh]; // D hi, lo [column][token]: B of K'^T D
    __shared__ __attribute__((aligned(16))) float sDummy[64];        // sink of the L2 warm-up loads
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
    int64_t nh;
    int vb;
    chain_unit<NVB>(blockIdx.x, mp.N * a.H, nh, vb);
    auto* dummy = reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(&sDummy[0]));
    const int h = (int)(nh % a.H);
    const int64_t n = nh / a.H;
    const int H = a.H;
    for (int e = tid; e < DK * kBV; e += kThreads) {
        const int i = e / kBV, j = e % kBV;
        const float x = a.s0 ? a.s0[((n * H + h) * DK + i) * (int64_t)DV + vb * kBV + j] : 0.f;
        sSt[j * LW + i] = x;
        const __bf16 hi = (__bf16)x;
        reinterpret_cast<__bf16*>(sSh[0])[j * 2 * LWh + i] = hi;
        reinterpret_cast<__bf16*>(sSh[1])[j * 2 * LWh + i] = (__bf16)(x - (float)hi);
    }
    const int64_t slot0 = mp.base(n);
    int64_t c0, c1;
    mp.range(n, c0, c1);
    float* s_fin = a.s_fin ? a.s_fin + ((n * H + h) * DK) * (int64_t)DV + vb * kBV : nullptr;
    if (c0 >= c1) {  // uniform: no chunk here, the state passes through (each thread its own elements)
        if (s_fin)
            for (int e = tid; e < DK * kBV; e += kThreads) s_fin[(e / kBV) * DV + e % kBV] = sSt[(e % kBV) * LW + e / kBV];
        return;
    }
    Stage<C, DK / 2> pWh, pWl;
    Stage<DK, C / 2> pKh, pKl;
    Stage<C, kBV> pU;
    Stage<1, DK> pg;
    auto fetch = [&](int64_t c) {
        const float* rec = a.ws + ((slot0 + c) * H + h) * R::kFloats;
        pWh.load(rec + R::W, DK / 2);
        pWl.load(rec + R::W + C * DK / 2, DK / 2);
        pKh.load(rec + R::KdT, C / 2);
        pKl.load(rec + R::KdT + DK * C / 2, C / 2);
        pU.load(rec + R::U + vb * kBV, DV);
        pg.load(rec + R::gam, DK);
    };
    fetch(c0);
    for (int64_t c = c0; c < c1; ++c) {
        float* rec = a.ws + ((slot0 + c) * H + h) * R::kFloats;
        lds_barrier();  // the previous chunk is done with the LDS operands; the state is its final state
        pWh.store(sW[0], LWh);
        pWl.store(sW[1], LWh);
        pKh.store(sKT[0], LTh);
        pKl.store(sKT[1], LTh);
        pU.store(sU, kBV);
        pg.store(sg, DK);
        for_each_elem<DK * kBV>(tid, [&](int e) {
            rec[R::S0 + (e / kBV) * DV + vb * kBV + e % kBV] = sSt[(e % kBV) * LW + e / kBV];
        });
        lds_barrier();
        // D = U - W S (rows 16 w .. 16 w + 15)
        if (w < NR) {
            floatx4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks)
                acc = mfma_split(frag16(sW[0], 16 * w, LWh, ks, lane), frag16(sW[1], 16 * w, LWh, ks, lane),
                                 frag16(sSh[0], 0, LWh, ks, lane), frag16(sSh[1], 0, LWh, ks, lane), acc);
            float4 dv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * w + 4 * lg + e;
                const float d = sU[r * kBV + lr] - acc[e];
                (&dv.x)[e] = d;
                rec[R::D + r * DV + vb * kBV + lr] = d;
            }
            bf16x4 dh, dl;
            split4(dv, dh, dl);
            *reinterpret_cast<bf16x4*>(sDh[0] + lr * LTh + 8 * w + 2 * lg) = dh;
            *reinterpret_cast<bf16x4*>(sDh[1] + lr * LTh + 8 * w + 2 * lg) = dl;
        }
        lds_barrier();
        // the next chunk's operands and the L2 warm-up are requested here, after D (issued right after
        // the staging stores instead, they made this chain slower: 2.46 against 2.42 ms)
        fetch(c + 1 < c1 ? c + 1 : c);
        {  // W, U and K'^T (one contiguous range) of the chunk kWarm ahead
            const float* wrec = a.ws + ((slot0 + (c + kWarm < c1 ? c + kWarm : c1 - 1)) * H + h) * R::kFloats;
            warm_range<R::Kd>(wrec, 0, vb, NVB, dummy);
        }
        // S <- Diag(gamma) S + K'^T D
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int cb = w + 4 * t;
            const int i0 = 16 * cb + 4 * lg;
            const float4 s4 = *reinterpret_cast<const float4*>(sSt + lr * LW + i0);
            floatx4 acc = {sg[i0] * s4.x, sg[i0 + 1] * s4.y, sg[i0 + 2] * s4.z, sg[i0 + 3] * s4.w};
#pragma unroll
            for (int ks = 0; ks < C / 32; ++ks)
                acc = mfma_split(frag16(sKT[0], 16 * cb, LTh, ks, lane), frag16(sKT[1], 16 * cb, LTh, ks, lane),
                                 frag16(sDh[0], 0, LTh, ks, lane), frag16(sDh[1], 0, LTh, ks, lane), acc);
            const float4 ns = make_float4(acc[0], acc[1], acc[2], acc[3]);
            *reinterpret_cast<float4*>(sSt + lr * LW + i0) = ns;
            bf16x4 hh, ll;
            split4(ns, hh, ll);
            *reinterpret_cast<bf16x4*>(sSh[0] + lr * LWh + 8 * cb + 2 * lg) = hh;
            *reinterpret_cast<bf16x4*>(sSh[1] + lr * LWh + 8 * cb + 2 * lg) = ll;
        }
    }
    if (s_fin) {  // the state after the last chunk (a checkpoint for a later window)
        lds_barrier();
        for (int e = tid; e < DK * kBV; e += kThreads) s_fin[(e / kBV) * DV + e % kBV] = sSt[(e % kBV) * LW + e / kBV];
    }
}

// ------------------------------------------------------------------------------------------
// rev_chain: one workgroup per (sequence, head, 16 value columns); chunks in reverse.  dS, dO and
// dD are kept transposed in LDS ([value column][contraction index]).
// ------------------------------------------------------------------------------------------
template <int DK, int DV, int C>
__global__ __launch_bounds__(kThreads) void rev_chain_kernel(BwdArgs a, Map<C> mp) {
    using R = Rec<DK, DV, C>;
    constexpr int NVB = DV / kBV, LW = DK + 4, LT = C + 4;
    __shared__ __attribute__((aligned(16))) float sKd[C * LW];   // K': A of K' dS
    __shared__ __attribute__((aligned(16))) float sMT[C * LT];   // M^T: A of M^T dO
    __shared__ __attribute__((aligned(16))) float sQT[DK * LT];  // Q+^T: A of Q+^T dO
    __shared__ __attribute__((aligned(16))) float sWT[DK * LT];  // W^T: A of W^T dD
    __shared__ __attribute__((aligned(16))) float sg[DK];
    __shared__ __attribute__((aligned(16))) float sdSt[kBV * LW];  // dS [column][key channel]
    __shared__ __attribute__((aligned(16))) float sdOt[kBV * LT];  // dO [column][token]
    __shared__ __attribute__((aligned(16))) float sdDt[kBV * LT];  // dD [column][token]
    __shared__ __attribute__((aligned(16))) float sDummy[64];      // sink of the L2 warm-up loads
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
    int64_t nh;
    int vb;
    chain_unit<NVB>(blockIdx.x, mp.N * a.H, nh, vb);
    auto* dummy = reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(&sDummy[0]));
    const int h = (int)(nh % a.H);
    const int64_t n = nh / a.H;
    const int H = a.H;
    for (int e = tid; e < DK * kBV; e += kThreads) {
        const int i = e / kBV, j = e % kBV;
        sdSt[j * LW + i] = a.dsT ? a.dsT[((n * H + h) * DK + i) * (int64_t)DV + vb * kBV + j] : 0.f;
    }
    const int64_t bos = mp.cu[n], eos = mp.cu[n + 1];
    const int64_t slot0 = mp.base(n);
    int64_t c0, c1;
    mp.range(n, c0, c1);
    Stage<C, DK> pK;
    Stage<C, C> pM;
    Stage<DK, C> pQ, pW;
    Stage<1, DK> pg;
    constexpr int kDoPer = (C * kBV + kThreads - 1) / kThreads;
    float rdo[kDoPer];
    auto fetch = [&](int64_t c) {
        const float* rec = a.ws + ((slot0 + c) * H + h) * R::kFloats;
        pK.load(rec + R::Kd, DK);
        pM.load(rec + R::MT, C);
        pQ.load(rec + R::QpT, C);
        pW.load(rec + R::WT, C);
        pg.load(rec + R::gam, DK);
        const int64_t t0 = bos + c * C;
#pragma unroll
        for (int m = 0; m < kDoPer; ++m) {
            const int e = tid + m * kThreads, r = e / kBV, j = e % kBV;
            const bool in = e < C * kBV && t0 + r < eos;
            const int64_t tr = in ? t0 + r : eos - 1;
            const float x = a.dO[(tr * H + h) * (int64_t)DV + vb * kBV + j];
            rdo[m] = in ? x : 0.f;
        }
    };
    if (c1 > c0) fetch(c1 - 1);
    for (int64_t c = c1 - 1; c >= c0; --c) {
        float* rec = a.ws + ((slot0 + c) * H + h) * R::kFloats;
        lds_barrier();  // the previous chunk is done with the LDS operands; sdSt is its result
        pK.store(sKd, LW);
        pM.store(sMT, LT);
        pQ.store(sQT, LT);
        pW.store(sWT, LT);
        pg.store(sg, DK);
#pragma unroll
        for (int m = 0; m < kDoPer; ++m) {
            const int e = tid + m * kThreads;
            if (e < C * kBV) sdOt[(e % kBV) * LT + e / kBV] = rdo[m];
        }
        for_each_elem<DK * kBV>(tid, [&](int e) {
            rec[R::dS1 + (e / kBV) * DV + vb * kBV + e % kBV] = sdSt[(e % kBV) * LW + e / kBV];
        });
        lds_barrier();
        // dD = K' dS + M^T dO
        for_each_wave<C / 16>(w, [&](int rb) {
            floatx4 acc = mma_k4<DK / 16>(sKd + 16 * rb * LW, LW, sdSt, LW, zero4(), lane);
            acc = mma_k4<C / 16>(sMT + 16 * rb * LT, LT, sdOt, LT, acc, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) rec[R::dD + (16 * rb + 4 * lg + e) * DV + vb * kBV + lr] = acc[e];
            *reinterpret_cast<float4*>(sdDt + lr * LT + 16 * rb + 4 * lg) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        });
        lds_barrier();
        // the previous chunk's operands and the L2 warm-up are requested here, after dD (see
        // fwd_chain)
        fetch(c > c0 ? c - 1 : c);
        {  // K', Q+^T, W^T and M^T (one contiguous range) of the chunk kWarm behind
            const float* wrec = a.ws + ((slot0 + (c - kWarm >= c0 ? c - kWarm : c0)) * H + h) * R::kFloats;
            warm_range<R::T - R::Kd>(wrec, R::Kd, vb, NVB, dummy);
        }
        // dS <- Diag(gamma) dS + Q+^T dO - W^T dD
        for_each_wave<DK / 16>(w, [&](int cb) {
            const int i0 = 16 * cb + 4 * lg;
            const float4 s4 = *reinterpret_cast<const float4*>(sdSt + lr * LW + i0);
            floatx4 acc = {sg[i0] * s4.x, sg[i0 + 1] * s4.y, sg[i0 + 2] * s4.z, sg[i0 + 3] * s4.w};
            acc = mma_k4<C / 16>(sQT + 16 * cb * LT, LT, sdOt, LT, acc, lane);
            const floatx4 wd = mma_k4<C / 16>(sWT + 16 * cb * LT, LT, sdDt, LT, zero4(), lane);
            *reinterpret_cast<float4*>(sdSt + lr * LW + i0) =
                make_float4(acc[0] - wd[0], acc[1] - wd[1], acc[2] - wd[2], acc[3] - wd[3]);
        });
    }
    lds_barrier();
    if (a.gs0)
        for (int e = tid; e < DK * kBV; e += kThreads) {
            const int i = e / kBV, j = e % kBV;
            a.gs0[((n * H + h) * DK + i) * (int64_t)DV + vb * kBV + j] = sdSt[j * LW + i];
        }
}

// ------------------------------------------------------------------------------------------
// rev_chain with split-bf16 operands (bfloat16 storage at d = 128, chunk 64): K', M^T, Q+^T and W^T
// arrive as bf16 hi and lo; dS is kept in fp32 (for gamma * dS and the stored dS1) and, beside it,
// as bf16 hi and lo for K' dS; dO and dD as bf16 hi and lo.
// ------------------------------------------------------------------------------------------
template <int DK, int DV, int C>
__global__ __launch_bounds__(kThreads) void rev_chain_split_kernel(BwdArgs a, Map<C> mp) {
    using R = Rec<DK, DV, C>;
    static_assert(DK == 128 && DV == 128 && C == 64, "split-bf16 chains cover the d = 128, chunk 64 shape");
    constexpr int NVB = DV / kBV, NR = C / 16, LW = DK + 4, LWh = DK / 2 + 4, LTh = C / 2 + 4;
    __shared__ __attribute__((aligned(16))) float sK[2][C * LWh];     // K' hi, lo [token][channel]: A of K' dS
    __shared__ __attribute__((aligned(16))) float sM[2][C * LTh];     // M^T hi, lo: A of M^T dO
    __shared__ __attribute__((aligned(16))) float sQ[2][DK * LTh];    // Q+^T hi, lo: A of Q+^T dO
    __shared__ __attribute__((aligned(16))) float sW[2][DK * LTh];    // W^T hi, lo: A of W^T dD
    __shared__ __attribute__((aligned(16))) float sg[DK];
    __shared__ __attribute__((aligned(16))) float sdSt[kBV * LW];     // dS, fp32 [column][channel]
    __shared__ __attribute__((aligned(16))) float sdSh[2][kBV * LWh]; // its hi, lo: B of K' dS
    __shared__ __attribute__((aligned(16))) float sdOh[2][kBV * LTh]; // dO hi, lo [column][token]
    __shared__ __attribute__((aligned(16))) float sdDh[2][kBV * LTh]; // dD hi, lo [column][token]
    __shared__ __attribute__((aligned(16))) float sDummy[64];         // sink of the L2 warm-up loads
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
    int64_t nh;
    int vb;
    chain_unit<NVB>(blockIdx.x, mp.N * a.H, nh, vb);
    auto* dummy = reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(&sDummy[0]));
    const int h = (int)(nh % a.H);
    const int64_t n = nh / a.H;
    const int H = a.H;
    for (int e = tid; e < DK * kBV; e += kThreads) {
        const int i = e / kBV, j = e % kBV;
        const float x = a.dsT ? a.dsT[((n * H + h) * DK + i) * (int64_t)DV + vb * kBV + j] : 0.f;
        sdSt[j * LW + i] = x;
        const __bf16 hi = (__bf16)x;
        reinterpret_cast<__bf16*>(sdSh[0])[j * 2 * LWh + i] = hi;
        reinterpret_cast<__bf16*>(sdSh[1])[j * 2 * LWh + i] = (__bf16)(x - (float)hi);
    }
    const int64_t bos = mp.cu[n], eos = mp.cu[n + 1];
    const int64_t slot0 = mp.base(n);
    int64_t c0, c1;
    mp.range(n, c0, c1);
    Stage<C, DK / 2> pKh, pKl;
    Stage<C, C / 2> pMh, pMl;
    Stage<DK, C / 2> pQh, pQl, pWh, pWl;
    Stage<1, DK> pg;
    constexpr int kDoPer = (C * kBV + kThreads - 1) / kThreads;
    float rdo[kDoPer];
    auto fetch = [&](int64_t c) {
        const float* rec = a.ws + ((slot0 + c) * H + h) * R::kFloats;
        pKh.load(rec + R::Kd, DK / 2);
        pKl.load(rec + R::Kd + C * DK / 2, DK / 2);
        pMh.load(rec + R::MT, C / 2);
        pMl.load(rec + R::MT + C * C / 2, C / 2);
        pQh.load(rec + R::QpT, C / 2);
        pQl.load(rec + R::QpT + DK * C / 2, C / 2);
        pWh.load(rec + R::WT, C / 2);
        pWl.load(rec + R::WT + DK * C / 2, C / 2);
        pg.load(rec + R::gam, DK);
        // dO rows of the chunk through a descriptor that ends at the sequence's last token (0 past it),
        // so no select waits on the loads
        const int64_t t0 = bos + c * C;
        const int64_t L = eos - t0 < C ? eos - t0 : C;
        const __amdgpu_buffer_rsrc_t drs =
            make_rsrc(a.dO + (t0 * H + h) * (int64_t)DV + vb * kBV, (uint32_t)(((L - 1) * H * DV + kBV) * 4));
        static_assert(kDoPer * kThreads == C * kBV, "dO tile split evenly over the threads");
#pragma unroll
        for (int m = 0; m < kDoPer; ++m) {
            const int e = tid + m * kThreads, r = e / kBV, j = e % kBV;
            rdo[m] = ld_buf<float>(drs, r * H * DV + j);
        }
    };
    if (c1 > c0) fetch(c1 - 1);
    for (int64_t c = c1 - 1; c >= c0; --c) {
        float* rec = a.ws + ((slot0 + c) * H + h) * R::kFloats;
        lds_barrier();  // the previous chunk is done with the LDS operands; dS is its result
        pKh.store(sK[0], LWh);
        pKl.store(sK[1], LWh);
        pMh.store(sM[0], LTh);
        pMl.store(sM[1], LTh);
        pQh.store(sQ[0], LTh);
        pQl.store(sQ[1], LTh);
        pWh.store(sW[0], LTh);
        pWl.store(sW[1], LTh);
        pg.store(sg, DK);
#pragma unroll
        for (int m = 0; m < kDoPer; ++m) {
            const int e = tid + m * kThreads;
            if (e < C * kBV) {
                const int r = e / kBV, j = e % kBV;
                const __bf16 hi = (__bf16)rdo[m];  // rows past the sequence's end read 0
                reinterpret_cast<__bf16*>(sdOh[0])[j * 2 * LTh + r] = hi;
                reinterpret_cast<__bf16*>(sdOh[1])[j * 2 * LTh + r] = (__bf16)(rdo[m] - (float)hi);
            }
        }
        // the previous chunk's operands are requested as soon as the staging registers are free, so
        // that dD and the dS update of this chunk hide their latency
        fetch(c > c0 ? c - 1 : c);
        for_each_elem<DK * kBV>(tid, [&](int e) {
            rec[R::dS1 + (e / kBV) * DV + vb * kBV + e % kBV] = sdSt[(e % kBV) * LW + e / kBV];
        });
        lds_barrier();
        // dD = K' dS + M^T dO (rows 16 w .. 16 w + 15)
        if (w < NR) {
            floatx4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks)
                acc = mfma_split(frag16(sK[0], 16 * w, LWh, ks, lane), frag16(sK[1], 16 * w, LWh, ks, lane),
                                 frag16(sdSh[0], 0, LWh, ks, lane), frag16(sdSh[1], 0, LWh, ks, lane), acc);
#pragma unroll
            for (int ks = 0; ks < C / 32; ++ks)
                acc = mfma_split(frag16(sM[0], 16 * w, LTh, ks, lane), frag16(sM[1], 16 * w, LTh, ks, lane),
                                 frag16(sdOh[0], 0, LTh, ks, lane), frag16(sdOh[1], 0, LTh, ks, lane), acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) rec[R::dD + (16 * w + 4 * lg + e) * DV + vb * kBV + lr] = acc[e];
            bf16x4 dh, dl;
            split4(make_float4(acc[0], acc[1], acc[2], acc[3]), dh, dl);
            *reinterpret_cast<bf16x4*>(sdDh[0] + lr * LTh + 8 * w + 2 * lg) = dh;
            *reinterpret_cast<bf16x4*>(sdDh[1] + lr * LTh + 8 * w + 2 * lg) = dl;
        }
        lds_barrier();
        {  // the L2 warm-up, after dD: K', Q+^T, W^T and M^T (one contiguous range) of the chunk kWarm behind
            const float* wrec = a.ws + ((slot0 + (c - kWarm >= c0 ? c - kWarm : c0)) * H + h) * R::kFloats;
            warm_range<R::T - R::Kd>(wrec, R::Kd, vb, NVB, dummy);
        }
        // dS <- Diag(gamma) dS + Q+^T dO - W^T dD
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int cb = w + 4 * t;
            const int i0 = 16 * cb + 4 * lg;
            const float4 s4 = *reinterpret_cast<const float4*>(sdSt + lr * LW + i0);
            floatx4 acc = {sg[i0] * s4.x, sg[i0 + 1] * s4.y, sg[i0 + 2] * s4.z, sg[i0 + 3] * s4.w};
            floatx4 wd = zero4();
#pragma unroll
            for (int ks = 0; ks < C / 32; ++ks) {
                acc = mfma_split(frag16(sQ[0], 16 * cb, LTh, ks, lane), frag16(sQ[1], 16 * cb, LTh, ks, lane),
                                 frag16(sdOh[0], 0, LTh, ks, lane), frag16(sdOh[1], 0, LTh, ks, lane), acc);
                wd = mfma_split(frag16(sW[0], 16 * cb, LTh, ks, lane), frag16(sW[1], 16 * cb, LTh, ks, lane),
                                frag16(sdDh[0], 0, LTh, ks, lane), frag16(sdDh[1], 0, LTh, ks, lane), wd);
            }
            const float4 ns = make_float4(acc[0] - wd[0], acc[1] - wd[1], acc[2] - wd[2], acc[3] - wd[3]);
            *reinterpret_cast<float4*>(sdSt + lr * LW + i0) = ns;
            bf16x4 hh, ll;
            split4(ns, hh, ll);
            *reinterpret_cast<bf16x4*>(sdSh[0] + lr * LWh + 8 * cb + 2 * lg) = hh;
            *reinterpret_cast<bf16x4*>(sdSh[1] + lr * LWh + 8 * cb + 2 * lg) = ll;
        }
    }
    lds_barrier();
    if (a.gs0)
        for (int e = tid; e < DK * kBV; e += kThreads) {
            const int i = e / kBV, j = e % kBV;
            a.gs0[((n * H + h) * DK + i) * (int64_t)DV + vb * kBV + j] = sdSt[j * LW + i];
        }
}

// ------------------------------------------------------------------------------------------
// grad_state: one workgroup per (chunk slot, head); the products over the value axis, staged
// through LDS 32 value columns at a time
// ------------------------------------------------------------------------------------------
template <int DK, int DV, int C>
__global__ __launch_bounds__(kThreads) void grad_state_kernel(BwdArgs a, Map<C> mp) {
    using R = Rec<DK, DV, C>;
    constexpr int JT = DV < 32 ? DV : 32, LJ = JT + 4;
    constexpr int NR = C / 16, NC = DK / 16, NT3 = NR * NC, NTM = NR * NR;
    constexpr int T3W = (NT3 + 3) / 4, TMW = (NTM + 3) / 4;
    __shared__ __attribute__((aligned(16))) float sD[C * LJ];
    __shared__ __attribute__((aligned(16))) float sdD[C * LJ];
    __shared__ __attribute__((aligned(16))) float sdO[C * LJ];
    __shared__ __attribute__((aligned(16))) float sS0[DK * LJ];
    __shared__ __attribute__((aligned(16))) float sdS1[DK * LJ];
    const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t slot = blockIdx.x;
    int64_t n, c, t0;
    int L;
    if (!mp.locate(slot, n, c, t0, L)) return;
    const int H = a.H;
    float* rec = a.ws + (slot * H + h) * R::kFloats;
    floatx4 kd[T3W], qp[T3W], dw[T3W], dm[TMW];
#pragma unroll
    for (int m = 0; m < T3W; ++m) kd[m] = qp[m] = dw[m] = zero4();
#pragma unroll
    for (int m = 0; m < TMW; ++m) dm[m] = zero4();
    float dgam = 0.f;
    // value tile j0 .. j0 + JT - 1 of D, dD, S0, dS1 (record) and dO (rows >= L zero), one tile ahead
    Stage<C, JT> pD, pdD;
    Stage<DK, JT> pS, pdS;
    constexpr int kDoPer = (C * JT + kThreads - 1) / kThreads;
    float rdo[kDoPer];
    auto fetch = [&](int j0) {
        pD.load(rec + R::D + j0, DV);
        pdD.load(rec + R::dD + j0, DV);
        pS.load(rec + R::S0 + j0, DV);
        pdS.load(rec + R::dS1 + j0, DV);
#pragma unroll
        for (int m = 0; m < kDoPer; ++m) {
            const int e = tid + m * kThreads, r = e / JT, j = e % JT;
            const bool in = e < C * JT && r < L;
            const int rr = in ? r : L - 1;
            const float x = a.dO[((t0 + rr) * H + h) * (int64_t)DV + j0 + j];
            rdo[m] = in ? x : 0.f;
        }
    };
    fetch(0);
    for (int j0 = 0; j0 < DV; j0 += JT) {
        pD.store(sD, LJ);
        pdD.store(sdD, LJ);
        pS.store(sS0, LJ);
        pdS.store(sdS1, LJ);
#pragma unroll
        for (int m = 0; m < kDoPer; ++m) {
            const int e = tid + m * kThreads;
            if (e < C * JT) sdO[(e / JT) * LJ + e % JT] = rdo[m];
        }
        fetch(j0 + JT < DV ? j0 + JT : j0);
        lds_barrier();
        // dK' = D dS1^T, dQ+ = dO S0^T, dW = -dD S0^T   ([C][DK] each)
#pragma unroll
        for (int m = 0; m < T3W; ++m) {
            const int t = w + 4 * m, rb = t % NR, cb = t / NR;
            if (t < NT3) {
                kd[m] = mma_k4<JT / 16>(sD + 16 * rb * LJ, LJ, sdS1 + 16 * cb * LJ, LJ, kd[m], lane);
                qp[m] = mma_k4<JT / 16>(sdO + 16 * rb * LJ, LJ, sS0 + 16 * cb * LJ, LJ, qp[m], lane);
                dw[m] = mma_k4<JT / 16>(sdD + 16 * rb * LJ, LJ, sS0 + 16 * cb * LJ, LJ, dw[m], lane);
            }
        }
        // dM = tril(dO D^T)   ([C][C], the tiles on or below the diagonal)
#pragma unroll
        for (int m = 0; m < TMW; ++m) {
            const int t = w + 4 * m, rb = t / NR, sb = t % NR;
            if (t < NTM && sb <= rb)
                dm[m] = mma_k4<JT / 16>(sdO + 16 * rb * LJ, LJ, sD + 16 * sb * LJ, LJ, dm[m], lane);
        }
        // dgamma = rowsum(dS1 * S0): two threads per key channel (half the tile's columns each, so
        // that all four waves share the work), 16-byte reads
        if (tid < 2 * DK) {
            const int off = (tid >> 1) * LJ + (tid & 1) * (JT / 2);
#pragma unroll
            for (int j = 0; j < JT / 2; j += 4) {
                const float4 x = *reinterpret_cast<const float4*>(sdS1 + off + j);
                const float4 y = *reinterpret_cast<const float4*>(sS0 + off + j);
                dgam += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
            }
        }
        lds_barrier();
    }
#pragma unroll
    for (int m = 0; m < T3W; ++m) {
        const int t = w + 4 * m, rb = t % NR, cb = t / NR;
        if (t < NT3)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t o = (16 * rb + 4 * (lane >> 4) + e) * DK + 16 * cb + (lane & 15);
                rec[R::dKd + o] = kd[m][e];
                rec[R::dQp + o] = qp[m][e];
                rec[R::dW + o] = -dw[m][e];
            }
    }
#pragma unroll
    for (int m = 0; m < TMW; ++m) {
        const int t = w + 4 * m, rb = t / NR, sb = t % NR;
        if (t < NTM)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * (lane >> 4) + e, s = 16 * sb + (lane & 15);
                rec[R::dM + r * C + s] = s <= r ? dm[m][e] : 0.f;
            }
    }
    dgam += __shfl_xor(dgam, 1);
    if (tid < 2 * DK && !(tid & 1)) rec[R::dgam + (tid >> 1)] = dgam;
}

// ------------------------------------------------------------------------------------------
// grad_state with split-bf16 operands (bfloat16 storage at d_k = d_v = 128, chunk 64).  Each fp32
// operand x is staged in LDS as hi = bf16(x) and lo = bf16(x - hi), so x = hi + lo to within 2^-18
// of |x|, and every product is three bf16 matrix-core steps (hi hi + hi lo + lo hi; the lo lo term is
// below 2^-18 of the product), with fp32 accumulation and fp32's exponent range.  A value tile of 32
// columns is one 16x16x32 step, where the fp32 16x16x4 form needs eight steps of twice the cost.
// dgamma is summed from the staged fp32 values themselves.
// ------------------------------------------------------------------------------------------
template <int DK, int DV, int C>
__global__ __launch_bounds__(kThreads) void grad_state_split_kernel(BwdArgs a, Map<C> mp) {
    using R = Rec<DK, DV, C>;
    static_assert(DK == 128 && DV == 128 && C == 64, "split-bf16 grad_state covers the d = 128, chunk 64 shape");
    constexpr int JT = 32, LH = JT + 8;  // value columns per tile; bf16 row stride (80 bytes)
    constexpr int NR = C / 16;
    // hi and lo of D, dD, dO ([C][LH]) and of S0, dS1 ([DK][LH])
    __shared__ __attribute__((aligned(16))) __bf16 sD[2][C * LH];
    __shared__ __attribute__((aligned(16))) __bf16 sdD[2][C * LH];
    __shared__ __attribute__((aligned(16))) __bf16 sdO[2][C * LH];
    __shared__ __attribute__((aligned(16))) __bf16 sS0[2][DK * LH];
    __shared__ __attribute__((aligned(16))) __bf16 sdS1[2][DK * LH];
    const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
    const int64_t slot = blockIdx.x;
    int64_t n, c, t0;
    int L;
    if (!mp.locate(slot, n, c, t0, L)) return;
    const int H = a.H;
    float* rec = a.ws + (slot * H + h) * R::kFloats;
    // dO rows of this chunk through a descriptor that ends at its last token (rows past it read 0)
    const __amdgpu_buffer_rsrc_t dors =
        make_rsrc(a.dO + (t0 * H + h) * (int64_t)DV, (uint32_t)((((int64_t)L - 1) * H * DV + DV) * 4));
    floatx4 kd[8], qp[8], dw[8], dm[4];
#pragma unroll
    for (int m = 0; m < 8; ++m) kd[m] = qp[m] = dw[m] = zero4();
#pragma unroll
    for (int m = 0; m < 4; ++m) dm[m] = zero4();
    float dgam[4] = {0.f, 0.f, 0.f, 0.f};  // rows (tid >> 3) + 32 m, summed over this thread's columns
    // value tile j0 .. j0 + 31, one tile ahead: thread tid holds rows tid / 8 + 32 m, columns 4 (tid % 8) .. +3
    Stage<C, JT> pD, pdD, pdO;
    Stage<DK, JT> pS, pdS;
    auto fetch = [&](int j0) {
        pD.load(rec + R::D + j0, DV);
        pdD.load(rec + R::dD + j0, DV);
        pS.load(rec + R::S0 + j0, DV);
        pdS.load(rec + R::dS1 + j0, DV);
#pragma unroll
        for (int m = 0; m < Stage<C, JT>::kPer; ++m) {
            const int e = tid + m * kThreads, row = e / (JT / 4), c4 = e % (JT / 4);
            pdO.r[m] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      dors, (row * H * DV + j0 + 4 * c4) * 4, 0, 0));
        }
    };
    auto store_split = [&](const float4* r, int kper, __bf16* hi, __bf16* lo) {
        for (int m = 0; m < kper; ++m) {
            const int e = tid + m * kThreads, row = e / (JT / 4), c4 = e % (JT / 4);
            bf16x4 bh, bl;
            split4(r[m], bh, bl);
            *reinterpret_cast<bf16x4*>(hi + row * LH + 4 * c4) = bh;
            *reinterpret_cast<bf16x4*>(lo + row * LH + 4 * c4) = bl;
        }
    };
    auto frag = [&](const __bf16* base, int rb) {
        return *reinterpret_cast<const bf16x8*>(base + (16 * rb + lr) * LH + 8 * lg);
    };
    fetch(0);
    for (int j0 = 0; j0 < DV; j0 += JT) {
#pragma unroll
        for (int m = 0; m < Stage<DK, JT>::kPer; ++m) {  // dgamma from the fp32 values
            const float4 x = pS.r[m], y = pdS.r[m];
            dgam[m] += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
        }
        store_split(pD.r, Stage<C, JT>::kPer, sD[0], sD[1]);
        store_split(pdD.r, Stage<C, JT>::kPer, sdD[0], sdD[1]);
        store_split(pdO.r, Stage<C, JT>::kPer, sdO[0], sdO[1]);
        store_split(pS.r, Stage<DK, JT>::kPer, sS0[0], sS0[1]);
        store_split(pdS.r, Stage<DK, JT>::kPer, sdS1[0], sdS1[1]);
        fetch(j0 + JT < DV ? j0 + JT : j0);
        lds_barrier();
        // token block w: D, dO, dD rows (A operands of the three [C][DK] products, and D the B
        // operand of dM)
        const bf16x8 aDh = frag(sD[0], w), aDl = frag(sD[1], w);
        const bf16x8 aOh = frag(sdO[0], w), aOl = frag(sdO[1], w);
        const bf16x8 adh = frag(sdD[0], w), adl = frag(sdD[1], w);
        // dK' = D dS1^T, dQ+ = dO S0^T, dW = -dD S0^T: tile (w, m) for key channel block m
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const bf16x8 sh = frag(sS0[0], m), sl = frag(sS0[1], m);
            const bf16x8 gh = frag(sdS1[0], m), gl = frag(sdS1[1], m);
            kd[m] = mfma_split(aDh, aDl, gh, gl, kd[m]);
            qp[m] = mfma_split(aOh, aOl, sh, sl, qp[m]);
            dw[m] = mfma_split(adh, adl, sh, sl, dw[m]);
        }
        // dM = tril(dO D^T): tile (m, w) for token blocks m >= w
#pragma unroll
        for (int m = 0; m < NR; ++m)
            if (w <= m) dm[m] = mfma_split(frag(sdO[0], m), frag(sdO[1], m), aDh, aDl, dm[m]);
        lds_barrier();
    }
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t o = (16 * w + 4 * lg + e) * DK + 16 * m + lr;
            rec[R::dKd + o] = kd[m][e];
            rec[R::dQp + o] = qp[m][e];
            rec[R::dW + o] = -dw[m][e];
        }
#pragma unroll
    for (int m = 0; m < NR; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * m + 4 * lg + e, s2 = 16 * w + lr;
            rec[R::dM + r * C + s2] = (w <= m && s2 <= r) ? dm[m][e] : 0.f;
        }
    // each row's sum over its 8 threads (columns 4 (tid % 8) .. +3 of every tile)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        float x = dgam[m];
        x += __shfl_xor(x, 1);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 4);
        if ((tid & 7) == 0) rec[R::dgam + (tid >> 3) + 32 * m] = x;
    }
}

// ------------------------------------------------------------------------------------------
// grad_chunk: one workgroup per (chunk slot, head); dq, dk, dv, dg, dbeta.  Under 80 KB of LDS
// (two workgroups per CU): the key channels are visited in blocks of 16, and each block's
// cumulative log-decay is recomputed there by a prefix sum over the rows (wave_prefix64).
// ------------------------------------------------------------------------------------------
template <int DK, int DV, int C>
struct ChunkLds {
    static constexpr int LC = C + 1, LB = 17;
    // value columns per staged tile; rows padded to a multiple of 4 floats for 16-byte operand reads
    static constexpr int JT = DV < 32 ? DV : 32, LJ = JT + 4;
    static constexpr int kStage0 = 3 * LJ > 6 * LB ? 3 * LJ : 6 * LB;
    static constexpr int kStage = kStage0 > LC ? kStage0 : LC;  // floats per row of the staging area
    static constexpr size_t kFloats = 3 * (size_t)C * LC      // T, dM, dT -> dP
                                      + (size_t)C * kStage    // staged tiles (see the kernel)
                                      + 6 * (size_t)C         // beta, dbeta per wave, dg (one gate per head)
                                      + 4 * 16;               // per-wave column sums of a channel block
    static constexpr size_t kBytes = kFloats * sizeof(float);
};

template <int DK, int DV, int C, typename TI>
__global__ __launch_bounds__(kThreads, 2) void grad_chunk_kernel(BwdArgs a, Map<C> mp) {
    using R = Rec<DK, DV, C>;
    using Lds = ChunkLds<DK, DV, C>;
    constexpr int LC = Lds::LC, LB = Lds::LB, NR = C / 16, JT = Lds::JT, LJ = Lds::LJ;
    constexpr int RPT = C / 16;  // rows per thread in the channel-block sweeps
    extern __shared__ float lds[];
    float* sT = lds;                    // [C][LC]
    float* sdM = sT + C * LC;           // [C][LC]
    float* sA = sdM + C * LC;           // [C][LC]  dT, then dP
    float* sX = sA + C * LC;            // [C][kStage] staging area
    float* sB = sX + C * Lds::kStage;   // [C]
    // dbeta and the column sums are accumulated per wave and added in wave order at the end, so
    // the result does not depend on the order the waves run in (no atomics)
    float* sdbw = sB + C;               // [4][C] dbeta partial sums of each wave
    float* sdgh = sdbw + 4 * C;         // [C]
    float* sColw = sdgh + C;            // [4][16] column sums of dK' * K' in the current channel block
    // value tiles: dD, V, beta V ([C][LJ] each); Z ([C][LC]); channel blocks ([C][LB] each): K, Q,
    // dW (then K scaled for the row role), G, beta K+ (first pass) or K scaled for the column role
    // (second pass), g (then Q scaled for the column role, then dG)
    float* tdD = sX;
    float* tV = tdD + C * LJ;
    float* tBV = tV + C * LJ;
    float* sZ = sX;
    float* tK = sX;
    float* tQ = tK + C * LB;
    float* tW = tQ + C * LB;
    float* tG = tW + C * LB;
    float* tKp = tG + C * LB;
    float* tdG = tKp + C * LB;
    float* tKc = tW;   // second pass: K_s exp(G_m - G_s), m the last row of s's block
    float* tKr = tKp;  // second pass: K_r exp(G_r - G_m), m the last row of the block before r's
    float* tQr = tdG;  // second pass: Q_r exp(G_r - G_m), likewise

    const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t slot = blockIdx.x;
    int64_t n, c, t0;
    int L;
    if (!mp.locate(slot, n, c, t0, L)) return;
    const int H = a.H;
    const TI* k = static_cast<const TI*>(a.k);
    const TI* q = static_cast<const TI*>(a.q);
    const TI* v = static_cast<const TI*>(a.v);
    const TI* beta = static_cast<const TI*>(a.beta);
    const float* rec = a.ws + (slot * H + h) * R::kFloats;
    // outputs through descriptors that end at the chunk's last token: stores of rows past it are
    // dropped, so no store needs a branch (a branch hides the count of outstanding memory
    // operations from the compiler, and the next prefetch wait then drains every store too)
    const int64_t tok0 = t0 * H + h;
    const __amdgpu_buffer_rsrc_t gvrs = make_rsrc(a.gv + tok0 * DV, (uint32_t)((((int64_t)L - 1) * H * DV + DV) * 4));
    const __amdgpu_buffer_rsrc_t gqrs = make_rsrc(a.gq + tok0 * DK, (uint32_t)((((int64_t)L - 1) * H * DK + DK) * 4));
    const __amdgpu_buffer_rsrc_t gkrs = make_rsrc(a.gk + tok0 * DK, (uint32_t)((((int64_t)L - 1) * H * DK + DK) * 4));
    const __amdgpu_buffer_rsrc_t ggrs = make_rsrc(a.gg + tok0 * DK, (uint32_t)((((int64_t)L - 1) * H * DK + DK) * 4));

    // value tiles (dD, v), loaded into registers one tile ahead (beta comes from sB)
    constexpr int VPT = (C * JT + kThreads - 1) / kThreads;
    struct ValueRegs {
        float dd[VPT], v[VPT];
    } vr;
    auto fetch_value = [&](int j0) {
#pragma unroll
        for (int m = 0; m < VPT; ++m) {
            const int e = tid + kThreads * m, r = e / JT, j = e % JT;
            const bool full = VPT * kThreads == C * JT || e < C * JT, in = full && r < L;
            const int rr = in ? r : L - 1;
            const float dx = rec[R::dD + (full ? r : 0) * DV + j0 + j];
            const float vx = ld_in<TI>(v, ((t0 + rr) * H + h) * (int64_t)DV + j0 + j);
            vr.dd[m] = full ? dx : 0.f;
            vr.v[m] = in ? vx : 0.f;
        }
    };
    fetch_value(0);
    {  // T and dM: every load requested before the stores (a static trip count lets them batch)
        constexpr int TPT = (C * C + kThreads - 1) / kThreads;
        float tv[TPT], mv[TPT];
#pragma unroll
        for (int m = 0; m < TPT; ++m) {
            const int e = tid + kThreads * m, ec = e < C * C ? e : C * C - 1;
            tv[m] = rec[R::T + ec];
            mv[m] = rec[R::dM + ec];
        }
#pragma unroll
        for (int m = 0; m < TPT; ++m) {
            const int e = tid + kThreads * m;
            if (TPT * kThreads == C * C || e < C * C) {
                sT[(e / C) * LC + e % C] = tv[m];
                sdM[(e / C) * LC + e % C] = mv[m];
            }
        }
    }
    if (tid < C) {
        sB[tid] = tid < L ? ld_in<TI>(beta, (t0 + tid) * H + h) : 0.f;
#pragma unroll
        for (int wv = 0; wv < 4; ++wv) sdbw[wv * C + tid] = 0.f;
        sdgh[tid] = 0.f;
    }

    // One 16-channel block of k, q, dW and g, loaded into registers one block ahead, then written to
    // LDS (k -> tK, q -> tQ, dW -> tW, g -> tdG); element i of a thread is row (tid >> 4) + 16 i,
    // channel tid & 15.  The second pass also fetches dQ+, dK' and dgamma in the matrix-core layout
    // (wave w < NR: rows 16 w + 4 (lane >> 4) + e, channel lane & 15).
    constexpr int NCB = DK / 16;
    const int cc = tid & 15, r0 = tid >> 4, lr = lane & 15, lg = lane >> 4;
    struct BlockRegs {
        float k[RPT], q[RPT], dw[RPT], g[RPT], dqp[4], dkd[4], dgam;
    };
    auto fetch_block = [&](int cb, bool second, BlockRegs& br) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = r0 + 16 * i, ch = 16 * cb + cc;
            const bool in = r < L;
            const int rr = in ? r : L - 1;  // see the note on unconditional loads
            const int64_t idx = ((t0 + rr) * H + h) * (int64_t)DK + ch;
            const float kx = ld_in<TI>(k, idx), gx = gate_at(a.g, a.gate_head, t0 + rr, H, h, DK, ch);
            br.k[i] = in ? kx : 0.f;
            br.dw[i] = rec[R::dW + r * DK + ch];
            br.g[i] = in ? gx : 0.f;
            if (second) {
                const float qx = ld_in<TI>(q, idx);
                br.q[i] = in ? qx : 0.f;
            }
        }
        if (second && w < NR) {
            const int ch = 16 * cb + lr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * w + 4 * lg + e;
                br.dqp[e] = rec[R::dQp + r * DK + ch];
                br.dkd[e] = rec[R::dKd + r * DK + ch];
            }
            br.dgam = rec[R::dgam + ch];
        }
    };
    auto put_block = [&](const BlockRegs& br, bool second) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = r0 + 16 * i;
            tK[r * LB + cc] = br.k[i];
            tW[r * LB + cc] = br.dw[i];
            tdG[r * LB + cc] = br.g[i];
            if (second) tQ[r * LB + cc] = br.q[i];
        }
        if (second && tid < 64) sColw[tid] = 0.f;
    };

    // ---- dT = dD (beta V)^T + dW (beta K+)^T, strictly lower part (wave w owns tiles w, w+4, ...),
    //      and with the value tiles staged: dV = beta (T^T dD), dbeta += rowsum(V * T^T dD)
    constexpr int NT = NR * NR, TPW = (NT + 3) / 4;
    floatx4 dT[TPW];
#pragma unroll
    for (int m = 0; m < TPW; ++m) dT[m] = zero4();
    lds_barrier();  // sB (read by the value-tile staging) is complete
    for (int j0 = 0; j0 < DV; j0 += JT) {
        // this tile from registers; the next one is loaded while this one is used
#pragma unroll
        for (int m = 0; m < VPT; ++m) {
            const int e = tid + kThreads * m, r = e / JT, j = e % JT;
            if (VPT * kThreads == C * JT || e < C * JT) {
                tdD[r * LJ + j] = vr.dd[m];
                tV[r * LJ + j] = vr.v[m];
                tBV[r * LJ + j] = sB[r] * vr.v[m];  // sB is 0 past the chunk end
            }
        }
        fetch_value(j0 + JT < DV ? j0 + JT : j0);
        lds_barrier();
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int t = w + 4 * m, rb = t / NR, sb = t % NR;
            if (t < NT && sb <= rb)  // both operands contiguous along the value columns
                dT[m] = mma_k4<JT / 16>(tdD + 16 * rb * LJ, LJ, tBV + 16 * sb * LJ, LJ, dT[m], lane);
        }
        for_each_wave<NR * (JT / 16)>(w, [&](int t) {
            const int rb = t % NR, jb = t / NR;
            const floatx4 x = mma<C / 4>(sT + 16 * rb, 1, LC, tdD + 16 * jb, LJ, 1, zero4(), lane);
            float part[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * (lane >> 4) + e, j = 16 * jb + (lane & 15);
                part[e] = tV[r * LJ + j] * x[e];
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sB[r] * x[e]), gvrs, (r * H * DV + j0 + j) * 4, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = sum16(part[e]);
                if ((lane & 15) == 0) sdbw[w * C + 16 * rb + 4 * (lane >> 4) + e] += p;
            }
        });
        lds_barrier();
    }
    BlockRegs br;
    fetch_block(0, false, br);
    for (int cb = 0; cb < NCB; ++cb) {
        put_block(br, false);
        fetch_block(cb + 1 < NCB ? cb + 1 : cb, false, br);
        lds_barrier();
        // G = tril(ones) g by columns (wave w: columns w, w + 4, ...; one lane per row), then
        // beta K+ = beta k exp(G) into tKp
        for_each_wave<16>(w, [&](int j) {
            const float G = wave_prefix64(lane < C ? tdG[lane * LB + j] : 0.f);
            if (lane < C) tKp[lane * LB + j] = sB[lane] * tK[lane * LB + j] * fast_exp(G);
        });
        lds_barrier();
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int t = w + 4 * m, rb = t / NR, sb = t % NR;
            if (t < NT && sb <= rb) dT[m] = mma<4>(tW + 16 * rb * LB, LB, 1, tKp + 16 * sb * LB, 1, LB, dT[m], lane);
        }
        lds_barrier();
    }
    fetch_block(0, true, br);  // the second pass's first block, in flight during dA
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
        const int t = w + 4 * m, rb = t / NR, sb = t % NR;
        if (t < NT)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * (lane >> 4) + e, s = 16 * sb + (lane & 15);
                sA[r * LC + s] = s < r ? dT[m][e] : 0.f;
            }
    }
    lds_barrier();
    // ---- dA = -T^T dT T^T (strictly lower): Z = T^T dT, then dA = -Z T^T; dP = Diag(beta) dA,
    //      dbeta += rowsum(dA * P) (P loaded first, in flight during the two products)
    float pv[TPW][4];
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
        const int t = w + 4 * m, rb = t / NR, sb = t % NR;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            pv[m][e] = t < NT ? rec[R::P + (16 * rb + 4 * (lane >> 4) + e) * C + 16 * sb + (lane & 15)] : 0.f;
    }
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
        const int t = w + 4 * m, rb = t / NR, sb = t % NR;
        if (t < NT) {
            const floatx4 z = mma<C / 4>(sT + 16 * rb, 1, LC, sA + 16 * sb, LC, 1, zero4(), lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) sZ[(16 * rb + 4 * (lane >> 4) + e) * LC + 16 * sb + (lane & 15)] = z[e];
        }
    }
    lds_barrier();
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
        const int t = w + 4 * m, rb = t / NR, sb = t % NR;
        if (t < NT) dT[m] = mma<C / 4>(sZ + 16 * rb * LC, LC, 1, sT + 16 * sb * LC, 1, LC, zero4(), lane);
    }
    lds_barrier();  // every read of sA (dT) and sZ is done
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
        const int t = w + 4 * m, rb = t / NR, sb = t % NR;
        if (t < NT) {
            float part[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * (lane >> 4) + e, s = 16 * sb + (lane & 15);
                const float da = s < r ? -dT[m][e] : 0.f;
                part[e] = da * pv[m][e];
                sA[r * LC + s] = sB[r] * da;  // dP
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = sum16(part[e]);
                if ((lane & 15) == 0) sdbw[w * C + 16 * rb + 4 * (lane >> 4) + e] += p;
            }
        }
    }
    lds_barrier();

    // ---- channel blocks of 16, wave w < NR owning row block w: G, dK+ = beta T^T dW, the gradients
    //      through the pairwise products P and M, dq, dk, dG, and dg as the suffix sums of dG.
    //      Pairs (r, s) in different 16-row blocks go through the matrix cores: with m a block's last
    //      row, exp(G_r - G_s) = exp(G_r - G_m) exp(G_m - G_s) where both exponents are <= 0
    //      (s <= m < r), so every scaled operand is bounded by the unscaled one.  Pairs inside a block
    //      take the exponential of their own difference.
    for (int cb = 0; cb < NCB; ++cb) {
        const int ch = 16 * cb + lr;
        float rdq[4], rdk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            rdq[e] = br.dqp[e];
            rdk[e] = br.dkd[e];
        }
        const float dgam = br.dgam;
        put_block(br, true);
        fetch_block(cb + 1 < NCB ? cb + 1 : cb, true, br);
        lds_barrier();
        // G = tril(ones) g into tG by columns (wave w: columns w, w + 4, ...; one lane per row)
        for_each_wave<16>(w, [&](int j) {
            const float G = wave_prefix64(lane < C ? tdG[lane * LB + j] : 0.f);
            if (lane < C) tG[lane * LB + j] = G;
        });
        lds_barrier();
        float Gr[4] = {0.f, 0.f, 0.f, 0.f}, xk[4] = {0.f, 0.f, 0.f, 0.f};
        if (w < NR) {
            const floatx4 x = mma<C / 4>(sT + 16 * w, 1, LC, tW, LB, 1, zero4(), lane);
            float part[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * w + 4 * lg + e;
                Gr[e] = tG[r * LB + lr];
                xk[e] = sB[r] * x[e];
                part[e] = tK[r * LB + lr] * fast_exp(Gr[e]) * x[e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = sum16(part[e]);
                if (lr == 0) sdbw[w * C + 16 * w + 4 * lg + e] += p;
            }
        }
        lds_barrier();  // G complete; dW and g no longer needed
        // block w's scaled tiles: against its last row (K) and against the row before it (Q, K; row -1
        // has G = 0)
        float gend = 0.f, gprev = 0.f;
        if (w < NR) {
            gend = tG[(16 * w + 15) * LB + lr];
            gprev = w > 0 ? tG[(16 * w - 1) * LB + lr] : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * w + 4 * lg + e;
                const float kr = tK[r * LB + lr], qr = tQ[r * LB + lr];
                tKc[r * LB + lr] = kr * fast_exp(gend - Gr[e]);
                const float f = fast_exp(Gr[e] - gprev);
                tQr[r * LB + lr] = qr * f;
                tKr[r * LB + lr] = kr * f;
            }
        }
        lds_barrier();
        float dGr[4] = {0.f, 0.f, 0.f, 0.f}, glast = 0.f;
        if (w < NR) {
            float rq[4] = {0.f, 0.f, 0.f, 0.f}, rk[4] = {0.f, 0.f, 0.f, 0.f}, ck[4] = {0.f, 0.f, 0.f, 0.f};
            // row role, blocks j < w:  sum_s dM[r][s] K_s exp(G_r - G_s), and the same with dP
            for (int j = 0; j < w; ++j) {
                const floatx4 xm = mma<4>(sdM + 16 * w * LC + 16 * j, LC, 1, tKc + 16 * j * LB, LB, 1, zero4(), lane);
                const floatx4 xp = mma<4>(sA + 16 * w * LC + 16 * j, LC, 1, tKc + 16 * j * LB, LB, 1, zero4(), lane);
                const float gm = tG[(16 * j + 15) * LB + lr];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float f = fast_exp(Gr[e] - gm);
                    rq[e] += f * xm[e];
                    rk[e] += f * xp[e];
                }
            }
            // column role, blocks i > w:  sum_r exp(G_r - G_s) (dM[r][s] Q_r + dP[r][s] K_r)
            for (int i = w + 1; i < NR; ++i) {
                floatx4 y = mma<4>(sdM + 16 * i * LC + 16 * w, 1, LC, tQr + 16 * i * LB, LB, 1, zero4(), lane);
                y = mma<4>(sA + 16 * i * LC + 16 * w, 1, LC, tKr + 16 * i * LB, LB, 1, y, lane);
                const float gm = tG[(16 * i - 1) * LB + lr];
#pragma unroll
                for (int e = 0; e < 4; ++e) ck[e] += fast_exp(gm - Gr[e]) * y[e];
            }
            // pairs inside block w.  On the matrix cores with the decay split at the block's last row
            // (row role) or at the row before it (column role): the products are bounded by the scaled
            // tiles, and the other factor by exp(D), D the block's 16-token decay.  If D > 64 for some
            // channel of the wave the pairs take their own exponentials instead (the wrong side of the
            // diagonal masked with a -inf exponent).
            if (!__any(gprev - gend > 64.f)) {
                const floatx4 xm = mma<4>(sdM + 16 * w * LC + 16 * w, LC, 1, tKc + 16 * w * LB, LB, 1, zero4(), lane);
                const floatx4 xp = mma<4>(sA + 16 * w * LC + 16 * w, LC, 1, tKc + 16 * w * LB, LB, 1, zero4(), lane);
                floatx4 y = mma<4>(sdM + 16 * w * LC + 16 * w, 1, LC, tQr + 16 * w * LB, LB, 1, zero4(), lane);
                y = mma<4>(sA + 16 * w * LC + 16 * w, 1, LC, tKr + 16 * w * LB, LB, 1, y, lane);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float fr = fast_exp(Gr[e] - gend), fc = fast_exp(gprev - Gr[e]);
                    rq[e] += fr * xm[e];
                    rk[e] += fr * xp[e];
                    ck[e] += fc * y[e];
                }
            } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * w + 4 * lg + e;
#pragma unroll 1
                for (int i = 0; i < 16; ++i) {
                    const int s2 = 16 * w + i;
                    const float gs = tG[s2 * LB + lr];
                    // row role: s2 <= r
                    const float er = fast_exp(s2 <= r ? Gr[e] - gs : -INFINITY) * tK[s2 * LB + lr];
                    rq[e] += sdM[r * LC + s2] * er;
                    rk[e] += sA[r * LC + s2] * er;  // dP is zero on the diagonal
                    // column role: s2 > r, and the diagonal term dM[r][r] q_r
                    const float ec = s2 > r ? fast_exp(gs - Gr[e]) : (s2 == r ? 1.f : 0.f);
                    ck[e] += ec * (sdM[s2 * LC + r] * tQ[s2 * LB + lr] + (s2 > r ? sA[s2 * LC + r] : 0.f) *
                                                                             tK[s2 * LB + lr]);
                }
            }
            }
            glast = tG[(C - 1) * LB + lr];
            float colsum = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // rows past the chunk end have zero k and q, so their dG and column-sum terms are
                // zero; their dq and dk stores fall past the descriptors' ends and are dropped
                const int r = 16 * w + 4 * lg + e;
                const float kr = tK[r * LB + lr], qr = tQ[r * LB + lr];
                const float eg = fast_exp(Gr[e]), ed = fast_exp(glast - Gr[e]);
                const float dq = rdq[e] * eg + rq[e];
                const float dk = xk[e] * eg + rdk[e] * ed + rk[e] + ck[e];
                dGr[e] = xk[e] * kr * eg + rdq[e] * qr * eg - rdk[e] * kr * ed + qr * rq[e] + kr * rk[e] -
                         kr * ck[e];
                colsum += rdk[e] * kr * ed;
                const int go = (r * H * DK + ch) * 4;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dq), gqrs, go, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dk), gkrs, go, 0, 0);
            }
            colsum += __shfl_xor(colsum, 16);
            colsum += __shfl_xor(colsum, 32);
            if (lg == 0) sColw[16 * w + lr] = colsum;
        }
        lds_barrier();  // every read of the scaled tiles is done; the column sums are complete
        if (w < NR)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * w + 4 * lg + e;
                float col = 0.f;
#pragma unroll
                for (int wv = 0; wv < NR; ++wv) col += sColw[16 * wv + lr];
                tdG[r * LB + lr] = dGr[e] + (r == L - 1 ? col + dgam * fast_exp(glast) : 0.f);
            }
        lds_barrier();
        // dg = suffix sums over the chunk's rows, by columns: wave w scans columns w, w + 4, ..., lane
        // l on row C - 1 - l, so that its prefix sum is that row's suffix sum (in place)
        for_each_wave<16>(w, [&](int j) {
            const int row = lane < C ? C - 1 - lane : 0;
            const float sfx = wave_prefix64(lane < C ? tdG[row * LB + j] : 0.f);
            if (lane < C) tdG[row * LB + j] = sfx;
        });
        lds_barrier();
        if (w < NR) {
            float hsum[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = 16 * w + 4 * lg + e;
                const float dg = tdG[rr * LB + lr];
                if (!a.gate_head)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dg), ggrs, (rr * H * DK + ch) * 4, 0, 0);
                hsum[e] = sum16(dg);
            }
            if (a.gate_head && lr == 0)
#pragma unroll
                for (int e = 0; e < 4; ++e) sdgh[16 * w + 4 * lg + e] += hsum[e];
        }
        lds_barrier();  // the tiles are rewritten by the next block
    }
    if (tid < L) {
        a.gbeta[(t0 + tid) * H + h] = sdbw[tid] + sdbw[C + tid] + sdbw[2 * C + tid] + sdbw[3 * C + tid];
        if (a.gate_head) a.gg[(t0 + tid) * H + h] = sdgh[tid];
    }
}

// ------------------------------------------------------------------------------------------
// launch
// ------------------------------------------------------------------------------------------
template <typename K>
hipError_t set_lds(K kernel, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

int64_t num_slots(int64_t N, int64_t T_total, int C) { return T_total / C + N + 1; }

// Workspace plan.  One pass keeps a record for every chunk (its bytes grow with T).  When that
// exceeds the cap, the chunks are taken in windows of wlen chunks of every sequence: a forward
// sweep over the windows keeps only the states at window boundaries (checkpoints), then a
// reverse sweep recomputes each window's records from its checkpoint and runs the reverse
// chain, carrying the state gradient from one window to the one before it.  That costs a second
// evaluation of the factors and the forward chain; the workspace is then the records of one
// window plus the checkpoints and the carried gradient.
struct BwdPlan {
    bool windowed;
    int64_t wlen, W;
    size_t records, ckpt, carry;  // bytes
    size_t total() const { return records + ckpt + carry; }
};

size_t workspace_cap() {
    // default 20 GiB; KDA_BWD_WORKSPACE_CAP (bytes) overrides it, e.g. to take the windowed path
    // at small sizes
    const char* v = std::getenv("KDA_BWD_WORKSPACE_CAP");
    if (v && v[0]) {
        const unsigned long long x = std::strtoull(v, nullptr, 10);
        if (x > 0) return (size_t)x;
    }
    return size_t(20) << 30;
}

BwdPlan plan_bwd(int64_t N, int64_t T_total, int H, int DK, int DV, int C, size_t rec_floats) {
    BwdPlan p{};
    const size_t rec = rec_floats * sizeof(float);
    const size_t full = (size_t)num_slots(N, T_total, C) * (size_t)H * rec;
    const size_t cap = workspace_cap();
    if (full <= cap || N * (int64_t)H == 0 || T_total == 0) {
        p.windowed = false;
        p.records = full;
        return p;
    }
    const size_t state = (size_t)N * H * DK * DV * sizeof(float);
    const size_t per_chunk = (size_t)N * H * rec;  // one window chunk of every sequence
    const int64_t nck_max = (T_total + C - 1) / C;
    int64_t wlen = (int64_t)(cap / per_chunk);
    if (wlen < 1) wlen = 1;
    int64_t W = (nck_max + wlen - 1) / wlen;
    // room for the checkpoints (one per window boundary) and the carried gradient
    const size_t extra = (size_t)W * state;
    if (cap > extra + per_chunk) {
        wlen = (int64_t)((cap - extra) / per_chunk);
        W = (nck_max + wlen - 1) / wlen;
    }
    p.windowed = true;
    p.wlen = wlen;
    p.W = W;
    p.records = (size_t)wlen * per_chunk;
    p.ckpt = (size_t)(W - 1) * state;
    p.carry = state;
    return p;
}

template <int DK, int DV, int C, typename TI>
hipError_t launch_typed(const BwdArgs& a, hipStream_t s) {
    constexpr bool kSplit = SplitShape<DK, DV, C, TI>::value;
    const bool timed = timing_on();
    hipError_t e;
    constexpr size_t f_lds = FactorsLds<DK, DV, C>::kBytes, c_lds = ChunkLds<DK, DV, C>::kBytes;
    if ((e = set_lds(factors_kernel<DK, DV, C, TI>, f_lds)) != hipSuccess) return e;
    if ((e = set_lds(grad_chunk_kernel<DK, DV, C, TI>, c_lds)) != hipSuccess) return e;
    const dim3 chains((unsigned)(a.N * a.H * (DV / kBV)));
    // the five kernels (or the first two) over the chunks that `mp` selects
    auto run = [&](const BwdArgs& x, const Map<C>& mp, int64_t slots, bool forward_only) -> hipError_t {
        const dim3 per_chunk((unsigned)slots, (unsigned)x.H);
        if (timed) timed_begin(kKernelBwdFactors, s);
        hipLaunchKernelGGL((factors_kernel<DK, DV, C, TI>), per_chunk, dim3(kThreads), f_lds, s, x, mp);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (timed) timed_end(s);
        if (timed) timed_begin(kKernelBwdFwdChain, s);
        if constexpr (kSplit)
            hipLaunchKernelGGL((fwd_chain_split_kernel<DK, DV, C>), chains, dim3(kThreads), 0, s, x, mp);
        else
            hipLaunchKernelGGL((fwd_chain_kernel<DK, DV, C>), chains, dim3(kThreads), 0, s, x, mp);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (timed) timed_end(s);
        if (forward_only) return hipSuccess;
        if (timed) timed_begin(kKernelBwdRevChain, s);
        if constexpr (kSplit)
            hipLaunchKernelGGL((rev_chain_split_kernel<DK, DV, C>), chains, dim3(kThreads), 0, s, x, mp);
        else
            hipLaunchKernelGGL((rev_chain_kernel<DK, DV, C>), chains, dim3(kThreads), 0, s, x, mp);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (timed) timed_end(s);
        if (timed) timed_begin(kKernelBwdGradState, s);
        if constexpr (kSplit)
            hipLaunchKernelGGL((grad_state_split_kernel<DK, DV, C>), per_chunk, dim3(kThreads), 0, s, x, mp);
        else
            hipLaunchKernelGGL((grad_state_kernel<DK, DV, C>), per_chunk, dim3(kThreads), 0, s, x, mp);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (timed) timed_end(s);
        if (timed) timed_begin(kKernelBwdGradChunk, s);
        hipLaunchKernelGGL((grad_chunk_kernel<DK, DV, C, TI>), per_chunk, dim3(kThreads), c_lds, s, x, mp);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (timed) timed_end(s);
        return hipSuccess;
    };
    const BwdPlan p = plan_bwd(a.N, a.T_total, a.H, DK, DV, C, Rec<DK, DV, C>::kFloats);
    if (!p.windowed) {
        const Map<C> mp{a.cu, a.N, 0, 0};
        if (a.T_total > 0) return run(a, mp, num_slots(a.N, a.T_total, C), false);
        // no tokens: only the reverse chain, which passes dL/dS_T through to dL/dS_0
        if (timed) timed_begin(kKernelBwdRevChain, s);
        hipLaunchKernelGGL((rev_chain_kernel<DK, DV, C>), chains, dim3(kThreads), 0, s, a, mp);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (timed) timed_end(s);
        return hipSuccess;
    }
    const int64_t state = a.N * a.H * (int64_t)DK * DV;  // floats
    float* ckpt = a.ws + p.records / sizeof(float);       // state entering window j (j >= 1) at j - 1
    float* carry = ckpt + p.ckpt / sizeof(float);
    auto ckpt_of = [&](int64_t j) -> const float* { return j == 0 ? a.s0 : ckpt + (j - 1) * state; };
    const int64_t slots = a.N * p.wlen;
    for (int64_t j = 0; j + 1 < p.W; ++j) {  // forward sweep: the checkpoints
        BwdArgs x = a;
        x.s0 = ckpt_of(j);
        x.s_fin = ckpt + j * state;
        if ((e = run(x, Map<C>{a.cu, a.N, j * p.wlen, p.wlen}, slots, true)) != hipSuccess) return e;
    }
    for (int64_t j = p.W - 1; j >= 0; --j) {  // reverse sweep
        BwdArgs x = a;
        x.s0 = ckpt_of(j);
        x.s_fin = nullptr;
        x.dsT = j == p.W - 1 ? a.dsT : carry;  // read at the start of each chain, then
        x.gs0 = j == 0 ? a.gs0 : carry;        // written at its end by the same workgroup
        if ((e = run(x, Map<C>{a.cu, a.N, j * p.wlen, p.wlen}, slots, false)) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DK, int DV, int C>
hipError_t launch_shape(const BwdArgs& a, hipStream_t s) {
    return a.bf16 ? launch_typed<DK, DV, C, uint16_t>(a, s) : launch_typed<DK, DV, C, float>(a, s);
}

}  // namespace

bool chunk_bwd_supported(int dk, int dv, int chunk) {
    const bool okd = dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
    return okd && (chunk == 16 || chunk == 32 || chunk == 64);
}

size_t chunk_bwd_workspace(int64_t N, int64_t T_total, int H, int dk, int dv, int chunk) {
    int64_t per = 0;
#define KDA_BWD(DK_, DV_, C_) \
    if (dk == DK_ && dv == DV_ && chunk == C_) per = Rec<DK_, DV_, C_>::kFloats;
#define KDA_BWD_C(DK_, DV_) KDA_BWD(DK_, DV_, 16) KDA_BWD(DK_, DV_, 32) KDA_BWD(DK_, DV_, 64)
#define KDA_BWD_DV(DK_) KDA_BWD_C(DK_, DK_)
    KDA_BWD_DV(16) KDA_BWD_DV(32) KDA_BWD_DV(64) KDA_BWD_DV(128)
#undef KDA_BWD
    return plan_bwd(N, T_total, H, dk, dv, chunk, (size_t)per).total();
}

hipError_t launch_chunk_bwd(const BwdArgs& a, hipStream_t s) {
    if (a.N * a.H == 0) return hipSuccess;
#define KDA_BWD(DK_, DV_, C_) \
    if (a.dk == DK_ && a.dv == DV_ && a.chunk == C_) return launch_shape<DK_, DV_, C_>(a, s);
#define KDA_BWD_C(DK_, DV_) KDA_BWD(DK_, DV_, 16) KDA_BWD(DK_, DV_, 32) KDA_BWD(DK_, DV_, 64)
#define KDA_BWD_DV(DK_) KDA_BWD_C(DK_, DK_)
    KDA_BWD_DV(16) KDA_BWD_DV(32) KDA_BWD_DV(64) KDA_BWD_DV(128)
#undef KDA_BWD_DV
#undef KDA_BWD_C
#undef KDA_BWD
    return hipErrorInvalidValue;
}

}  // namespace kda
