// KDA chunked backward: gradients of the chunked prefill with respect to q, k, v, g = log(alpha),
// beta and the initial state, given dL/do and dL/dS_T.  fp32 arithmetic throughout.
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
// tile on the fp32 matrix cores (v_mfma_f32_16x16x4f32).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves
constexpr int kBV = 16;        // value columns per chain workgroup

// acc += A (16 x 4KS) * B (4KS x 16) with A(r, k) = A[r * ar + k * ak] and B(k, c) = B[k * bk + c * bc].
// Result layout: acc[e] is row 4 * (lane >> 4) + e, column lane & 15.
template <int KS>
__device__ __forceinline__ floatx4 mma(const float* A, int ar, int ak, const float* B, int bk, int bc, floatx4 acc,
                                       int lane) {
    const int r = lane & 15, kq = lane >> 4;
    const float* pa = A + r * ar + kq * ak;
    const float* pb = B + kq * bk + r * bc;
#pragma unroll 4
    for (int ks = 0; ks < KS; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[4 * ks * ak], pb[4 * ks * bk], acc, 0, 0, 0);
    return acc;
}

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// sum over the 16 lanes that share (lane >> 4)
__device__ __forceinline__ float sum16(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    return x;
}

// Workspace record of one (chunk slot, head), in floats.
template <int DK, int DV, int C>
struct Rec {
    static constexpr int64_t W = 0;                       // [C][DK]  T Diag(beta) K+
    static constexpr int64_t U = W + C * DK;              // [C][DV]  T Diag(beta) V
    static constexpr int64_t Kd = U + C * DV;             // [C][DK]  K'
    static constexpr int64_t Qp = Kd + C * DK;            // [C][DK]  Q+
    static constexpr int64_t M = Qp + C * DK;             // [C][C]
    static constexpr int64_t T = M + C * C;               // [C][C]
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

// Sequences (device cu_seqlens) and chunk slots: sequence n owns slots base(n) .. base(n) + chunks - 1.
template <int C>
struct Map {
    const int32_t* cu;
    int64_t N;
    __device__ __forceinline__ int64_t base(int64_t n) const { return (int64_t)cu[n] / C + n; }
    __device__ __forceinline__ bool locate(int64_t slot, int64_t& n, int64_t& c, int64_t& t0, int& L) const {
        if (N <= 0 || base(0) > slot) return false;
        int64_t lo = 0, hi = N - 1;
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) >> 1;
            if (base(mid) <= slot) lo = mid; else hi = mid - 1;
        }
        n = lo;
        c = slot - base(n);
        const int64_t bos = cu[n], eos = cu[n + 1];
        t0 = bos + c * C;
        if (t0 >= eos) return false;
        L = (int)(eos - t0 < C ? eos - t0 : C);
        return true;
    }
};

__device__ __forceinline__ float gate_at(const float* g, int gate_head, int64_t t, int H, int h, int DK, int c) {
    return gate_head ? g[t * H + h] : g[(t * H + h) * (int64_t)DK + c];
}

// In-chunk cumulative log-decay into G[C][ldg] (rows >= L take g = 0, so they repeat G[L-1]).
// Thread (c, half) sums its half of the rows in registers; the second half then adds the first's total.
template <int DK, int C>
__device__ __forceinline__ void cumulative_decay(const BwdArgs& a, int64_t t0, int L, int h, float* G, int ldg) {
    constexpr int HALF = C / 2;
    for (int task = threadIdx.x; task < 2 * DK; task += kThreads) {
        const int c = task % DK, half = task / DK;
        float acc = 0.f;
#pragma unroll 8
        for (int i = 0; i < HALF; ++i) {
            const int r = half * HALF + i;
            acc += r < L ? gate_at(a.g, a.gate_head, t0 + r, a.H, h, DK, c) : 0.f;
            G[r * ldg + c] = acc;
        }
    }
    __syncthreads();
    for (int task = threadIdx.x; task < DK * HALF; task += kThreads) {
        const int c = task % DK, r = HALF + task / DK;
        G[r * ldg + c] += G[(HALF - 1) * ldg + c];
    }
    __syncthreads();
}

// ------------------------------------------------------------------------------------------
// factors: one workgroup per (chunk slot, head)
// ------------------------------------------------------------------------------------------
template <int DK, int DV, int C, typename TI>
__global__ __launch_bounds__(kThreads) void factors_kernel(BwdArgs a, Map<C> mp) {
    using R = Rec<DK, DV, C>;
    constexpr int LK = DK + 1, DX = DK > DV ? DK : DV, LX = DX + 1, LC = C + 1;
    extern __shared__ float lds[];
    float* sK = lds;             // [C][LK]  k, then beta K+
    float* sX = sK + C * LK;     // [C][LX]  q, then beta V
    float* sG = sX + C * LX;     // [C][LK]
    float* sP = sG + C * LK;     // [C][LC]
    float* sM = sP + C * LC;     // [C][LC]
    float* sT = sM + C * LC;     // [C][LC]
    float* sB = sT + C * LC;     // [C]

    const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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

    for (int e = tid; e < C * DK; e += kThreads) {
        const int r = e / DK, cc = e % DK;
        const int64_t idx = ((t0 + r) * H + h) * (int64_t)DK + cc;
        sK[r * LK + cc] = r < L ? ld_in<TI>(k, idx) : 0.f;
        sX[r * LX + cc] = r < L ? ld_in<TI>(q, idx) : 0.f;
    }
    if (tid < C) sB[tid] = tid < L ? ld_in<TI>(beta, (t0 + tid) * H + h) : 0.f;
    cumulative_decay<DK, C>(a, t0, L, h, sG, LK);  // (ends with a barrier)

    // pairwise P and M: thread owns column s, rows r = rg, rg + NG, ...
    {
        constexpr int NG = kThreads / C;
        const int s = tid % C, rg = tid / C;
        for (int r = rg; r < C; r += NG) {
            float p = 0.f, m = 0.f;
            if (s <= r) {
                const float* kr = sK + r * LK;
                const float* ks = sK + s * LK;
                const float* qr = sX + r * LX;
                const float* gr = sG + r * LK;
                const float* gs = sG + s * LK;
#pragma unroll 4
                for (int cc = 0; cc < DK; ++cc) {
                    const float e = fast_exp(gr[cc] - gs[cc]);
                    const float ke = ks[cc] * e;
                    p += kr[cc] * ke;
                    m += qr[cc] * ke;
                }
            }
            sP[r * LC + s] = s < r ? p : 0.f;
            sM[r * LC + s] = s <= r ? m : 0.f;
        }
    }
    __syncthreads();

    // Q+, K', gamma, M, P out
    for (int e = tid; e < C * DK; e += kThreads) {
        const int r = e / DK, cc = e % DK;
        const float g = sG[r * LK + cc], gl = sG[(C - 1) * LK + cc];
        rec[R::Qp + e] = sX[r * LX + cc] * fast_exp(g);
        rec[R::Kd + e] = sK[r * LK + cc] * fast_exp(gl - g);
    }
    for (int cc = tid; cc < DK; cc += kThreads) rec[R::gam + cc] = fast_exp(sG[(C - 1) * LK + cc]);
    for (int e = tid; e < C * C; e += kThreads) {
        const int r = e / C, s = e % C;
        rec[R::M + e] = sM[r * LC + s];
        rec[R::P + e] = sP[r * LC + s];
    }
    __syncthreads();
    // A = Diag(beta) P into M's buffer; T zeroed; K becomes beta K+ and q's buffer beta V
    float* sA = sM;
    for (int e = tid; e < C * C; e += kThreads) {
        const int r = e / C, s = e % C;
        sA[r * LC + s] = sB[r] * sP[r * LC + s];
        sT[r * LC + s] = 0.f;
    }
    for (int e = tid; e < C * DK; e += kThreads) {
        const int r = e / DK, cc = e % DK;
        sK[r * LK + cc] *= sB[r] * fast_exp(sG[r * LK + cc]);
    }
    for (int e = tid; e < C * DV; e += kThreads) {
        const int r = e / DV, j = e % DV;
        sX[r * LX + j] = r < L ? sB[r] * ld_in<TI>(v, ((t0 + r) * H + h) * (int64_t)DV + j) : 0.f;
    }
    __syncthreads();

    // T = (I + A)^{-1}, unit lower triangular.  Diagonal 16x16 blocks by forward substitution (lane =
    // column, the block's rows in registers); then the blocks below the diagonal, nearest first:
    // T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj.
    constexpr int NR = C / 16;
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
    __syncthreads();
    float* sXs = sP + w * 16 * 17;  // per-wave 16x16 scratch (P is in the record already)
    for (int dist = 1; dist < NR; ++dist) {
        const int j = w, i = w + dist;
        if (i < NR) {
            floatx4 acc = zero4();
            for (int m = j; m < i; ++m)
                acc = mma<4>(sA + 16 * i * LC + 16 * m, LC, 1, sT + 16 * m * LC + 16 * j, LC, 1, acc, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) sXs[(4 * (lane >> 4) + e) * 17 + (lane & 15)] = acc[e];
        }
        __syncthreads();
        if (i < NR) {
            const floatx4 t = mma<4>(sT + 16 * i * LC + 16 * i, LC, 1, sXs, 17, 1, zero4(), lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) sT[(16 * i + 4 * (lane >> 4) + e) * LC + 16 * j + (lane & 15)] = -t[e];
        }
        __syncthreads();
    }
    for (int e = tid; e < C * C; e += kThreads) rec[R::T + e] = sT[(e / C) * LC + e % C];

    // W = T (beta K+), U = T (beta V): 16x16 tiles over the waves
    for (int t = w; t < NR * (DK / 16); t += 4) {
        const int rb = t % NR, cb = t / NR;
        floatx4 acc = mma<C / 4>(sT + 16 * rb * LC, LC, 1, sK + 16 * cb, LK, 1, zero4(), lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) rec[R::W + (16 * rb + 4 * (lane >> 4) + e) * DK + 16 * cb + (lane & 15)] = acc[e];
    }
    for (int t = w; t < NR * (DV / 16); t += 4) {
        const int rb = t % NR, cb = t / NR;
        floatx4 acc = mma<C / 4>(sT + 16 * rb * LC, LC, 1, sX + 16 * cb, LX, 1, zero4(), lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) rec[R::U + (16 * rb + 4 * (lane >> 4) + e) * DV + 16 * cb + (lane & 15)] = acc[e];
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
                float* p = dst + row * ld + 4 * c4;
                p[0] = r[m].x;
                p[1] = r[m].y;
                p[2] = r[m].z;
                p[3] = r[m].w;
            }
        }
    }
};

// ------------------------------------------------------------------------------------------
// fwd_chain: one workgroup per (sequence, head, 16 value columns); states entering each chunk
// ------------------------------------------------------------------------------------------
template <int DK, int DV, int C>
__global__ __launch_bounds__(kThreads) void fwd_chain_kernel(BwdArgs a, Map<C> mp) {
    using R = Rec<DK, DV, C>;
    constexpr int NVB = DV / kBV, LW = DK + 4, LQ = DK + 16;
    __shared__ float sW[C * LW];   // W rows (A operand by rows)
    __shared__ float sKd[C * LQ];  // K' rows (A operand by columns)
    __shared__ float sU[C * kBV];
    __shared__ float sg[DK];
    __shared__ float sS[DK * kBV];
    __shared__ float sD[C * kBV];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t gid = blockIdx.x;
    const int vb = (int)(gid % NVB), h = (int)((gid / NVB) % a.H);
    const int64_t n = gid / NVB / a.H;
    const int H = a.H;
    for (int e = tid; e < DK * kBV; e += kThreads) {
        const int i = e / kBV, j = e % kBV;
        sS[e] = a.s0 ? a.s0[((n * H + h) * DK + i) * (int64_t)DV + vb * kBV + j] : 0.f;
    }
    const int64_t bos = mp.cu[n], eos = mp.cu[n + 1];
    const int64_t nck = (eos - bos + C - 1) / C, slot0 = mp.base(n);
    if (nck == 0) return;  // uniform
    Stage<C, DK> pW, pK;
    Stage<C, kBV> pU;
    Stage<1, DK> pg;
    auto fetch = [&](int64_t c) {
        const float* rec = a.ws + ((slot0 + c) * H + h) * R::kFloats;
        pW.load(rec + R::W, DK);
        pK.load(rec + R::Kd, DK);
        pU.load(rec + R::U + vb * kBV, DV);
        pg.load(rec + R::gam, DK);
    };
    fetch(0);
    for (int64_t c = 0; c < nck; ++c) {
        float* rec = a.ws + ((slot0 + c) * H + h) * R::kFloats;
        __syncthreads();  // the previous chunk is done with the LDS operands; sS is its final state
        pW.store(sW, LW);
        pK.store(sKd, LQ);
        pU.store(sU, kBV);
        pg.store(sg, DK);
        fetch(c + 1 < nck ? c + 1 : c);
        for (int e = tid; e < DK * kBV; e += kThreads) rec[R::S0 + (e / kBV) * DV + vb * kBV + e % kBV] = sS[e];
        __syncthreads();
        // D = U - W S
        for (int rb = w; rb < C / 16; rb += 4) {
            const floatx4 acc = mma<DK / 4>(sW + 16 * rb * LW, LW, 1, sS, kBV, 1, zero4(), lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * (lane >> 4) + e, j = lane & 15;
                const float d = sU[r * kBV + j] - acc[e];
                sD[r * kBV + j] = d;
                rec[R::D + r * DV + vb * kBV + j] = d;
            }
        }
        __syncthreads();
        // S <- Diag(gamma) S + K'^T D
        for (int cb = w; cb < DK / 16; cb += 4) {
            floatx4 acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * cb + 4 * (lane >> 4) + e;
                acc[e] = sg[i] * sS[i * kBV + (lane & 15)];
            }
            acc = mma<C / 4>(sKd + 16 * cb, 1, LQ, sD, kBV, 1, acc, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) sS[(16 * cb + 4 * (lane >> 4) + e) * kBV + (lane & 15)] = acc[e];
        }
    }
}

// ------------------------------------------------------------------------------------------
// rev_chain: one workgroup per (sequence, head, 16 value columns); chunks in reverse
// ------------------------------------------------------------------------------------------
template <int DK, int DV, int C>
__global__ __launch_bounds__(kThreads) void rev_chain_kernel(BwdArgs a, Map<C> mp) {
    using R = Rec<DK, DV, C>;
    constexpr int NVB = DV / kBV, LW = DK + 4, LQ = DK + 16, LM = C + 16;
    __shared__ float sKd[C * LW];  // K' rows (A operand by rows)
    __shared__ float sM[C * LM];   // M (A operand by columns)
    __shared__ float sQp[C * LQ];  // Q+ (A operand by columns)
    __shared__ float sW[C * LQ];   // W (A operand by columns)
    __shared__ float sg[DK];
    __shared__ float sdS[DK * kBV];
    __shared__ float sdO[C * kBV];
    __shared__ float sdD[C * kBV];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t gid = blockIdx.x;
    const int vb = (int)(gid % NVB), h = (int)((gid / NVB) % a.H);
    const int64_t n = gid / NVB / a.H;
    const int H = a.H;
    for (int e = tid; e < DK * kBV; e += kThreads) {
        const int i = e / kBV, j = e % kBV;
        sdS[e] = a.dsT ? a.dsT[((n * H + h) * DK + i) * (int64_t)DV + vb * kBV + j] : 0.f;
    }
    const int64_t bos = mp.cu[n], eos = mp.cu[n + 1];
    const int64_t nck = (eos - bos + C - 1) / C, slot0 = mp.base(n);
    Stage<C, DK> pK, pQ, pW;
    Stage<C, C> pM;
    Stage<1, DK> pg;
    constexpr int kDoPer = (C * kBV + kThreads - 1) / kThreads;
    float rdo[kDoPer];
    auto fetch = [&](int64_t c) {
        const float* rec = a.ws + ((slot0 + c) * H + h) * R::kFloats;
        pK.load(rec + R::Kd, DK);
        pM.load(rec + R::M, C);
        pQ.load(rec + R::Qp, DK);
        pW.load(rec + R::W, DK);
        pg.load(rec + R::gam, DK);
        const int64_t t0 = bos + c * C;
#pragma unroll
        for (int m = 0; m < kDoPer; ++m) {
            const int e = tid + m * kThreads, r = e / kBV, j = e % kBV;
            rdo[m] = (e < C * kBV && t0 + r < eos) ? a.dO[((t0 + r) * H + h) * (int64_t)DV + vb * kBV + j] : 0.f;
        }
    };
    if (nck > 0) fetch(nck - 1);
    for (int64_t c = nck - 1; c >= 0; --c) {
        float* rec = a.ws + ((slot0 + c) * H + h) * R::kFloats;
        __syncthreads();  // the previous chunk is done with the LDS operands; sdS is its result
        pK.store(sKd, LW);
        pM.store(sM, LM);
        pQ.store(sQp, LQ);
        pW.store(sW, LQ);
        pg.store(sg, DK);
#pragma unroll
        for (int m = 0; m < kDoPer; ++m) {
            const int e = tid + m * kThreads;
            if (e < C * kBV) sdO[e] = rdo[m];
        }
        fetch(c > 0 ? c - 1 : c);
        for (int e = tid; e < DK * kBV; e += kThreads) rec[R::dS1 + (e / kBV) * DV + vb * kBV + e % kBV] = sdS[e];
        __syncthreads();
        // dD = K' dS + M^T dO
        for (int rb = w; rb < C / 16; rb += 4) {
            floatx4 acc = mma<DK / 4>(sKd + 16 * rb * LW, LW, 1, sdS, kBV, 1, zero4(), lane);
            acc = mma<C / 4>(sM + 16 * rb, 1, LM, sdO, kBV, 1, acc, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * (lane >> 4) + e, j = lane & 15;
                sdD[r * kBV + j] = acc[e];
                rec[R::dD + r * DV + vb * kBV + j] = acc[e];
            }
        }
        __syncthreads();
        // dS <- Diag(gamma) dS + Q+^T dO - W^T dD
        for (int cb = w; cb < DK / 16; cb += 4) {
            floatx4 acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * cb + 4 * (lane >> 4) + e;
                acc[e] = sg[i] * sdS[i * kBV + (lane & 15)];
            }
            acc = mma<C / 4>(sQp + 16 * cb, 1, LQ, sdO, kBV, 1, acc, lane);
            const floatx4 wd = mma<C / 4>(sW + 16 * cb, 1, LQ, sdD, kBV, 1, zero4(), lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) sdS[(16 * cb + 4 * (lane >> 4) + e) * kBV + (lane & 15)] = acc[e] - wd[e];
        }
    }
    __syncthreads();
    if (a.gs0)
        for (int e = tid; e < DK * kBV; e += kThreads) {
            const int i = e / kBV, j = e % kBV;
            a.gs0[((n * H + h) * DK + i) * (int64_t)DV + vb * kBV + j] = sdS[e];
        }
}

// ------------------------------------------------------------------------------------------
// grad_state: one workgroup per (chunk slot, head); the products over the value axis, staged
// through LDS 32 value columns at a time
// ------------------------------------------------------------------------------------------
template <int DK, int DV, int C>
__global__ __launch_bounds__(kThreads) void grad_state_kernel(BwdArgs a, Map<C> mp) {
    using R = Rec<DK, DV, C>;
    constexpr int JT = DV < 32 ? DV : 32, LJ = JT + 1;
    constexpr int NR = C / 16, NC = DK / 16, NT3 = NR * NC, NTM = NR * NR;
    constexpr int T3W = (NT3 + 3) / 4, TMW = (NTM + 3) / 4;
    __shared__ float sD[C * LJ];
    __shared__ float sdD[C * LJ];
    __shared__ float sdO[C * LJ];
    __shared__ float sS0[DK * LJ];
    __shared__ float sdS1[DK * LJ];
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
    for (int j0 = 0; j0 < DV; j0 += JT) {
        for (int e = tid; e < C * JT; e += kThreads) {
            const int r = e / JT, j = e % JT;
            sD[r * LJ + j] = rec[R::D + r * DV + j0 + j];
            sdD[r * LJ + j] = rec[R::dD + r * DV + j0 + j];
            sdO[r * LJ + j] = r < L ? a.dO[((t0 + r) * H + h) * (int64_t)DV + j0 + j] : 0.f;
        }
        for (int e = tid; e < DK * JT; e += kThreads) {
            const int i = e / JT, j = e % JT;
            sS0[i * LJ + j] = rec[R::S0 + i * DV + j0 + j];
            sdS1[i * LJ + j] = rec[R::dS1 + i * DV + j0 + j];
        }
        __syncthreads();
        // dK' = D dS1^T, dQ+ = dO S0^T, dW = -dD S0^T   ([C][DK] each)
#pragma unroll
        for (int m = 0; m < T3W; ++m) {
            const int t = w + 4 * m, rb = t % NR, cb = t / NR;
            if (t < NT3) {
                kd[m] = mma<JT / 4>(sD + 16 * rb * LJ, LJ, 1, sdS1 + 16 * cb * LJ, 1, LJ, kd[m], lane);
                qp[m] = mma<JT / 4>(sdO + 16 * rb * LJ, LJ, 1, sS0 + 16 * cb * LJ, 1, LJ, qp[m], lane);
                dw[m] = mma<JT / 4>(sdD + 16 * rb * LJ, LJ, 1, sS0 + 16 * cb * LJ, 1, LJ, dw[m], lane);
            }
        }
        // dM = tril(dO D^T)   ([C][C], the tiles on or below the diagonal)
#pragma unroll
        for (int m = 0; m < TMW; ++m) {
            const int t = w + 4 * m, rb = t / NR, sb = t % NR;
            if (t < NTM && sb <= rb)
                dm[m] = mma<JT / 4>(sdO + 16 * rb * LJ, LJ, 1, sD + 16 * sb * LJ, 1, LJ, dm[m], lane);
        }
        // dgamma = rowsum(dS1 * S0)
        if (tid < DK)
            for (int j = 0; j < JT; ++j) dgam += sdS1[tid * LJ + j] * sS0[tid * LJ + j];
        __syncthreads();
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
    if (tid < DK) rec[R::dgam + tid] = dgam;
}

// ------------------------------------------------------------------------------------------
// grad_chunk: one workgroup per (chunk slot, head); dq, dk, dv, dg, dbeta
// ------------------------------------------------------------------------------------------
template <int DK, int DV, int C>
struct ChunkLds {
    static constexpr int LC = C + 1, LK = DK + 1, LB = 17;
    static constexpr int JT = DV < 32 ? DV : 32, LJ = JT + 1;  // value columns per staged tile
    static constexpr int CT = DK < 32 ? DK : 32, LCT = CT + 1; // key channels per staged tile
    static constexpr int kStage0 = 3 * LJ > 2 * LCT ? 3 * LJ : 2 * LCT;
    static constexpr int kStage = kStage0 > 5 * LB ? kStage0 : 5 * LB;  // floats per row of the staging area
    static constexpr size_t kFloats = 4 * (size_t)C * LC      // T, dM, dT -> dA -> dP, Z
                                      + (size_t)C * LK        // G
                                      + (size_t)C * kStage    // staged tiles (see the kernel)
                                      + 4 * (size_t)C         // beta, dbeta, dg (one gate per head), spare
                                      + 2 * 16;               // per-block column sums
    static constexpr size_t kBytes = kFloats * sizeof(float);
};

template <int DK, int DV, int C, typename TI>
__global__ __launch_bounds__(kThreads) void grad_chunk_kernel(BwdArgs a, Map<C> mp) {
    using R = Rec<DK, DV, C>;
    using Lds = ChunkLds<DK, DV, C>;
    constexpr int LC = Lds::LC, LK = Lds::LK, LB = Lds::LB, NR = C / 16;
    constexpr int JT = Lds::JT, LJ = Lds::LJ, CT = Lds::CT, LCT = Lds::LCT;
    extern __shared__ float lds[];
    float* sT = lds;             // [C][LC]
    float* sdM = sT + C * LC;    // [C][LC]
    float* sA = sdM + C * LC;    // [C][LC]  dT, then dP
    float* sZ = sA + C * LC;     // [C][LC]
    float* sG = sZ + C * LC;     // [C][LK]
    float* sX = sG + C * LK;     // [C][kStage] staging area
    float* sB = sX + C * Lds::kStage;  // [C]
    float* sdb = sB + C;         // [C]
    float* sdgh = sdb + C;       // [C]
    float* sCol = sdgh + 2 * C;  // [16] column sums of dK' * K' in the current channel block
    // staged tiles inside sX: value tiles dD, V, beta V ([C][LJ] each); key tiles dW, beta K+
    // ([C][LCT] each); channel blocks K, Q, dK+, dG, dW ([C][LB] each)
    float* tdD = sX;
    float* tV = tdD + C * LJ;
    float* tBV = tV + C * LJ;
    float* tdW = sX;
    float* tBK = tdW + C * LCT;
    float* tK = sX;
    float* tQ = tK + C * LB;
    float* tKp = tQ + C * LB;
    float* tdG = tKp + C * LB;
    float* tW = tdG + C * LB;

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

    for (int e = tid; e < C * C; e += kThreads) {
        const int r = e / C, s = e % C;
        sT[r * LC + s] = rec[R::T + e];
        sdM[r * LC + s] = rec[R::dM + e];
    }
    if (tid < C) {
        sB[tid] = tid < L ? ld_in<TI>(beta, (t0 + tid) * H + h) : 0.f;
        sdb[tid] = 0.f;
        sdgh[tid] = 0.f;
    }
    cumulative_decay<DK, C>(a, t0, L, h, sG, LK);  // (ends with a barrier)

    // ---- dT = dD (beta V)^T + dW (beta K+)^T, strictly lower part (wave w owns tiles w, w+4, ...),
    //      and with the value tiles staged: dV = beta (T^T dD), dbeta += rowsum(V * T^T dD)
    constexpr int NT = NR * NR, TPW = (NT + 3) / 4;
    floatx4 dT[TPW];
#pragma unroll
    for (int m = 0; m < TPW; ++m) dT[m] = zero4();
    for (int j0 = 0; j0 < DV; j0 += JT) {
        for (int e = tid; e < C * JT; e += kThreads) {
            const int r = e / JT, j = e % JT;
            const float vv = r < L ? ld_in<TI>(v, ((t0 + r) * H + h) * (int64_t)DV + j0 + j) : 0.f;
            tdD[r * LJ + j] = rec[R::dD + r * DV + j0 + j];
            tV[r * LJ + j] = vv;
            tBV[r * LJ + j] = sB[r] * vv;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int t = w + 4 * m, rb = t / NR, sb = t % NR;
            if (t < NT && sb <= rb)
                dT[m] = mma<JT / 4>(tdD + 16 * rb * LJ, LJ, 1, tBV + 16 * sb * LJ, 1, LJ, dT[m], lane);
        }
        for (int t = w; t < NR * (JT / 16); t += 4) {
            const int rb = t % NR, jb = t / NR;
            const floatx4 x = mma<C / 4>(sT + 16 * rb, 1, LC, tdD + 16 * jb, LJ, 1, zero4(), lane);
            float part[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * (lane >> 4) + e, j = 16 * jb + (lane & 15);
                part[e] = tV[r * LJ + j] * x[e];
                if (r < L) a.gv[((t0 + r) * H + h) * (int64_t)DV + j0 + j] = sB[r] * x[e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = sum16(part[e]);
                if ((lane & 15) == 0) atomicAdd(&sdb[16 * rb + 4 * (lane >> 4) + e], p);
            }
        }
        __syncthreads();
    }
    for (int c0 = 0; c0 < DK; c0 += CT) {
        for (int e = tid; e < C * CT; e += kThreads) {
            const int r = e / CT, cc = e % CT;
            tdW[r * LCT + cc] = rec[R::dW + r * DK + c0 + cc];
            tBK[r * LCT + cc] = r < L ? sB[r] * ld_in<TI>(k, ((t0 + r) * H + h) * (int64_t)DK + c0 + cc) *
                                            fast_exp(sG[r * LK + c0 + cc])
                                      : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int t = w + 4 * m, rb = t / NR, sb = t % NR;
            if (t < NT && sb <= rb)
                dT[m] = mma<CT / 4>(tdW + 16 * rb * LCT, LCT, 1, tBK + 16 * sb * LCT, 1, LCT, dT[m], lane);
        }
        __syncthreads();
    }
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
    __syncthreads();
    // ---- dA = -T^T dT T^T (strictly lower): Z = T^T dT, then dA = -Z T^T
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
        const int t = w + 4 * m, rb = t / NR, sb = t % NR;
        if (t < NT) {
            const floatx4 z = mma<C / 4>(sT + 16 * rb, 1, LC, sA + 16 * sb, LC, 1, zero4(), lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) sZ[(16 * rb + 4 * (lane >> 4) + e) * LC + 16 * sb + (lane & 15)] = z[e];
        }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
        const int t = w + 4 * m, rb = t / NR, sb = t % NR;
        if (t < NT) dT[m] = mma<C / 4>(sZ + 16 * rb * LC, LC, 1, sT + 16 * sb * LC, 1, LC, zero4(), lane);
    }
    __syncthreads();  // every read of sA (dT) is done
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
        const int t = w + 4 * m, rb = t / NR, sb = t % NR;
        if (t < NT) {
            float part[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * (lane >> 4) + e, s = 16 * sb + (lane & 15);
                const float da = s < r ? -dT[m][e] : 0.f;
                part[e] = da * rec[R::P + r * C + s];
                sA[r * LC + s] = sB[r] * da;  // dP
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = sum16(part[e]);
                if ((lane & 15) == 0) atomicAdd(&sdb[16 * rb + 4 * (lane >> 4) + e], p);
            }
        }
    }
    __syncthreads();  // dP complete; sX free

    // ---- channel blocks of 16: dK+, the pairwise sweeps, dq, dk, dG and its suffix sums
    for (int cb = 0; cb < DK / 16; ++cb) {
        for (int e = tid; e < C * 16; e += kThreads) {
            const int r = e / 16, cc = e % 16;
            const int64_t idx = ((t0 + r) * H + h) * (int64_t)DK + 16 * cb + cc;
            tK[r * LB + cc] = r < L ? ld_in<TI>(k, idx) : 0.f;
            tQ[r * LB + cc] = r < L ? ld_in<TI>(q, idx) : 0.f;
            tW[r * LB + cc] = rec[R::dW + r * DK + 16 * cb + cc];
        }
        if (tid < 16) sCol[tid] = 0.f;
        __syncthreads();
        // X2 = T^T dW (rows block w), dK+ = beta X2, dbeta += rowsum(K+ * X2)
        if (w < NR) {
            const floatx4 x = mma<C / 4>(sT + 16 * w, 1, LC, tW, LB, 1, zero4(), lane);
            float part[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * w + 4 * (lane >> 4) + e, cc = lane & 15;
                part[e] = tK[r * LB + cc] * fast_exp(sG[r * LK + 16 * cb + cc]) * x[e];
                tKp[r * LB + cc] = sB[r] * x[e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = sum16(part[e]);
                if ((lane & 15) == 0) atomicAdd(&sdb[16 * w + 4 * (lane >> 4) + e], p);
            }
        }
        __syncthreads();
        // thread: channel cc = tid & 15, rows r = (tid >> 4) + 16 i
        {
            const int cc = tid & 15, ch = 16 * cb + cc;
            const float glast = sG[(C - 1) * LK + ch];
            float colsum = 0.f;
            for (int r = tid >> 4; r < C; r += 16) {
                const float gr = sG[r * LK + ch];
                const float kr = tK[r * LB + cc], qr = tQ[r * LB + cc];
                float rq = 0.f, rk = 0.f, ck = 0.f;
                // row role (this row r, columns s <= r) and column role (this row as s, rows r2 >= s)
                for (int s = 0; s < C; ++s) {
                    const float gs = sG[s * LK + ch];
                    if (s <= r) {
                        const float e = fast_exp(gr - gs) * tK[s * LB + cc];
                        rq += sdM[r * LC + s] * e;
                        rk += sA[r * LC + s] * e;  // dP is zero on the diagonal
                    } else {
                        const float e = fast_exp(gs - gr);
                        ck += e * (sdM[s * LC + r] * tQ[s * LB + cc] + sA[s * LC + r] * tK[s * LB + cc]);
                    }
                }
                // the diagonal term of the column role: only M has one (dM[r][r] q_r)
                ck += sdM[r * LC + r] * qr;
                float dq = 0.f, dk = 0.f, dG = 0.f;
                if (r < L) {
                    const float eg = fast_exp(gr), ed = fast_exp(glast - gr);
                    const int64_t o = r * DK + ch;
                    const float dQp = rec[R::dQp + o], dKd = rec[R::dKd + o], dKp = tKp[r * LB + cc];
                    dq = dQp * eg + rq;
                    dk = dKp * eg + rec[R::dKd + o] * ed + rk + ck;
                    dG = dKp * kr * eg + dQp * qr * eg - dKd * kr * ed + qr * rq + kr * rk - kr * ck;
                    colsum += dKd * kr * ed;
                    const int64_t go = ((t0 + r) * H + h) * (int64_t)DK + ch;
                    a.gq[go] = dq;
                    a.gk[go] = dk;
                }
                tdG[r * LB + cc] = dG;
            }
            atomicAdd(&sCol[cc], colsum);
        }
        __syncthreads();
        if (tid < 16) {
            const int ch = 16 * cb + tid;
            const float glast = sG[(C - 1) * LK + ch];
            tdG[(L - 1) * LB + tid] += sCol[tid] + rec[R::dgam + ch] * fast_exp(glast);
        }
        __syncthreads();
        // dg = suffix sums over the chunk's rows: dg = Triu(ones) dG
        if (w < NR) {
            const int r = lane & 15, kq = lane >> 4;
            floatx4 acc = zero4();
#pragma unroll 4
            for (int ks = 0; ks < C / 4; ++ks) {
                const int s = 4 * ks + kq;
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(s >= 16 * w + r ? 1.f : 0.f, tdG[s * LB + r], acc, 0, 0, 0);
            }
            float hsum[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = 16 * w + 4 * (lane >> 4) + e, cc = lane & 15;
                if (!a.gate_head && rr < L) a.gg[((t0 + rr) * H + h) * (int64_t)DK + 16 * cb + cc] = acc[e];
                hsum[e] = sum16(acc[e]);
            }
            if (a.gate_head && (lane & 15) == 0)
#pragma unroll
                for (int e = 0; e < 4; ++e) sdgh[16 * w + 4 * (lane >> 4) + e] += hsum[e];
        }
        __syncthreads();  // the tiles are rewritten by the next block
    }
    if (tid < L) {
        a.gbeta[(t0 + tid) * H + h] = sdb[tid];
        if (a.gate_head) a.gg[(t0 + tid) * H + h] = sdgh[tid];
    }
}

// ------------------------------------------------------------------------------------------
// launch
// ------------------------------------------------------------------------------------------
template <int DK, int DV, int C>
constexpr size_t factors_lds() {
    constexpr int DX = DK > DV ? DK : DV;
    return ((size_t)C * (DK + 1) * 2 + (size_t)C * (DX + 1) + 3 * (size_t)C * (C + 1) + C) * sizeof(float);
}

template <typename K>
hipError_t set_lds(K kernel, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

int64_t num_slots(int64_t N, int64_t T_total, int C) { return T_total / C + N + 1; }

template <int DK, int DV, int C, typename TI>
hipError_t launch_typed(const BwdArgs& a, hipStream_t s) {
    const Map<C> mp{a.cu, a.N};
    const int64_t slots = num_slots(a.N, a.T_total, C);
    const dim3 per_chunk((unsigned)slots, (unsigned)a.H), chains((unsigned)(a.N * a.H * (DV / kBV)));
    const bool timed = timing_on();
    hipError_t e;
    constexpr size_t f_lds = factors_lds<DK, DV, C>(), c_lds = ChunkLds<DK, DV, C>::kBytes;
    if ((e = set_lds(factors_kernel<DK, DV, C, TI>, f_lds)) != hipSuccess) return e;
    if ((e = set_lds(grad_chunk_kernel<DK, DV, C, TI>, c_lds)) != hipSuccess) return e;
    if (a.T_total > 0) {
        if (timed) timed_begin(kKernelBwdFactors, s);
        hipLaunchKernelGGL((factors_kernel<DK, DV, C, TI>), per_chunk, dim3(kThreads), f_lds, s, a, mp);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (timed) timed_end(s);
        if (timed) timed_begin(kKernelBwdFwdChain, s);
        hipLaunchKernelGGL((fwd_chain_kernel<DK, DV, C>), chains, dim3(kThreads), 0, s, a, mp);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (timed) timed_end(s);
    }
    if (timed) timed_begin(kKernelBwdRevChain, s);
    hipLaunchKernelGGL((rev_chain_kernel<DK, DV, C>), chains, dim3(kThreads), 0, s, a, mp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (timed) timed_end(s);
    if (a.T_total > 0) {
        if (timed) timed_begin(kKernelBwdGradState, s);
        hipLaunchKernelGGL((grad_state_kernel<DK, DV, C>), per_chunk, dim3(kThreads), 0, s, a, mp);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (timed) timed_end(s);
        if (timed) timed_begin(kKernelBwdGradChunk, s);
        hipLaunchKernelGGL((grad_chunk_kernel<DK, DV, C, TI>), per_chunk, dim3(kThreads), c_lds, s, a, mp);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (timed) timed_end(s);
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
    return (size_t)num_slots(N, T_total, chunk) * (size_t)H * (size_t)per * sizeof(float);
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
