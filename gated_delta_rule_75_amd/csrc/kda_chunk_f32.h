// The fp32 chunked evaluation of one (sequence, head, 16-column value block) chain, as a
// device function: the body of the fp32 chunked kernel, and the path the matrix-core state pass
// takes for a chain that met a value beyond the fp16 range.
//
// "Training in chunks" in "Kimi K3, explained" rewrites the product of the per-token
// decay-and-erase transitions inside a chunk into dense products and carries only the state
// across chunks.  The chunk equations follow from unrolling the gated delta rule ("The math")
// over a chunk of L tokens r, s = 0..L-1, with G[r] = sum_{s<=r} g_s per key channel
// (restarting at the chunk) and S0 the state entering the chunk:
//   A[r,s] = beta_r sum_c k_rc k_sc exp(G_rc - G_sc)   (s < r)
//   M[r,s] =        sum_c q_rc k_sc exp(G_rc - G_sc)   (s <= r)
//   T      = (I + A)^{-1}          (unit lower triangular, forward substitution)
//   R      = Diag(beta) (V - K+ S0),         K+[r,c] = k_rc exp(G_rc)
//   D      = T R                  (the per-token corrections delta_r)
//   O      = Q+ S0 + M D,                    Q+[r,c] = q_rc exp(G_rc)
//   S1     = Diag(exp(G_{L-1})) S0 + K'^T D, K'[s,c] = k_sc exp(G_{L-1,c} - G_sc)
// Every exponential is of a non-positive difference, so nothing overflows for any decay
// strength.  fp32 inputs are used as given and every product is fp32 FMA on the vector ALUs.
// With one forget gate per head (Gated DeltaNet) every key channel takes the same log-decay.
#pragma once
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kF32BV = 16;  // value columns per chain

template <int DK, int C>
struct F32Lds {
    static constexpr int kLdc = C + 1;
    static constexpr size_t kFloats =
        3 * (size_t)C * DK       // k, q, G
        + 3 * (size_t)C * kLdc   // A, M, T
        + (size_t)DK * kF32BV       // S
        + 2 * (size_t)C * kF32BV    // R, D
        + C                      // beta
        + 2 * (size_t)C;         // 1/|k|, 1/|q| per row (fused prologue)
    static constexpr size_t kBytes = kFloats * sizeof(float);
};

// One (sequence n, head h, 16-column value block vb) chain over all its chunks, computed by the
// NT threads of the calling workgroup (every one of them calls it: it contains barriers).
// lds: F32Lds<DK, C>::kBytes bytes of LDS.
template <int DK, int DV, int C, int NT, typename TI>
__device__ void f32_chain(const PrefillArgs& a, int64_t n, int h, int vb, float* lds) {
    using Lds = F32Lds<DK, C>;
    constexpr int LDC = Lds::kLdc;
    float* sk = lds;                    // [C][DK] keys
    float* sq = sk + C * DK;            // [C][DK] queries
    float* sG = sq + C * DK;            // [C][DK] cumulative log-decay
    float* sA = sG + C * DK;            // [C][LDC]
    float* sM = sA + C * LDC;           // [C][LDC]
    float* sT = sM + C * LDC;           // [C][LDC]
    float* sS = sT + C * LDC;           // [DK][kF32BV] state block
    float* sR = sS + DK * kF32BV;          // [C][kF32BV]
    float* sD = sR + C * kF32BV;           // [C][kF32BV]
    float* sb = sD + C * kF32BV;           // [C]
    float* sik = sb + C;                // [C] 1/|k_r| (fused prologue)
    float* siq = sik + C;               // [C] 1/|q_r|

    const TI* q = static_cast<const TI*>(a.q);
    const TI* k = static_cast<const TI*>(a.k);
    const TI* v = static_cast<const TI*>(a.v);
    const TI* beta = static_cast<const TI*>(a.beta);
    const int H = a.H;
    const int tid = threadIdx.x;
    const int64_t bos = a.cu ? (int64_t)a.cu[n] : n * a.T_fixed;
    const int64_t eos = a.cu ? (int64_t)a.cu[n + 1] : bos + a.T_fixed;
    const int64_t sbase = (n * H + h) * (int64_t)DK * DV + vb * kF32BV;

    for (int e = tid; e < DK * kF32BV; e += NT) {
        const int i = e / kF32BV, j = e % kF32BV;
        sS[e] = a.s0 ? a.s0[sbase + (int64_t)i * DV + j] : 0.f;
    }

    for (int64_t t0 = bos; t0 < eos; t0 += C) {
        const int L = (int)((eos - t0) < C ? (eos - t0) : C);
        __syncthreads();  // previous chunk done with every buffer
        for (int e = tid; e < C * DK; e += NT) {
            const int r = e / DK, i = e % DK;
            const int64_t src = ((t0 + r) * H + h) * (int64_t)DK + i;
            sk[e] = r < L ? ld_in(k, src) : 0.f;
            sq[e] = r < L ? ld_in(q, src) : 0.f;
        }
        for (int i = tid; i < DK; i += NT) {
            float acc = 0.f;
            for (int r = 0; r < C; ++r) {
                if (r < L) {
                    float gv = a.gate_head ? a.g[(t0 + r) * H + h] : a.g[((t0 + r) * H + h) * (int64_t)DK + i];
                    acc += a.prologue ? gate_from_raw(gv, a.gate_scale) : gv;
                }
                sG[r * DK + i] = acc;
            }
        }
        for (int r = tid; r < C; r += NT) {
            const float bt = r < L ? ld_in(beta, (t0 + r) * H + h) : 0.f;
            sb[r] = r < L && a.prologue ? sigmoid(bt) : bt;
        }
        __syncthreads();
        if (a.prologue) {  // fused prologue: unit-length keys and queries
            for (int r = tid; r < C; r += NT) {
                float ssk = 0.f, ssq = 0.f;
                for (int c = 0; c < DK; ++c) {
                    ssk += sk[r * DK + c] * sk[r * DK + c];
                    ssq += sq[r * DK + c] * sq[r * DK + c];
                }
                sik[r] = ssk > 0.f ? rsqrtf(ssk) : 0.f;
                siq[r] = ssq > 0.f ? rsqrtf(ssq) : 0.f;
            }
            __syncthreads();
            for (int e = tid; e < C * DK; e += NT) {
                sk[e] *= sik[e / DK];
                sq[e] *= siq[e / DK];
            }
            __syncthreads();
        }

        // gated Gram matrices
        for (int e = tid; e < C * C; e += NT) {
            const int r = e / C, s = e % C;
            float am = 0.f, mm = 0.f;
            if (s <= r && r < L) {
                for (int c = 0; c < DK; ++c) {
                    const float w = sk[s * DK + c] * expf(sG[r * DK + c] - sG[s * DK + c]);
                    am += sk[r * DK + c] * w;
                    mm += sq[r * DK + c] * w;
                }
            }
            sA[r * LDC + s] = s < r ? sb[r] * am : 0.f;
            sM[r * LDC + s] = mm;
        }
        __syncthreads();

        // T = (I + A)^{-1}: thread j owns column j
        if (tid < C) {
            const int j = tid;
            for (int r = 0; r < C; ++r) {
                float t;
                if (r < j) {
                    t = 0.f;
                } else if (r == j) {
                    t = 1.f;
                } else {
                    float acc = 0.f;
                    for (int s = j; s < r; ++s) acc += sA[r * LDC + s] * sT[s * LDC + j];
                    t = -acc;
                }
                sT[r * LDC + j] = t;
            }
        }
        // R = Diag(beta) (V - K+ S0)
        for (int e = tid; e < C * kF32BV; e += NT) {
            const int r = e / kF32BV, j = e % kF32BV;
            float ks = 0.f;
            for (int c = 0; c < DK; ++c) ks += sk[r * DK + c] * expf(sG[r * DK + c]) * sS[c * kF32BV + j];
            const float vv = r < L ? ld_in(v, ((t0 + r) * H + h) * (int64_t)DV + vb * kF32BV + j) : 0.f;
            sR[e] = sb[r] * (vv - ks);
        }
        __syncthreads();

        // D = T R
        for (int e = tid; e < C * kF32BV; e += NT) {
            const int r = e / kF32BV, j = e % kF32BV;
            float acc = 0.f;
            for (int s = 0; s <= r; ++s) acc += sT[r * LDC + s] * sR[s * kF32BV + j];
            sD[e] = acc;
        }
        __syncthreads();

        // O = Q+ S0 + M D
        for (int e = tid; e < C * kF32BV; e += NT) {
            const int r = e / kF32BV, j = e % kF32BV;
            if (r >= L) continue;
            float acc = 0.f;
            for (int c = 0; c < DK; ++c) acc += sq[r * DK + c] * expf(sG[r * DK + c]) * sS[c * kF32BV + j];
            for (int s = 0; s <= r; ++s) acc += sM[r * LDC + s] * sD[s * kF32BV + j];
            a.o[((t0 + r) * H + h) * (int64_t)DV + vb * kF32BV + j] = acc;
        }
        __syncthreads();

        // S1 = Diag(exp(G_{L-1})) S0 + K'^T D
        for (int e = tid; e < DK * kF32BV; e += NT) {
            const int c = e / kF32BV, j = e % kF32BV;
            const float gl = sG[(L - 1) * DK + c];
            float acc = expf(gl) * sS[e];
            for (int s = 0; s < L; ++s) acc += sk[s * DK + c] * expf(gl - sG[s * DK + c]) * sD[s * kF32BV + j];
            sS[e] = acc;
            // state snapshot after every snap_every full chunks (this thread's own elements)
            const int64_t chunks_done = (t0 - bos) / C + 1;
            if (a.snap && L == C && chunks_done % a.snap_every == 0) {
                const int64_t row = (a.snap_cu ? (int64_t)a.snap_cu[n] : n * a.snap_per_seq) + chunks_done / a.snap_every - 1;
                a.snap[((row * H + h) * DK + c) * (int64_t)DV + vb * kF32BV + j] = acc;
            }
        }
    }
    __syncthreads();
    if (a.sT) {
        for (int e = tid; e < DK * kF32BV; e += NT) {
            const int i = e / kF32BV, j = e % kF32BV;
            a.sT[sbase + (int64_t)i * DV + j] = sS[e];
        }
    }
}


}  // namespace kda
