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
// With one forget gate per head (Gated DeltaNet) alpha is the same for every key row.
//
// Work decomposition: one workgroup of up to 1024 threads per (sequence, head).  A thread
// owns 4 consecutive value columns (one 16-byte vector) of RPT rows, and a wave covers whole
// rows, so every load and store instruction moves contiguous memory.  Small per-thread
// batches (RPT = 4 at d = 128) keep many independent streams in flight, which is what a
// read-once/write-once HBM stream needs (measured on MI355X at N = 256, H = 32, d = 128:
// 1024 threads x 4 rows beat 256 x 16, 512 x 8 and column-sliced workgroups).  The column
// reductions over key rows go through wave shuffles, then a small LDS table.
//
// Small batches: value columns never interact (each column of S is its own chain), so when
// there are few (sequence, head) pairs each one is split over DV / 16 workgroups of 16 columns
// (256 threads, two rows each).  A single sequence with 32 heads then launches 256 workgroups
// instead of 32, one per CU, and its state stays in L2 from step to step.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// DVB: value columns per workgroup (DV, or 16 for the column-split variant)
template <int DK, int DVB>
struct DecodeShape {
    static constexpr int kColThreads = DVB / 4;                   // threads per row
    // the column-split variant is latency-bound (one small block per workgroup): 256 threads of
    // two rows each finish sooner than 512 of one (measured at one sequence, 32 heads)
    static constexpr int kMaxThreads = DVB == 16 ? 256 : 1024;
    static constexpr int kRowGroups = DK < kMaxThreads / kColThreads ? DK : kMaxThreads / kColThreads;
    static constexpr int kThreads = kColThreads * kRowGroups;
    static constexpr int kWaves = kThreads / 64;
    static constexpr int kRowsPerThread = DK / kRowGroups;
    static_assert(DVB % 4 == 0 && kThreads % 64 == 0, "shape");
    static_assert(DK % kRowGroups == 0, "rows must split evenly");
    static_assert(kThreads >= DK, "one thread per key row stages alpha, k, q");
};

template <int DK, int DV, int DVB, typename TI, bool PROLOGUE>
__global__ __launch_bounds__(1024) void decode_kernel(
    const TI* __restrict__ q, const TI* __restrict__ k, const TI* __restrict__ v, const float* __restrict__ g,
    const TI* __restrict__ beta, const float* s_in, float* s_out, float* __restrict__ o, int gate_head,
    float gate_scale) {
    using Sh = DecodeShape<DK, DVB>;
    constexpr int CT = Sh::kColThreads, RG = Sh::kRowGroups, RPT = Sh::kRowsPerThread;
    constexpr int NW = Sh::kWaves;
    constexpr int NCB = DV / DVB;   // workgroups per (sequence, head)
    const int64_t nh = blockIdx.x / NCB;  // sequence * H + head
    const int col0 = (int)(blockIdx.x % NCB) * DVB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c4 = tid % CT;  // owns columns col0 + 4*c4 .. +3
    const int rg = tid / CT;  // owns rows rg, rg + RG, ...

    __shared__ floatx4 s_red[NW][2][CT];  // per wave: partial u and p of each column group
    __shared__ float s_kq[NW];
    __shared__ float s_a[DK], s_k[DK], s_q[DK];
    __shared__ float s_nrm[2][DK / 64 > 0 ? DK / 64 : 1];

    const float* Sin = s_in + nh * (int64_t)DK * DV + col0 + 4 * c4;
    float* Sout = s_out + nh * (int64_t)DK * DV + col0 + 4 * c4;

    // the state loads first: they are the bulk of the traffic.  A large batch streams its state
    // once per step (non-temporal); the column-split small batches keep theirs in L2 from one step
    // to the next (the same workgroup index, hence the same XCD, reads the block it wrote).
    constexpr bool kStream = DVB == DV;
    floatx4 st[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const floatx4* src = reinterpret_cast<const floatx4*>(Sin + (int64_t)(rg + i * RG) * DV);
        st[i] = kStream ? __builtin_nontemporal_load(src) : *src;
    }
    // v and beta of this thread's columns, needed only after the reductions, are requested now so
    // that their latency overlaps the state loads instead of following the reductions
    float vv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vv[j] = ld_in(v, nh * DV + col0 + 4 * c4 + j);
    const float braw = ld_in(beta, nh);
    // alpha, k, q of every key row, one row per thread, shared through LDS
    float kt = 0.f, qt = 0.f;
    if (tid < DK) {
        kt = ld_in(k, nh * DK + tid);
        qt = ld_in(q, nh * DK + tid);
    }
    if (PROLOGUE) {  // fused prologue: unit-length key and query (threads 0 .. DK-1 hold them)
        float sk = kt * kt, sq = qt * qt;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            sk += __shfl_xor(sk, off, 64);
            sq += __shfl_xor(sq, off, 64);
        }
        if (tid < DK && lane == 0) {
            s_nrm[0][wave] = sk;
            s_nrm[1][wave] = sq;
        }
        __syncthreads();
        sk = 0.f;
        sq = 0.f;
#pragma unroll
        for (int wv = 0; wv < (DK + 63) / 64; ++wv) {
            sk += s_nrm[0][wv];
            sq += s_nrm[1][wv];
        }
        kt *= sk > 0.f ? rsqrtf(sk) : 0.f;
        qt *= sq > 0.f ? rsqrtf(sq) : 0.f;
    }
    if (tid < DK) {
        float gv = gate_head ? g[nh] : g[nh * DK + tid];  // one decay per head, or per key channel
        if (PROLOGUE) gv = gate_from_raw(gv, gate_scale);
        s_a[tid] = expf(gv);
        s_k[tid] = kt;
        s_q[tid] = qt;
    }
    __syncthreads();
    float a[RPT], kk[RPT], u[4] = {0.f, 0.f, 0.f, 0.f}, p[4] = {0.f, 0.f, 0.f, 0.f}, kq = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + i * RG;
        a[i] = s_a[r];
        kk[i] = s_k[r];
        const float qq = s_q[r];
        const float ak = a[i] * kk[i], aq = a[i] * qq;
        kq += kk[i] * qq;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u[j] += ak * st[i][j];
            p[j] += aq * st[i][j];
        }
    }
    // reduce over the row groups of this wave (lanes with the same column group) ...
#pragma unroll
    for (int off = CT; off < 64; off <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u[j] += __shfl_xor(u[j], off, 64);
            p[j] += __shfl_xor(p[j], off, 64);
        }
        kq += __shfl_xor(kq, off, 64);
    }
    // ... then over the waves
    if (lane < CT) {
        s_red[wave][0][lane] = floatx4{u[0], u[1], u[2], u[3]};
        s_red[wave][1][lane] = floatx4{p[0], p[1], p[2], p[3]};
        if (lane == 0) s_kq[wave] = kq;
    }
    __syncthreads();
    floatx4 uu = s_red[0][0][c4], pp = s_red[0][1][c4];
    float kqt = s_kq[0];
#pragma unroll
    for (int wv = 1; wv < NW; ++wv) {
        uu += s_red[wv][0][c4];
        pp += s_red[wv][1][c4];
        kqt += s_kq[wv];
    }

    float d[4];
    const float b = PROLOGUE ? sigmoid(braw) : braw;
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = b * (vv[j] - uu[j]);
    if (rg == 0) {
        floatx4 ov;
#pragma unroll
        for (int j = 0; j < 4; ++j) ov[j] = pp[j] + kqt * d[j];
        *reinterpret_cast<floatx4*>(o + nh * DV + col0 + 4 * c4) = ov;
    }

#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        floatx4 ns;
#pragma unroll
        for (int j = 0; j < 4; ++j) ns[j] = a[i] * st[i][j] + kk[i] * d[j];
        floatx4* dst = reinterpret_cast<floatx4*>(Sout + (int64_t)(rg + i * RG) * DV);
        if (kStream) __builtin_nontemporal_store(ns, dst);
        else *dst = ns;
    }
}

template <int DK, int DV, int DVB, typename TI>
void launch_typed(const DecodeArgs& a, hipStream_t s) {
    using Sh = DecodeShape<DK, DVB>;
    const dim3 grid(static_cast<unsigned>(a.N * a.H * (DV / DVB))), block(Sh::kThreads);
    const TI* q = static_cast<const TI*>(a.q);
    const TI* k = static_cast<const TI*>(a.k);
    const TI* v = static_cast<const TI*>(a.v);
    const TI* b = static_cast<const TI*>(a.beta);
    if (a.prologue)
        hipLaunchKernelGGL((decode_kernel<DK, DV, DVB, TI, true>), grid, block, 0, s, q, k, v, a.g, b, a.s_in,
                           a.s_out, a.o, a.gate_head, a.gate_scale);
    else
        hipLaunchKernelGGL((decode_kernel<DK, DV, DVB, TI, false>), grid, block, 0, s, q, k, v, a.g, b, a.s_in,
                           a.s_out, a.o, a.gate_head, a.gate_scale);
}

// (sequence, head) pairs below which each pair is split over 16-column workgroups: with fewer
// than two workgroups per CU the whole-row layout leaves most of the chip idle
constexpr int64_t kSplitBelow = 512;

template <int DK, int DV>
hipError_t launch_shape(const DecodeArgs& a, hipStream_t s) {
    const bool timed = timing_on();
    if (timed) timed_begin(kKernelDecode, s);
    const bool split = DV > 16 && a.N * a.H < kSplitBelow;
    if (a.bf16) {
        if (split) launch_typed<DK, DV, 16, uint16_t>(a, s);
        else launch_typed<DK, DV, DV, uint16_t>(a, s);
    } else {
        if (split) launch_typed<DK, DV, 16, float>(a, s);
        else launch_typed<DK, DV, DV, float>(a, s);
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
