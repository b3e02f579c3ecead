// KDA chunked prefill on the gfx950 matrix cores (bfloat16 storage, d_k = d_v = 128,
// 64-token chunks).
//
// Method ("Kimi K3, explained": "Training in chunks", "The math"): inside a chunk the
// product of per-token decay-and-erase transitions becomes dense products plus one
// unit-lower-triangular inverse, and only the state crosses chunk boundaries.  With
// G[r] = sum_{s<=r} g_s per key channel (restarting at the chunk), S0 the entering
// state and L the chunk length:
//   A[r,s] = beta_r sum_c k_rc k_sc exp(G_rc - G_sc)  (s < r)     T = (I + A)^{-1}
//   M[r,s] =        sum_c q_rc k_sc exp(G_rc - G_sc)  (s <= r)
//   K+ = K * exp(G),  Q+ = Q * exp(G),  K' = K * exp(G_{L-1} - G),  gamma = exp(G_{L-1})
//   D  = T Diag(beta) (V - K+ S0)          (per-token corrections)
//   O  = Q+ S0 + M D
//   S1 = Diag(gamma) S0 + K'^T D
//
// Two kernels:
//  * prep (one workgroup per chunk and head, all chunks in parallel): the decay
//    factors, the gated Gram matrices A and M (fp16 matrix-core products with fp32
//    accumulation), T by blocked forward substitution (fp32 matrix-core products),
//    and the fp16 operand tiles K+, Q+, K'^T, T, M plus fp32 gamma, written to the
//    workspace already in the lane order of the matrix-core operand registers.
//  * state (one workgroup per sequence, head and 16-column value block; value
//    columns never interact): walks the chunks in order with the fp32 state block in
//    registers, four waves each owning 16 tokens of the chunk (R, D, O) and 32 key
//    channels of the state (the update).
//
// Decay factors never overflow: the Gram matrices use per-16-token reference points.
// For rows r in token block i and columns s in block j < i,
//   exp(G_r - G_s) = exp(G_r - P_i) * exp(P_i - P_{j+1}) * exp(P_{j+1} - G_s)
// (P_i = G at the end of block i-1), every factor <= 1.  Inside a diagonal block the
// reference is the block's 8th token; those factors are bounded by the decay of at
// most 8 tokens.  Where that decay exceeds e^10 for some channel (beyond fp16), the
// chunk's diagonal tiles are summed exactly in fp32 with per-pair exponentials instead.
//
// Magnitudes beyond fp16: every value that is rounded to an fp16 operand is checked against
// the fp16 range first (q and k entries, M, T, W in prep; beta*V, the corrections D and the
// state in the state pass).  A (sequence, head, value block) chain that meets such a value is
// recomputed at the end of its state workgroup by the fp32 chunked evaluation, before any of its
// final state is written.
#include <mutex>
#include <type_traits>
#include <vector>

#include "kda.h"
#include "kda_chunk_f32.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;   // tokens per chunk
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int BV = 16;  // value columns per state workgroup
constexpr int NVB = DV / BV;

// chunk record in the workspace (bytes); tiles are 64 lanes x 16 bytes
constexpr int kTile = 1024;
constexpr int kOffW = 0;                  // 16 tiles (token block tb, k-step ks): tb*4+ks
constexpr int kOffQp = 16 * kTile;        // 16 tiles
constexpr int kOffKdT = 32 * kTile;       // 16 tiles (channel block cb, k-step ks): cb*2+ks
constexpr int kOffT = 48 * kTile;         // 6 tiles (row block rb, k-step kb): t6(rb, kb)
constexpr int kOffM = 54 * kTile;         // 6 tiles
constexpr int kOffGamma = 60 * kTile;     // 128 floats
constexpr int kRecord = 60 * kTile + 512; // 61952 bytes (multiple of 256)
constexpr int kWarmAhead = 2;             // chunks of L2 warm-up ahead of the state pass (1, 2, 4 equal; 3, 6, 12 slower)

// T and M are lower triangular: row blocks 0 and 1 have no entries in tokens 32..63 (k-step 1),
// so those two tiles of each are not stored.  Tile index of row block rb, k-step kb:
__host__ __device__ constexpr int t6(int rb, int kb) { return rb < 2 ? rb : 2 * rb - 2 + kb; }

__device__ __forceinline__ floatx4 mfma16x16x32(half8 a, half8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma16x16x4f32(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Sequence bounds and chunk -> workspace slot.
struct SeqMap {
    const int32_t* cu;
    int64_t T_fixed;
    int64_t nck_fixed;  // chunks per sequence when fixed-length
    int64_t N;

    __device__ __forceinline__ void bounds(int64_t n, int64_t& bos, int64_t& eos) const {
        if (cu) {
            bos = cu[n];
            eos = cu[n + 1];
        } else {
            bos = n * T_fixed;
            eos = bos + T_fixed;
        }
    }
    // first slot of sequence n; slots of n are base(n) .. base(n) + chunks(n) - 1
    __device__ __forceinline__ int64_t base(int64_t n) const {
        return cu ? (int64_t)cu[n] / C + n : n * nck_fixed;
    }
    // slot -> (sequence, chunk index); false for a slot no chunk uses
    __device__ __forceinline__ bool locate(int64_t slot, int64_t& n, int64_t& c) const {
        if (!cu) {
            n = slot / nck_fixed;
            c = slot % nck_fixed;
            return n < N;
        }
        int64_t lo = 0, hi = N - 1;
        if (N <= 0 || base(0) > slot) return false;
        while (lo < hi) {  // largest n with base(n) <= slot
            const int64_t mid = (lo + hi + 1) >> 1;
            if (base(mid) <= slot) lo = mid; else hi = mid - 1;
        }
        n = lo;
        c = slot - base(n);
        int64_t bos, eos;
        bounds(n, bos, eos);
        return c * C < eos - bos;
    }
};

__device__ __forceinline__ float bf(uint16_t b) { return bf16_to_f32(b); }

// ------------------------------------------------------------------------------------------
// prep kernel: one workgroup (4 waves) per (slot, head); wave w owns token block w
// ------------------------------------------------------------------------------------------
// The prep kernel keeps log-decays in base-2 units (G * log2(e)), so that every decay factor is
// one hardware exp2 with no scaling multiply.
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// the diagonal-tile factors leave the fp16 range beyond e^10 = 2^(10 log2 e)
constexpr float kDiagBound2 = 10.f * kLog2e;

// 8 consecutive floats of an LDS table (32-byte aligned) as two 128-bit reads
__device__ __forceinline__ void ld8(const float* p, float (&o)[8]) {
    const float4 x = *reinterpret_cast<const float4*>(p), y = *reinterpret_cast<const float4*>(p + 4);
    o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
    o[4] = y.x; o[5] = y.y; o[6] = y.z; o[7] = y.w;
}

// 16-byte aligned, so that the compiler may use 128-bit LDS accesses for the fragment and
// table rows (with the 4-byte alignment of its members it splits every access into 32-bit ones)
struct alignas(16) PrepLds {
    // per key channel, per 16-token block b (all fp32):
    // log-decays in base-2 units; factors are 2^(...) = e^(natural-log value)
    float tot[4][DK];     // D_b = sum of g over block b
    float gmid[4][DK];    // within-block cumulative g at the block's 8th token
    float eP[4][DK];      // exp(P_b), P_b = G at the end of block b-1 (0 for b = 0)
    float etail[4][DK];   // exp(G_{L-1} - P_{b+1}), decay after block b to the chunk end
    float emr[4][DK];     // exp(-gmid_b): diagonal-block row factor = exp(gloc) * emr
    float emc[4][DK];     // exp(gmid_b - D_b): diagonal-block column factor = exp(D_b - gloc) * emc
    float Z[3][DK];       // decay between blocks: pairs (2,0), (3,1): exp(D_1), exp(D_2); (3,0): exp(D_1 + D_2)
    _Float16 kdT[DK][C + 8];       // K'^T (transposed through LDS)
    float AT[C][C + 1];            // A below the block diagonal; T on and above it (see inverse)
    union {
        _Float16 kc[3][4][64][8];  // off-diagonal column operands of blocks 0..2, fragment order
        _Float16 bkT[DK][C + 8];   // Diag(beta) K+ as [channel][token]: B operand of W
    } u;
    int exact_diag;  // some channel's 8-token decay is beyond the fp16 factors
    int range_bad;   // some value rounded to an fp16 operand is beyond the fp16 range
};

// per-unit flag word written by prep: bit 0 = exact diagonal tiles needed (the unit's second
// pass), bit 1 = a value beyond the fp16 range (the chains through the chunk are redone in fp32)
constexpr int kFlagExact = 1;
constexpr int kFlagRange = 2;

__device__ __forceinline__ float dpp_row_shr(float x, int d) {
    // lanes whose source is outside their 16-lane row read 0 (bound_ctrl)
    switch (d) {
    case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
    case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
    case 4: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
    }
}

// T block (i, j), i >= j: diagonal blocks sit on the diagonal of AT, blocks below it are
// stored in the mirrored position above the diagonal (row-major inside the block).
__device__ __forceinline__ float* t_block(PrepLds& L, int i, int j) {
    return i == j ? &L.AT[16 * i][16 * i] : &L.AT[16 * j][16 * i];
}

// A matrix-core product with the operands in swapped order leaves lane (lr, lg) holding four
// consecutive columns 4*lg .. 4*lg+3 of row lr of the 16 x 16 result tile.  Those four values
// are half of one lane's 16-byte operand fragment in a record tile: column block cb (16 wide)
// of a row block lands in k-step cb / 2, fragment lane 16 * (2 * (cb & 1) + lg / 2) + lr, bytes
// 8 * (lg & 1) .. +7.  Returns the byte offset of that half inside the tile.
__device__ __forceinline__ int frag_half_offset(int cb, int lr, int lg) {
    return (16 * (2 * (cb & 1) + (lg >> 1)) + lr) * 16 + 8 * (lg & 1);
}

// bfloat16 element i (0..7) of a packed 8-element row fragment
__device__ __forceinline__ uint32_t bf_elem(const u32x4& v, int i) {
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
    return (i & 1) ? (wv[i >> 1] >> 16) : (wv[i >> 1] & 0xFFFF);
}

// PRO: fused input prologue (raw q, k, beta logits, raw gate inputs); a template parameter so
// that the plain kernel carries none of its code.
// EXACT: the second pass over a unit whose first pass found a decay beyond the fp16 factors; it
// rewrites the record with exact diagonal Gram tiles.  Both passes write the unit's flag word
// (`exact_flags`, one per slot and head).
// One (slot, head) unit; the whole workgroup calls it with the same arguments.  Returns whether
// the unit needs the second pass (always false for the second pass itself, and for a slot that
// no chunk uses).
template <bool PRO, bool EXACT>
__device__ __forceinline__ bool prep_unit(const PrefillArgs& a, const SeqMap& sm, int64_t slot, int h,
                                          int32_t* exact_flags, PrepLds& L) {
    // wave index, wave-uniform (readfirstlane lets the compiler keep it in a scalar register)
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const int H = a.H;
    int64_t n, c;
    if (!sm.locate(slot, n, c)) return false;  // uniform over the workgroup
    int32_t* flag = exact_flags + slot * H + h;
    int64_t bos, eos;
    sm.bounds(n, bos, eos);
    const int64_t t0 = bos + c * C;
    const int Lc = (int)((eos - t0) < C ? (eos - t0) : C);
    unsigned char* rec = static_cast<unsigned char*>(a.ws) + (slot * H + h) * (int64_t)kRecord;
    const uint16_t* q = static_cast<const uint16_t*>(a.q);
    const uint16_t* k = static_cast<const uint16_t*>(a.k);
    const uint16_t* beta = static_cast<const uint16_t*>(a.beta);

    if (threadIdx.x == 0) {
        L.exact_diag = 0;
        L.range_bad = 0;
    }

    // ---- this lane: token r = 16w + lr, channels 32*ks + 8*lg + i (the matrix-core operand
    //      layout).  The inputs are read through descriptors that end at the chunk's last token,
    //      so rows past it read 0 (zero keys, queries and log-decays) with no clamping or selects.
    const int r = 16 * w + lr;
    const bool valid = r < Lc;
    const int64_t rowH = (int64_t)H * DK;  // elements between consecutive tokens
    const int64_t row0 = (t0 * H + h) * (int64_t)DK;
    const uint32_t span = (uint32_t)((Lc - 1) * rowH + DK);  // elements from row 0 to the last row's end
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + row0, span * 2), qrs = make_rsrc(q + row0, span * 2);
    const __amdgpu_buffer_rsrc_t brs = make_rsrc(beta + t0 * H + h, (uint32_t)(((Lc - 1) * H + 1) * 2));
    const int lofs = (int)(r * rowH + 8 * lg);  // this lane's first element
    u32x4 kv[4], qv[4];
    float4 gv[8];
    // g first: the decay scan needs it before anything else (with one gate per head, the
    // token's single log-decay on every channel)
    if (a.gate_head) {
        const __amdgpu_buffer_rsrc_t grs = make_rsrc(a.g + t0 * H + h, (uint32_t)(((Lc - 1) * H + 1) * 4));
        float gs = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(grs, r * H * 4, 0, 0));
        if (PRO) gs = valid ? gate_from_raw(gs, a.gate_scale) : 0.f;
        gs *= kLog2e;
#pragma unroll
        for (int j = 0; j < 8; ++j) gv[j] = make_float4(gs, gs, gs, gs);
    } else {
        const __amdgpu_buffer_rsrc_t grs = make_rsrc(a.g + row0, span * 4);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            gv[2 * ks] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(grs, lofs * 4, 128 * ks, 0));
            gv[2 * ks + 1] =
                __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(grs, lofs * 4, 128 * ks + 16, 0));
        }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        kv[ks] = __builtin_amdgcn_raw_buffer_load_b128(krs, lofs * 2, 64 * ks, 0);
        qv[ks] = __builtin_amdgcn_raw_buffer_load_b128(qrs, lofs * 2, 64 * ks, 0);
    }
    // beta of this lane's token and of the accumulator rows 16w + 4lg + i, requested with the
    // other inputs so that their latency does not open a later phase (0 past the chunk end)
    const uint16_t beta_r = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(brs, r * H * 2, 0, 0);
    uint16_t beta_q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        beta_q[i] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(brs, (16 * w + 4 * lg + i) * H * 2, 0, 0);
    // g as floats in base-2 units (zero past the chunk end); k, q stay packed bf16 until used
    float gl[4][8];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const float4 g0 = gv[2 * ks], g1 = gv[2 * ks + 1];
        gl[ks][0] = g0.x; gl[ks][1] = g0.y; gl[ks][2] = g0.z; gl[ks][3] = g0.w;
        gl[ks][4] = g1.x; gl[ks][5] = g1.y; gl[ks][6] = g1.z; gl[ks][7] = g1.w;
        if (!a.gate_head) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (PRO) gl[ks][i] = valid ? gate_from_raw(gl[ks][i], a.gate_scale) : 0.f;
                gl[ks][i] *= kLog2e;
            }
        }
    }

    // ---- within-block inclusive cumulative sum of g over the 16 tokens (16-lane rows)
#pragma unroll
    for (int d = 1; d < 16; d <<= 1)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i) gl[ks][i] += dpp_row_shr(gl[ks][i], d);
    if (lr == 15 || lr == 7) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int ch = 32 * ks + 8 * lg + i;
                if (lr == 15) L.tot[w][ch] = gl[ks][i];
                else L.gmid[w][ch] = gl[ks][i];
            }
    }
    __syncthreads();

    // ---- per-channel factor tables (threads 0..127: one channel each)
    if (threadIdx.x < DK) {
        const int ch = threadIdx.x;
        const float d0 = L.tot[0][ch], d1 = L.tot[1][ch], d2 = L.tot[2][ch], d3 = L.tot[3][ch];
        const float Pb[4] = {0.f, d0, d0 + d1, d0 + d1 + d2};
        const float Db[4] = {d0, d1, d2, d3};
        const float Ct = d0 + d1 + d2 + d3;
        bool bad = false;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float gm = L.gmid[b][ch];
            L.eP[b][ch] = exp2_hw(Pb[b]);
            L.etail[b][ch] = exp2_hw(Ct - Pb[b] - Db[b]);
            L.emr[b][ch] = exp2_hw(-gm);
            L.emc[b][ch] = exp2_hw(gm - Db[b]);
            // diagonal-block factors are bounded by exp(-gm) (rows) and exp(gm - D_b) (columns);
            // beyond e^10 they leave the fp16 range, and the chunk is redone by the second pass
            bad |= (-gm > kDiagBound2) || (gm - Db[b] > kDiagBound2);
        }
        L.Z[0][ch] = exp2_hw(d1);
        L.Z[1][ch] = exp2_hw(d2);
        L.Z[2][ch] = exp2_hw(d1 + d2);
        if (bad) L.exact_diag = 1;  // benign race: every writer stores 1
    }
    __syncthreads();

    // ---- operand tiles for this lane's token and 32 channels
    // beta of this lane's token (0 past the chunk end) for Diag(beta) K+
    float brow_r = bf(beta_r);
    brow_r = valid ? (PRO ? sigmoid(brow_r) : brow_r) : 0.f;
    // fused prologue: this token's key and query are scaled to unit length (its 128 channels
    // are spread over the 4 lanes lr, lr + 16, lr + 32, lr + 48)
    float inv_k = 1.f, inv_q = 1.f;
    if (PRO) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const uint32_t kw[4] = {kv[ks].x, kv[ks].y, kv[ks].z, kv[ks].w};
            const uint32_t qw[4] = {qv[ks].x, qv[ks].y, qv[ks].z, qv[ks].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float kk = bf((uint16_t)((i & 1) ? (kw[i >> 1] >> 16) : (kw[i >> 1] & 0xFFFF)));
                const float qq = bf((uint16_t)((i & 1) ? (qw[i >> 1] >> 16) : (qw[i >> 1] & 0xFFFF)));
                sk += kk * kk;
                sq += qq * qq;
            }
        }
        sk += __shfl_xor(sk, 16, 64);
        sq += __shfl_xor(sq, 16, 64);
        sk += __shfl_xor(sk, 32, 64);
        sq += __shfl_xor(sq, 32, 64);
        inv_k = sk > 0.f ? rsqrtf(sk) : 0.f;
        inv_q = sq > 0.f ? rsqrtf(sq) : 0.f;
    }
    // Second pass: some channel decays so fast over 8 tokens that the half-block factors of the
    // diagonal Gram tile (w, w) would leave the fp16 range, so that tile takes its exact fp32
    // sums instead, sum_c k_rc k_sc exp(G_rc - G_sc) (q_rc in place of k_rc for M) with
    // G_rc - G_sc <= 0.  The lanes of row r sum their 8 channels of each k-step for every column
    // s of the block (row s sits in lane s of the same 16-lane row), add their partial sums, and
    // keep their own four columns.
    float exact_pmax = 0.f;
    if (EXACT) {
        float accA[4] = {0.f, 0.f, 0.f, 0.f}, accM[4] = {0.f, 0.f, 0.f, 0.f};  // columns 4*lg + j
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float kk[8], qq[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                kk[i] = bf(bf_elem(kv[ks], i)) * inv_k;
                qq[i] = bf(bf_elem(qv[ks], i)) * inv_q;
            }
#pragma unroll 1
            for (int s2 = 0; s2 < 16; ++s2) {
                float pa = 0.f, pm = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float ksv = __shfl(kk[i], 16 * lg + s2, 64), gs = __shfl(gl[ks][i], 16 * lg + s2, 64);
                    const float e = exp2_hw(fminf(gl[ks][i] - gs, 0.f)) * ksv;
                    pa += kk[i] * e;
                    pm += qq[i] * e;
                }
                pa += __shfl_xor(pa, 16, 64);
                pa += __shfl_xor(pa, 32, 64);
                pm += __shfl_xor(pm, 16, 64);
                pm += __shfl_xor(pm, 32, 64);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool mine = s2 == 4 * lg + j;
                    accA[j] += mine ? pa : 0.f;
                    accM[j] += mine ? pm : 0.f;
                }
            }
        }
        // accM holds M[r][16w + 4lg + j]: the layout of a swapped-operand product (see
        // frag_half_offset), stored straight into the record
        half4 mh;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int s2 = 4 * lg + j;
            L.AT[r][16 * w + s2] = (s2 < lr) ? brow_r * accA[j] : 0.f;
            mh[j] = (_Float16)((s2 <= lr) ? accM[j] : 0.f);
            exact_pmax = fmaxf(exact_pmax, __builtin_fabsf((float)mh[j]));
        }
        __builtin_nontemporal_store(mh, reinterpret_cast<half4*>(rec + kOffM + t6(w, w >> 1) * kTile + frag_half_offset(w, lr, lg)));
    }
    half8 KR[4], QR[4], BKp[4];
    floatx4 diagA = {0.f, 0.f, 0.f, 0.f}, diagM = {0.f, 0.f, 0.f, 0.f};  // tile (w, w)
    // largest |q|, |k| entry of this lane: the decay-folded operands are bounded by it (times
    // e^10 for the diagonal-tile factors, whose overflow shows up in M and T below)
    float qkmax = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        half8 kp, qp, kc, krd, qrd, kcd;
        const uint32_t kw[4] = {kv[ks].x, kv[ks].y, kv[ks].z, kv[ks].w};
        const uint32_t qw[4] = {qv[ks].x, qv[ks].y, qv[ks].z, qv[ks].w};
        // this k-step's 8 channels of the factor tables, read together
        const int c0 = 32 * ks + 8 * lg;
        float ttot[8], tep[8], ttail[8], tmr[8], tmc[8];
        ld8(&L.tot[w][c0], ttot);
        ld8(&L.eP[w][c0], tep);
        ld8(&L.etail[w][c0], ttail);
        ld8(&L.emr[w][c0], tmr);
        ld8(&L.emc[w][c0], tmc);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int ch = c0 + i;
            const float gloc = gl[ks][i];
            const uint32_t kb16 = (i & 1) ? (kw[i >> 1] >> 16) : (kw[i >> 1] & 0xFFFF);
            const uint32_t qb16 = (i & 1) ? (qw[i >> 1] >> 16) : (qw[i >> 1] & 0xFFFF);
            const float kk = bf(kb16) * inv_k, qq = bf(qb16) * inv_q;
            qkmax = fmaxf(qkmax, fmaxf(__builtin_fabsf(kk), __builtin_fabsf(qq)));
            const float eloc = exp2_hw(gloc);            // exp(G_r - P_w)          <= 1
            const float ecol = exp2_hw(ttot[i] - gloc);  // exp(P_{w+1} - G_r)      <= 1
            const float kl = kk * eloc, ql = qq * eloc, kcf = kk * ecol;
            kp[i] = (_Float16)(kl * (tep[i] * brow_r));
            qp[i] = (_Float16)(ql * tep[i]);
            L.kdT[ch][r] = (_Float16)(kcf * ttail[i]);
            KR[ks][i] = (_Float16)kl;
            QR[ks][i] = (_Float16)ql;
            kc[i] = (_Float16)kcf;
            krd[i] = (_Float16)(kl * tmr[i]);
            qrd[i] = (_Float16)(ql * tmr[i]);
            kcd[i] = (_Float16)(kcf * tmc[i]);
        }
        // diagonal Gram tile (w, w): this lane's operands are both the row and the column
        // fragments, so it accumulates k-step by k-step with nothing exchanged
        if (!EXACT) {
            diagA = mfma16x16x32(krd, kcd, diagA);
            diagM = mfma16x16x32(kcd, qrd, diagM);  // swapped: lane holds M[r][16w + 4lg + i]
        }
        BKp[ks] = kp;  // Diag(beta) K+, consumed by W after T is known
        __builtin_nontemporal_store(qp, reinterpret_cast<half8*>(rec + kOffQp + (w * 4 + ks) * kTile + lane * 16));
        if (w < 3) *reinterpret_cast<half8*>(&L.u.kc[w][ks][lane][0]) = kc;
        // keep the per-channel table reads of one k-step from being hoisted above the previous
        // one (bounds register pressure)
        asm volatile("" ::: "memory");
    }

    // ---- gated Gram matrices of row block w: first the diagonal tile (w, w) from this lane's
    //      own operands, then (after the column operands of the other blocks are visible) the
    //      tiles (w, j < w)
    float brow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rr = 16 * w + 4 * lg + i;
        const float bv = bf(beta_q[i]);
        brow[i] = rr < Lc ? (PRO ? sigmoid(bv) : bv) : 0.f;
    }
    // largest magnitude among the M, T and W values this lane rounds to fp16 (a running maximum;
    // a NaN leaves it unchanged and stays NaN in every result, as on the fp32 path)
    float pmax = exact_pmax;
    unsigned char* mrec = rec + kOffM;
    if (!EXACT) {  // the second pass has its exact tiles in place already
        // A accumulator: column s = lr of block w, rows 4*lg + i of block w
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = 16 * w + 4 * lg + i, ss = 16 * w + lr;
            L.AT[rr][ss] = (ss < rr) ? brow[i] * diagA[i] : 0.f;
        }
        // M accumulator (swapped operands): row r = 16w + lr, columns 16w + 4lg + i
        half4 mh;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float mv = (4 * lg + i <= lr) ? diagM[i] : 0.f;
            pmax = fmaxf(pmax, __builtin_fabsf(mv));
            mh[i] = (_Float16)mv;
        }
        __builtin_nontemporal_store(mh, reinterpret_cast<half4*>(mrec + t6(w, w >> 1) * kTile + frag_half_offset(w, lr, lg)));
    }
    // the stored M tiles of row blocks 0 and 2 also span the (zero) block to the right of the diagonal
    if (!(w & 1))
        __builtin_nontemporal_store(half4{(_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f}, reinterpret_cast<half4*>(mrec + t6(w, w >> 1) * kTile + frag_half_offset(w + 1, lr, lg)));
    __syncthreads();
    if (w == 0) {
        // ---- T = (I + A)^{-1}, diagonal 16x16 blocks by forward substitution: wave 0 inverts all
        //      four at once (lanes 16q .. 16q+15: block q, lane = column) while waves 1..3 form the
        //      off-diagonal Gram tiles; T_qq overwrites A_qq (no longer needed)
        const int j = lr, o = 16 * lg;
        float tc[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            float acc = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < rr; ++s2) acc += L.AT[o + rr][o + s2] * tc[s2];
            tc[rr] = rr < j ? 0.f : (rr == j ? 1.f : -acc);
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) L.AT[o + rr][o + j] = tc[rr];
    } else {
        for (int j = 0; j < w; ++j) {
            floatx4 accA = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
            const int zi = (w - j == 2) ? (w == 2 ? 0 : 1) : 2;  // Z table of pair (w, j) when j + 1 < w
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                half8 bcol = *reinterpret_cast<const half8*>(&L.u.kc[j][ks][lane][0]);
                if (j + 1 < w) {  // scale by exp(P_w - P_{j+1}), the decay of blocks j+1 .. w-1
                    float z[8];
                    ld8(&L.Z[zi][32 * ks + 8 * lg], z);
#pragma unroll
                    for (int i = 0; i < 8; ++i) bcol[i] = (_Float16)((float)bcol[i] * z[i]);
                }
                accA = mfma16x16x32(KR[ks], bcol, accA);
                accM = mfma16x16x32(bcol, QR[ks], accM);  // swapped: lane holds M[16w + lr][16j + 4lg + i]
            }
            half4 mh;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 16 * w + 4 * lg + i, ss = 16 * j + lr;
                L.AT[rr][ss] = brow[i] * accA[i];
                pmax = fmaxf(pmax, __builtin_fabsf(accM[i]));
                mh[i] = (_Float16)accM[i];
            }
            __builtin_nontemporal_store(mh, reinterpret_cast<half4*>(mrec + t6(w, j >> 1) * kTile + frag_half_offset(j, lr, lg)));
        }
    }
    __syncthreads();
    // off-diagonal blocks: T_ij = -T_ii * (sum_{m=j}^{i-1} A_im T_mj).  Wave j forms column j
    //      (T_{j+1,j}, T_{j+2,j}, T_{j+3,j} in turn), which needs only earlier blocks of the same
    //      column, so no wave waits for another.  The column's blocks stay in registers in the
    //      accumulator layout (lane: column lr, rows 4*lg + e); with the contraction index ordered
    //      k = 4*lg + step, that layout is the right-hand operand of the next product as it is.
    if (w < 3) {
        floatx4 tcol[4];  // T_{j+d, j}, d = 0 .. 3 - j
        const float* tjj = t_block(L, w, w);
#pragma unroll
        for (int e = 0; e < 4; ++e) tcol[0][e] = tjj[(4 * lg + e) * (C + 1) + lr];
#pragma unroll
        for (int dist = 1; dist < 4; ++dist) {
            const int i = w + dist;
            if (i < 4) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int mm = 0; mm < dist; ++mm) {  // m = w + mm
                    const float* ap = &L.AT[16 * i + lr][16 * (w + mm) + 4 * lg];
#pragma unroll
                    for (int kq = 0; kq < 4; ++kq) acc = mfma16x16x4f32(ap[kq], tcol[mm][kq], acc);
                }
                const float* tp = t_block(L, i, i) + lr * (C + 1) + 4 * lg;
                floatx4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kq = 0; kq < 4; ++kq) t = mfma16x16x4f32(tp[kq], acc[kq], t);
                tcol[dist] = -t;
                float* dst = t_block(L, i, w);
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[(4 * lg + e) * (C + 1) + lr] = -t[e];
            }
        }
    }
    // ---- meanwhile the waves with the shorter columns write gamma and the 16 K'^T operand tiles
    //      (wave 3: gamma and tiles 0..11, wave 2: tiles 12..15)
    if (w == 3) {
        float* gam = reinterpret_cast<float*>(rec + kOffGamma);
#pragma unroll
        for (int c2 = 0; c2 < DK / 64; ++c2) {
            const int ch = 64 * c2 + lane;
            gam[ch] = exp2_hw(L.tot[0][ch] + L.tot[1][ch] + L.tot[2][ch] + L.tot[3][ch]);
        }
    }
    if (w >= 2) {
        const int t0k = w == 3 ? 0 : 12, t1k = w == 3 ? 12 : 16;
        for (int t = t0k; t < t1k; ++t) {
            const int cb = t >> 1, ks = t & 1;
            const half8 kd = *reinterpret_cast<const half8*>(&L.kdT[16 * cb + lr][32 * ks + 8 * lg]);
            __builtin_nontemporal_store(kd, reinterpret_cast<half8*>(rec + kOffKdT + t * kTile + lane * 16));
        }
    }

    // ---- W's right-hand operand, Diag(beta) K+, staged transposed ([channel][token]) so that
    //      each matrix-core B fragment (8 consecutive tokens of one channel) is one 16-byte read.
    //      It shares the union with the off-diagonal column operands, dead since the barrier
    //      before the inverse, and the barrier below makes it visible.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int i = 0; i < 8; ++i) L.u.bkT[32 * ks + 8 * lg + i][r] = BKp[ks][i];
    __syncthreads();  // T complete; Diag(beta) K+ staged

    // ---- T rows of block w: the record's T tiles (w, kb) in operand order, and the right-hand
    //      operand of W^T below (zero above the diagonal)
    half8 ta[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int col = 32 * kb + 8 * lg + i, cb = col >> 4;
            const float val = cb <= w ? t_block(L, w, cb)[lr * (C + 1) + (col & 15)] : 0.f;
            pmax = fmaxf(pmax, __builtin_fabsf(val));
            ta[kb][i] = (_Float16)val;
        }
    __builtin_nontemporal_store(ta[0], reinterpret_cast<half8*>(rec + kOffT + t6(w, 0) * kTile + lane * 16));
    if (w >= 2) __builtin_nontemporal_store(ta[1], reinterpret_cast<half8*>(rec + kOffT + t6(w, 1) * kTile + lane * 16));

    // ---- W = T Diag(beta) K+ (64 x 128), rows of token block w, as W^T = (Diag(beta) K+)^T T^T
    //      tiles: each lane then holds 4 consecutive channels of its token row and stores them
    //      straight into the record (see frag_half_offset)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            acc = mfma16x16x32(*reinterpret_cast<const half8*>(&L.u.bkT[16 * cb + lr][32 * kb + 8 * lg]), ta[kb],
                               acc);
        half4 wh;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pmax = fmaxf(pmax, __builtin_fabsf(acc[i]));
            wh[i] = (_Float16)acc[i];
        }
        __builtin_nontemporal_store(wh, reinterpret_cast<half4*>(rec + kOffW + (w * 4 + (cb >> 1)) * kTile + frag_half_offset(cb, lr, lg)));
    }
    if (!(qkmax < 32768.f) || !(pmax < 65504.f)) L.range_bad = 1;  // benign race: every writer stores 1
    __syncthreads();
    if (threadIdx.x == 0) *flag = (L.exact_diag ? kFlagExact : 0) | (L.range_bad ? kFlagRange : 0);
    return !EXACT && L.exact_diag != 0;  // final since the factor tables' barrier
}

// One workgroup (4 waves) per (slot, head), heads fastest: workgroups that run at the same time
// read neighbouring token rows and write neighbouring records.  A unit that needs exact diagonal
// tiles takes its second pass in the same workgroup.
template <bool PRO>
__global__ __launch_bounds__(256, 2) void prep_kernel(PrefillArgs a, SeqMap sm, int32_t* exact_flags) {
    __shared__ PrepLds L;
    const int64_t unit = blockIdx.x, slot = unit / a.H;
    const int h = (int)(unit % a.H);
    if (prep_unit<PRO, false>(a, sm, slot, h, exact_flags, L)) {  // uniform over the workgroup
        __syncthreads();  // the second pass rewrites the LDS the first still reads at its end
        prep_unit<PRO, true>(a, sm, slot, h, exact_flags, L);
    }
}

// ------------------------------------------------------------------------------------------
// state kernel: one workgroup per (sequence, head, 16-column value block)
// ------------------------------------------------------------------------------------------
// Per chunk, with S0 the entering state block (128 x 16) and U = T Diag(beta) V:
//     D  = U - W S0                 (the corrections; W = T Diag(beta) K+ from the prep kernel)
//     O  = Q+ S0 + M D
//     S1 = Diag(gamma) S0 + K'^T D
// Only W S0 -> D -> K'^T D -> S1 is on the sequential path; U and Q+ S0 do not depend on the
// state.  Compute wave w (0..3) owns token block w (D, O) and key-channel blocks 2w, 2w+1 of
// the state (update).  Two LDS exchanges per chunk: D (all tokens, for M D and K'^T D) and S1
// (all channels, for the next chunk's products).  beta*V of the next chunk is staged in LDS,
// in the matrix-core B layout, in the same pass.

// Operands of one chunk as held by one lane of compute wave w.
struct ChunkFrags {
    half8 wt[4], qp[4];   // W, Q+ rows of token block w, k-steps 0..3
    half8 kd[2][2];       // K'^T rows of channel blocks 2w, 2w+1, k-steps 0..1
    half8 tt[2], mm[2];   // T, M rows of token block w, k-steps 0..1 (k-step 1 is zero for w < 2)
};

__device__ __forceinline__ half8 as_half8(u32x4 x) { return __builtin_bit_cast(half8, x); }

// The operand loads of one chunk in four groups.  Each wave-wide load costs the CU's address
// unit about as much whatever its width, and a wave stalls at issue when that unit is busy, so
// the groups are issued at three points spread over the previous chunk's compute rather than
// back to back: W before X, Q+ after it, and T, M and K'^T after the first barrier (measured on
// MI355X; any group moved into the stretch before the first barrier, or interleaved one load per
// matrix-core step, made the pass slower).
__device__ __forceinline__ void load_group(ChunkFrags& f, __amdgpu_buffer_rsrc_t rr, int g, int w, int lane) {
    const int lo = lane * 16;
    if (g == 0) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            f.wt[ks] = as_half8(__builtin_amdgcn_raw_buffer_load_b128(rr, lo, kOffW + (w * 4 + ks) * kTile, 0));
    } else if (g == 1) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            f.qp[ks] = as_half8(__builtin_amdgcn_raw_buffer_load_b128(rr, lo, kOffQp + (w * 4 + ks) * kTile, 0));
    } else if (g == 2) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                f.kd[t][ks] = as_half8(
                    __builtin_amdgcn_raw_buffer_load_b128(rr, lo, kOffKdT + ((2 * w + t) * 2 + ks) * kTile, 0));
    } else {
        f.tt[0] = as_half8(__builtin_amdgcn_raw_buffer_load_b128(rr, lo, kOffT + t6(w, 0) * kTile, 0));
        f.mm[0] = as_half8(__builtin_amdgcn_raw_buffer_load_b128(rr, lo, kOffM + t6(w, 0) * kTile, 0));
        if (w >= 2) {  // rows of token blocks 0, 1 have no entries in tokens 32..63 (not stored)
            f.tt[1] = as_half8(__builtin_amdgcn_raw_buffer_load_b128(rr, lo, kOffT + t6(w, 1) * kTile, 0));
            f.mm[1] = as_half8(__builtin_amdgcn_raw_buffer_load_b128(rr, lo, kOffM + t6(w, 1) * kTile, 0));
        }
    }
}

__device__ __forceinline__ void load_chunk(ChunkFrags& f, const unsigned char* rec, int w, int lane) {
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(rec, kRecord);
#pragma unroll
    for (int g = 0; g < 4; ++g) load_group(f, rr, g, w, lane);
}

// Warm L2 with the chunk record `rec` ahead of its use: each (sequence, head) has NVB state
// workgroups reading the same record, so workgroup vb touches every NVB-th 128-byte line of
// it, one line per lane, with 4-byte direct-to-LDS loads into a dummy slot (no registers are
// written and nothing waits on them).
constexpr int kLinesPerRecord = (kRecord + 127) / 128;

__device__ __forceinline__ void warm_l2(const unsigned char* rec, int vb, int lane,
                                        __attribute__((address_space(3))) void* dummy) {
    for (int base = 0; base * NVB < kLinesPerRecord; base += 64) {
        int line = vb + NVB * (base + lane);
        if (line >= kLinesPerRecord) line = kLinesPerRecord - 1;
        __builtin_amdgcn_global_load_lds(rec + (size_t)line * 128, dummy, 4, 0, 0);
    }
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations (lgkmcnt)
// but not for outstanding global loads, so operand prefetches and L2 warm-ups stay in flight
// across it (a full __syncthreads() fence would drain them).  The empty asm statements keep
// the compiler from moving memory operations across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // gfx9 encoding: vmcnt/expcnt at max, lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

struct StateLds {
    alignas(16) _Float16 S[BV][DK + 8];      // state block as B operand: [column][channel]
    alignas(16) _Float16 D[BV][C + 8];       // corrections as B operand: [column][token]
    alignas(16) _Float16 BVs[2][BV][C + 8];  // beta*V as B operand, double-buffered by chunk parity
    alignas(16) float gam[2][DK];            // gamma, double-buffered by chunk parity
    alignas(16) float Ost[4][16][20];        // per-wave output tile, transposed to token rows
    alignas(16) float warm_dummy[64];        // sink of the L2 warm-up loads (never read)
    int bad[8];                              // per wave: met a value beyond the fp16 range
};

// v, beta and gamma of one chunk as loaded by the staging wave: lane l covers token
// 32*j + l/2 (j = 0, 1), value columns 8*(l&1) .. +7 of this workgroup's block, and gamma
// channels 2l, 2l+1.  Descriptors end at the chunk's last token, so later tokens read 0.
struct StageRegs {
    u32x4 v[2];
    uint32_t b[2];
    uint32_t g[2];
};

// Token half J (tokens 32 J .. 32 J + 31) of a chunk's staging; half 0 also takes gamma.
template <int J>
__device__ __forceinline__ void stage_load(StageRegs& r, const uint16_t* v, const uint16_t* beta,
                                           const unsigned char* rec, int64_t t0, int Lc, int H, int h, int vb,
                                           int lane) {
    const int64_t rowv = (int64_t)H * DV;
    const __amdgpu_buffer_rsrc_t vrs =
        make_rsrc(v + (t0 * H + h) * (int64_t)DV + vb * BV, (uint32_t)(((Lc - 1) * rowv + BV) * 2));
    const __amdgpu_buffer_rsrc_t brs = make_rsrc(beta + t0 * H + h, (uint32_t)(((Lc - 1) * H + 1) * 2));
    const int tok = 32 * J + (lane >> 1);
    r.v[J] = __builtin_amdgcn_raw_buffer_load_b128(vrs, (int)((tok * rowv + 8 * (lane & 1)) * 2), 0, 0);
    r.b[J] = __builtin_amdgcn_raw_buffer_load_b16(brs, tok * H * 2, 0, 0);
    if (J == 0) {
        const __amdgpu_buffer_rsrc_t grs = make_rsrc(rec + kOffGamma, DK * 4);
        r.g[0] = __builtin_amdgcn_raw_buffer_load_b32(grs, lane * 8, 0, 0);
        r.g[1] = __builtin_amdgcn_raw_buffer_load_b32(grs, lane * 8 + 4, 0, 0);
    }
}

// amax: the largest |beta*v| staged so far by this lane (a running maximum; a NaN leaves it
// unchanged and stays NaN in every result, as on the fp32 path)
template <int J>
__device__ __forceinline__ void stage_store(StateLds& L, int buf, const StageRegs& r, int lane, bool beta_logits,
                                            float& amax) {
    const int tok = 32 * J + (lane >> 1);
    const float bt = beta_logits ? sigmoid(bf((uint16_t)r.b[J])) : bf((uint16_t)r.b[J]);
    const uint32_t words[4] = {r.v[J].x, r.v[J].y, r.v[J].z, r.v[J].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint16_t bits = (uint16_t)((e & 1) ? (words[e >> 1] >> 16) : (words[e >> 1] & 0xFFFF));
        const float x = bt * bf(bits);
        amax = fmaxf(amax, __builtin_fabsf(x));
        L.BVs[buf][8 * (lane & 1) + e][tok] = (_Float16)x;
    }
    if (J == 0) {
        L.gam[buf][2 * lane] = __uint_as_float(r.g[0]);
        L.gam[buf][2 * lane + 1] = __uint_as_float(r.g[1]);
    }
}

// Output rows of one chunk: the accumulator tile (lane = column, 4 rows) goes through LDS so
// that each lane stores 4 consecutive columns of one token row (one 16-byte store per lane);
// the descriptor ends at the chunk's last token.
__device__ __forceinline__ void store_o(StateLds& L, floatx4 O, float* obase, int Lc, int H, int w, int lane) {
    const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) L.Ost[w][4 * lg + i][lr] = O[i];
    const floatx4 row = *reinterpret_cast<const floatx4*>(&L.Ost[w][lane >> 2][4 * (lane & 3)]);
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(obase, (uint32_t)(((Lc - 1) * (int64_t)H * DV + BV) * 4));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, row), ors,
                                           (int)((((16 * w + (lane >> 2)) * (int64_t)H * DV) + 4 * (lane & 3)) * 4),
                                           0, 0);
}

// One chunk: operands `cur` (the next chunk's are already requested).  Returns this wave's
// output rows; the caller stores them after issuing the following prefetch (loads and stores
// share one in-order counter, so an early store would delay every later operand wait).
// amax: running maximum of |D| and |S1| over this lane's values (see stage_store)
__device__ __forceinline__ floatx4 state_chunk(StateLds& L, const ChunkFrags& cur, ChunkFrags& nxt,
                                               const unsigned char* nrec, bool has_next, int buf, floatx4 (&Sf)[2],
                                               int w, int lane, float& amax) {
    const int lr = lane & 15, lg = lane >> 4;
    const __amdgpu_buffer_rsrc_t nr = make_rsrc(nrec, kRecord);  // a valid record even when !has_next
    if (has_next) load_group(nxt, nr, 0, w, lane);
    __builtin_amdgcn_sched_barrier(0);
    half8 sb[4], bv[2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) sb[ks] = *reinterpret_cast<const half8*>(&L.S[lr][32 * ks + 8 * lg]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) bv[kb] = *reinterpret_cast<const half8*>(&L.BVs[buf][lr][32 * kb + 8 * lg]);
    // sequential path: X = W S0
    floatx4 X = {0.f, 0.f, 0.f, 0.f}, Y = {0.f, 0.f, 0.f, 0.f}, U = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) X = mfma16x16x32(cur.wt[ks], sb[ks], X);
    __builtin_amdgcn_sched_barrier(0);
    if (has_next) load_group(nxt, nr, 1, w, lane);
    __builtin_amdgcn_sched_barrier(0);
    // state-independent: U = T beta V, Y = Q+ S0
    U = mfma16x16x32(cur.tt[0], bv[0], U);
    if (w >= 2) U = mfma16x16x32(cur.tt[1], bv[1], U);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) Y = mfma16x16x32(cur.qp[ks], sb[ks], Y);
    __builtin_amdgcn_sched_barrier(0);
    half4 dh;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float d = U[i] - X[i];
        amax = fmaxf(amax, __builtin_fabsf(d));
        dh[i] = (_Float16)d;
    }
    *reinterpret_cast<half4*>(&L.D[lr][16 * w + 4 * lg]) = dh;
    lds_barrier();

    if (has_next) load_group(nxt, nr, 3, w, lane);  // T, M
    if (has_next) load_group(nxt, nr, 2, w, lane);  // K'^T
    __builtin_amdgcn_sched_barrier(0);
    half8 db[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) db[kb] = *reinterpret_cast<const half8*>(&L.D[lr][32 * kb + 8 * lg]);
    // sequential path: S1 = Diag(gamma) S0 + K'^T D for this wave's 32 channels
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const floatx4 gm = *reinterpret_cast<const floatx4*>(&L.gam[buf][16 * (2 * w + t) + 4 * lg]);
        floatx4 acc = gm * Sf[t];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) acc = mfma16x16x32(cur.kd[t][kb], db[kb], acc);
        Sf[t] = acc;
        half4 hv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            amax = fmaxf(amax, __builtin_fabsf(acc[i]));
            hv[i] = (_Float16)acc[i];
        }
        *reinterpret_cast<half4*>(&L.S[lr][16 * (2 * w + t) + 4 * lg]) = hv;
    }
    // O = Q+ S0 + M D
    floatx4 O = Y;
    O = mfma16x16x32(cur.mm[0], db[0], O);
    if (w >= 2) O = mfma16x16x32(cur.mm[1], db[1], O);
    lds_barrier();
    return O;
}

// Waves 0..3 compute.  Waves 4 and 5 stage beta*V of the next chunk in LDS, half the tokens
// each (wave 5 also gamma), and wave 4 warms L2 ahead of the compute waves.  Outstanding memory
// operations are counted per wave in issue order, so the warm-up's long-latency loads and the
// staging loads stay out of the compute waves' counters.
constexpr int kStateThreads = 384;

// uflags: prep's flag word per (slot, head).  A chain that met a value beyond the fp16 range is
// recomputed from its inputs by the fp32 chunked evaluation (f32_chain, 32-token chunks) in the
// same workgroup, before any of its final state is written (so an in-place state_in is intact);
// its LDS is the kernel's dynamic shared memory.
constexpr int kRedoChunk = 32;

__global__ __launch_bounds__(kStateThreads) void state_kernel(PrefillArgs a, SeqMap sm, const int32_t* uflags) {
    __shared__ StateLds L;
    extern __shared__ float redo_lds[];
    // wave index, wave-uniform (readfirstlane lets the compiler keep it in a scalar register)
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const int H = a.H;
    float amax = 0.f;  // largest magnitude this lane rounds to fp16 (beta*v; corrections, state)

    // workgroup -> (sequence, head, value block); the 8 value blocks of a (sequence, head)
    // land on one XCD (workgroups are dealt to the 8 XCDs round-robin) so they share its L2
    const int64_t L_id = blockIdx.x;
    const int64_t nh_total = sm.N * H;
    int64_t nh;
    int vb;
    if ((nh_total & 7) == 0) {
        const int64_t xcd = L_id & 7, u = L_id >> 3;
        vb = (int)(u & 7);
        nh = xcd + 8 * (u >> 3);
    } else {
        vb = (int)(L_id % NVB);
        nh = L_id / NVB;
    }
    const int64_t n = nh / H;
    const int h = (int)(nh % H);
    int64_t bos, eos;
    sm.bounds(n, bos, eos);
    const int64_t nchunks = (eos - bos + C - 1) / C;
    const int64_t slot0 = sm.base(n);
    const uint16_t* v = static_cast<const uint16_t*>(a.v);
    const uint16_t* beta = static_cast<const uint16_t*>(a.beta);
    const int64_t sbase = nh * (int64_t)DK * DV + vb * BV;
    const unsigned char* ws = static_cast<const unsigned char*>(a.ws);
    auto rec_of = [&](int64_t c) { return ws + ((slot0 + c) * H + h) * (int64_t)kRecord; };
    // After every chunk: each wave publishes whether it met a value beyond the fp16 range (and
    // the compute waves whether prep flagged one of this chain's chunks), one barrier, then the
    // compute waves take the decision together.
    auto publish_flag = [&](bool bad) {
        const bool any = __ballot(bad) != 0;
        if (lane == 0) L.bad[w] = any ? 1 : 0;
        lds_barrier();
    };
    auto len_of = [&](int64_t c) {
        const int64_t t = eos - (bos + c * C);
        return (int)(t < C ? t : C);
    };

    if (w >= 4) {
        // helper waves: chunk c+1's beta*V (wave 5 tokens 0..31 and gamma, wave 4 tokens 32..63)
        // goes to LDS between the two barriers of chunk c, from registers loaded one chunk
        // earlier; chunk c+2's loads are issued right after, away from the compute waves'
        // operand loads before the first barrier.  Wave 4 also warms L2 with the record
        // kWarmAhead chunks ahead.  Both take part in the compute waves' barriers (one before
        // the loop, two per chunk).
        auto* dummy = reinterpret_cast<__attribute__((address_space(3))) void*>(
            reinterpret_cast<uintptr_t>(&L.warm_dummy[0]));
        const bool warm = w == 4;
        auto run = [&](auto half) {
            constexpr int J = decltype(half)::value;
            StageRegs ra, rb;
            if (warm)
                for (int64_t c = 1; c <= kWarmAhead && c < nchunks; ++c) warm_l2(rec_of(c), vb, lane, dummy);
            if (nchunks > 0) {
                stage_load<J>(ra, v, beta, rec_of(0), bos, len_of(0), H, h, vb, lane);
                stage_store<J>(L, 0, ra, lane, a.prologue, amax);
            }
            if (nchunks > 1) stage_load<J>(rb, v, beta, rec_of(1), bos + C, len_of(1), H, h, vb, lane);
            lds_barrier();
            for (int64_t c = 0; c < nchunks; c += 2) {
                lds_barrier();
                if (c + 1 < nchunks) stage_store<J>(L, 1, rb, lane, a.prologue, amax);
                if (c + 2 < nchunks)
                    stage_load<J>(ra, v, beta, rec_of(c + 2), bos + (c + 2) * C, len_of(c + 2), H, h, vb, lane);
                if (warm && c + 1 + kWarmAhead < nchunks) warm_l2(rec_of(c + 1 + kWarmAhead), vb, lane, dummy);
                lds_barrier();
                if (c + 1 >= nchunks) break;
                lds_barrier();
                if (c + 2 < nchunks) stage_store<J>(L, 0, ra, lane, a.prologue, amax);
                if (c + 3 < nchunks)
                    stage_load<J>(rb, v, beta, rec_of(c + 3), bos + (c + 3) * C, len_of(c + 3), H, h, vb, lane);
                if (warm && c + 2 + kWarmAhead < nchunks) warm_l2(rec_of(c + 2 + kWarmAhead), vb, lane, dummy);
                lds_barrier();
            }
            __builtin_amdgcn_s_waitcnt(0);  // no direct-to-LDS write may outlive the workgroup
            publish_flag(!(amax < 65504.f));
        };
        if (w == 4) run(std::integral_constant<int, 1>{});
        else run(std::integral_constant<int, 0>{});
        if (L.bad[0] | L.bad[1] | L.bad[2] | L.bad[3] | L.bad[4] | L.bad[5]) {
            PrefillArgs r = a;  // 64-token snapshot intervals are twice as many 32-token chunks
            r.snap_every = a.snap_every * (C / kRedoChunk);
            f32_chain<DK, DV, kRedoChunk, kStateThreads, uint16_t>(r, n, h, vb, redo_lds);
        }
        return;
    }

    // fp32 state rows owned by this wave: channel blocks 2w, 2w+1 (accumulator layout)
    floatx4 Sf[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    if (a.s0) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) Sf[t][i] = a.s0[sbase + (int64_t)(16 * (2 * w + t) + 4 * lg + i) * DV + lr];
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        half4 hv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            amax = fmaxf(amax, __builtin_fabsf(Sf[t][i]));
            hv[i] = (_Float16)Sf[t][i];
        }
        *reinterpret_cast<half4*>(&L.S[lr][16 * (2 * w + t) + 4 * lg]) = hv;
    }

    // Two chunks per iteration with alternating operand registers: chunk c reads fa and loads
    // chunk c+1 into fb, chunk c+1 reads fb and loads chunk c+2 into fa, so no registers are
    // copied.  The explicit wait at the top of each chunk is the only place that waits on the
    // operand loads, which were issued a whole chunk earlier; the previous chunk's output store
    // follows it, so the chunk's compute overlaps both.
    ChunkFrags fa, fb;
    if (nchunks > 0) load_chunk(fa, rec_of(0), w, lane);
    lds_barrier();

    float* obase0 = a.o + (bos * H + h) * (int64_t)DV + vb * BV;
    const int64_t ostep = (int64_t)C * H * DV;
    floatx4 Oprev = {0.f, 0.f, 0.f, 0.f};
    // state snapshot after every snap_every full chunks
    auto snapshot = [&](int64_t c) {
        if (a.snap && (c + 1) % a.snap_every == 0 && len_of(c) == C) {
            const int64_t row = (a.snap_cu ? (int64_t)a.snap_cu[n] : n * a.snap_per_seq) + (c + 1) / a.snap_every - 1;
            float* dst = a.snap + (row * H + h) * (int64_t)DK * DV + vb * BV;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(int64_t)(16 * (2 * w + t) + 4 * lg + i) * DV + lr] = Sf[t][i];
        }
    };
    for (int64_t c = 0; c < nchunks; c += 2) {
        // every load issued during the previous chunk (this chunk's operands) and the previous
        // output store are complete here; stating it explicitly keeps the compiler's own wait
        // placement exact inside the chunk (it cannot track loads carried around the loop)
        __builtin_amdgcn_s_waitcnt(0x0F70);  // gfx9 encoding: vmcnt(0), expcnt/lgkmcnt at max
        if (c > 0) store_o(L, Oprev, obase0 + (c - 1) * ostep, len_of(c - 1), H, w, lane);
        const bool has_next = c + 1 < nchunks;
        Oprev = state_chunk(L, fa, fb, rec_of(has_next ? c + 1 : c), has_next, 0, Sf, w, lane, amax);
        snapshot(c);
        if (!has_next) break;
        __builtin_amdgcn_s_waitcnt(0x0F70);
        store_o(L, Oprev, obase0 + c * ostep, len_of(c), H, w, lane);
        const bool has_next2 = c + 2 < nchunks;
        Oprev = state_chunk(L, fb, fa, rec_of(has_next2 ? c + 2 : c + 1), has_next2, 1, Sf, w, lane, amax);
        snapshot(c + 1);
    }
    if (nchunks > 0) store_o(L, Oprev, obase0 + (nchunks - 1) * ostep, len_of(nchunks - 1), H, w, lane);

    // prep's range flags of this chain's chunks, a quarter per compute wave
    bool pbad = false;
#pragma unroll 4
    for (int64_t c = 64 * w + lane; c < nchunks; c += 256) pbad |= (uflags[(slot0 + c) * H + h] & kFlagRange) != 0;
    publish_flag(pbad || !(amax < 65504.f));
    // the same decision in all six waves (the helper waves read the same slots)
    if (L.bad[0] | L.bad[1] | L.bad[2] | L.bad[3] | L.bad[4] | L.bad[5]) {
        PrefillArgs r = a;
        r.snap_every = a.snap_every * (C / kRedoChunk);
        f32_chain<DK, DV, kRedoChunk, kStateThreads, uint16_t>(r, n, h, vb, redo_lds);
        return;
    }
    if (a.sT) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.sT[sbase + (int64_t)(16 * (2 * w + t) + 4 * lg + i) * DV + lr] = Sf[t][i];
    }
}

SeqMap make_map(const PrefillArgs& a) {
    SeqMap sm;
    sm.cu = a.cu;
    sm.T_fixed = a.T_fixed;
    sm.nck_fixed = a.cu ? 0 : (a.T_fixed + C - 1) / C;
    sm.N = a.N;
    return sm;
}

int64_t num_slots(int64_t N, int64_t T_fixed, int64_t T_total, bool fixed) {
    return fixed ? N * ((T_fixed + C - 1) / C) : T_total / C + N + 1;
}

}  // namespace

bool chunk_mfma_supported(int bf16, int dk, int dv, int chunk) {
    return bf16 && dk == DK && dv == DV && chunk == C;
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// Workspace layout: the records (one per slot and head), then one prep flag word per record
// (rounded up to 256 bytes).
size_t chunk_mfma_workspace(int64_t N, int64_t T_fixed, int64_t T_total, bool fixed, int H, int chunk) {
    (void)chunk;
    (void)N;
    const size_t units = (size_t)num_slots(N, T_fixed, T_total, fixed) * (size_t)H;
    return units * (size_t)kRecord + round256(units * sizeof(int32_t));
}

// ------------------------------------------------------------------------------------------
// Fixed scratch for the entry point that allocates nothing (kda_append_prefill_noalloc): the
// records and flags of one call live in this array instead of a caller workspace.
// Each GPU the library runs on holds its own copy from the code object's load until the process
// ends.  Host code never passes the array's name to a kernel (on the host it is a stand-in, not
// a device address): it takes the per-device address from hipGetSymbolAddress once per device.
// ------------------------------------------------------------------------------------------
constexpr size_t kScratchBytes = KDA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(hipStream_t s, void** out) {
    static std::mutex mu;
    static std::vector<void*> addr;  // per device, filled on the first call on that device
    int dev = 0, cur = 0;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if (addr.empty()) {
        int n = 0;
        if ((e = hipGetDeviceCount(&n)) != hipSuccess) return e;
        addr.assign((size_t)n, nullptr);
    }
    if (dev < 0 || (size_t)dev >= addr.size()) return hipErrorInvalidDevice;
    if (!addr[dev]) {
        // the symbol's address on `dev`, with `dev` current
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

hipError_t launch_chunk_mfma(const PrefillArgs& a, hipStream_t s) {
    if (a.N * a.H == 0) return hipSuccess;
    const SeqMap sm = make_map(a);
    const int64_t slots = num_slots(a.N, a.T_fixed, a.T_total, a.cu == nullptr);
    // one-dimensional grids: one prep workgroup per (slot, head), NVB state workgroups per
    // (sequence, head)
    if (slots * (int64_t)a.H > INT32_MAX || a.N * (int64_t)a.H * NVB > INT32_MAX) return hipErrorInvalidConfiguration;
    const bool timed = timing_on();
    const int64_t units = slots * (int64_t)a.H;
    int32_t* flags = reinterpret_cast<int32_t*>(static_cast<unsigned char*>(a.ws) + units * kRecord);
    if (slots > 0 && a.T_total > 0) {
        const dim3 grid((unsigned)units);
        if (timed) timed_begin(kKernelPrep, s);
        if (a.prologue)
            hipLaunchKernelGGL(prep_kernel<true>, grid, dim3(256), 0, s, a, sm, flags);
        else
            hipLaunchKernelGGL(prep_kernel<false>, grid, dim3(256), 0, s, a, sm, flags);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (timed) timed_end(s);
    }
    // the fp32 evaluation of flagged chains needs more LDS than the default dynamic limit
    constexpr size_t redo_bytes = F32Lds<DK, kRedoChunk>::kBytes;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(state_kernel),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)redo_bytes);
    if (attr != hipSuccess) return attr;
    if (timed) timed_begin(kKernelState, s);
    hipLaunchKernelGGL(state_kernel, dim3((unsigned)(a.N * a.H * NVB)), dim3(kStateThreads), redo_bytes, s, a, sm,
                       flags);
    hipError_t e = hipGetLastError();
    if (timed) timed_end(s);
    return e;
}

}  // namespace kda
