// Internal interface between the C-ABI layer (kda_api.cpp) and the kernel
// translation units.  Not installed; not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Per-kernel event timing (diagnostics).  When timing is on for the calling
// thread, launchers bracket each kernel with timed_begin/timed_end.
enum KernelId {
    kKernelPrep = 1,
    kKernelState = 2,
    kKernelChunkF32 = 3,
    kKernelDecode = 4,
    kKernelBwdFactors = 5,
    kKernelBwdFwdChain = 6,
    kKernelBwdRevChain = 7,
    kKernelBwdGradState = 8,
    kKernelBwdGradChunk = 9
};
bool timing_on();
void timed_begin(int kernel_id, hipStream_t s);
void timed_end(hipStream_t s);

// Sequences of a prefill/append call.  Either `cu` (device int32 [N+1]) is set,
// or every sequence has `T_fixed` tokens and sequence n starts at n * T_fixed.
struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const void* beta;
    const float* s0;  // [N, H, dk, dv] or nullptr
    float* o;         // [T_total, H, dv]
    float* sT;        // [N, H, dk, dv] or nullptr
    const int32_t* cu;
    int64_t N;
    int64_t T_fixed;
    int64_t T_total;
    int H, dk, dv, chunk;
    int bf16;  // storage type of q, k, v, beta
    void* ws;
    size_t ws_bytes;
    int gate_head;          // g is [T_total, H] (one decay per token and head) instead of [T_total, H, dk]
    float* snap;            // state snapshots, or nullptr
    int snap_every;         // chunks between snapshots
    const int32_t* snap_cu; // varlen: first snapshot row of each sequence (device)
    int64_t snap_per_seq;   // fixed length: snapshots per sequence
    int prologue;           // raw inputs: normalise q, k; beta = sigmoid(beta); g = -gate_scale * softplus(g)
    float gate_scale;
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const void* beta;
    const float* s_in;
    float* s_out;
    float* o;
    int64_t N;
    int H, dk, dv;
    int bf16;
    int gate_head;  // g is [N, H] (one decay per sequence and head) instead of [N, H, dk]
    int prologue;   // raw inputs, as in PrefillArgs
    float gate_scale;
};

// Chunked backward.  Sequences are packed (device cu_seqlens [N+1]); outputs are fp32.
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const void* beta;
    const int32_t* cu;
    int64_t N;
    int64_t T_total;
    int H, dk, dv, chunk;
    int bf16;       // storage type of q, k, v, beta
    int gate_head;  // g is [T_total, H]; gg is then [T_total, H] too
    const float* s0;   // [N, H, dk, dv] or nullptr
    const float* dO;   // [T_total, H, dv]
    const float* dsT;  // [N, H, dk, dv] or nullptr
    float* gq;         // [T_total, H, dk]
    float* gk;         // [T_total, H, dk]
    float* gv;         // [T_total, H, dv]
    float* gg;         // [T_total, H, dk] or [T_total, H]
    float* gbeta;      // [T_total, H]
    float* gs0;        // [N, H, dk, dv] or nullptr
    float* ws;
    float* s_fin;      // windowed passes: the forward chain's state after the window [N, H, dk, dv], or nullptr
};

bool chunk_bwd_supported(int dk, int dv, int chunk);
size_t chunk_bwd_workspace(int64_t N, int64_t T_total, int H, int dk, int dv, int chunk);
hipError_t launch_chunk_bwd(const BwdArgs& a, hipStream_t s);

// generic fp32-arithmetic chunked kernel (any supported shape, either storage type)
bool chunk_f32_supported(int dk, int dv, int chunk);
hipError_t launch_chunk_f32(const PrefillArgs& a, hipStream_t s);

// matrix-core chunked path (bfloat16 storage, dk = dv = 128, chunk = 64)
bool chunk_mfma_supported(int bf16, int dk, int dv, int chunk);
size_t chunk_mfma_workspace(int64_t N, int64_t T_fixed, int64_t T_total, bool fixed, int H, int chunk);
hipError_t launch_chunk_mfma(const PrefillArgs& a, hipStream_t s);
// the fixed device scratch of the entry point that allocates nothing: its size, and its address
// on the device of stream s (resolved once per device)
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(hipStream_t s, void** out);

// decode step
bool decode_supported(int dk, int dv);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

}  // namespace kda
