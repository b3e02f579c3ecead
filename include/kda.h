/*
 * kda.h — C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) library.
 *
 * What is computed ("Kimi K3, explained", vibeengines.com/paper/kimi-k3,
 * sections "How Kimi Delta Attention works, step by step" and "The math",
 * gated delta rule equation; the page writes the state as d_v x d_k, this
 * library stores its transpose):
 *
 *   per sequence and head, state S in R^{d_k x d_v} (row = key channel,
 *   column = value channel), alpha_t = exp(g_t) per key channel:
 *       S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *       o_t = S_t^T q_t                      (read after the write)
 *
 * Prefill and append-prefill evaluate this recurrence in chunks of `chunk`
 * tokens ("Training in chunks": inside a chunk the product of decay-and-erase
 * transitions becomes dense products plus one triangular solve; only S
 * crosses chunk boundaries).  Decode applies one token per sequence at a cost
 * independent of the context length ("The decode wall"; "KDA: trade the cache
 * for a fixed-size state").
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; tensors are
 *     contiguous and row-major.  Alignment: for prefill and append, q, k and g
 *     16 bytes and the workspace 256 bytes; for decode, both states 16 bytes;
 *     every other pointer its element size.
 *   - Sizes: H * max(d_k, d_v) must be below 2^23 (a chunk's rows are
 *     addressed with 32-bit byte offsets); KDA_ERR_INVALID_ARG otherwise.
 *   - q, k, v and beta have the storage type `dtype` (KDA_F32: float,
 *     KDA_BF16: bfloat16).  g = log(alpha) is always float (fp32, values <= 0
 *     expected), states and outputs are always float.
 *   - Calls are asynchronous on `hip_stream` (a hipStream_t; NULL = the null
 *     stream).  The library never synchronises (unless KDA_DEBUG_SYNC=1 or
 *     KDA_DEBUG_CHECK=1 is set in the environment), never allocates or frees
 *     device memory, and keeps no pointer after returning.  The caller keeps
 *     every buffer alive until the stream has drained.
 *   - Return value: KDA_OK or a negative kda_status.  Arguments are validated
 *     on the host before any device work; a failed call launches nothing.
 *     kda_last_error() gives a message for the calling thread.
 *   - Device-resident data (cu_seqlens and snapshot_cu contents, gate ranges)
 *     is a caller contract and is not inspected by default.  With
 *     KDA_DEBUG_CHECK=1 in the environment every call first waits for its
 *     stream, copies those arrays to the host and checks them with the
 *     kda_validate_* functions below (cu_seqlens: cu[0] = 0, non-decreasing,
 *     cu[N] = T_total; snapshot_cu: consistent with cu_seqlens; g finite and
 *     <= 0, beta in [0, 1]; with the fused prologue, g and beta finite).  A
 *     violation returns KDA_ERR_INVALID_ARG before any launch.  Without the
 *     check, offsets that break the contract make the kernels read and write
 *     outside the caller's buffers.
 *   - bfloat16 path numerics (d_k = d_v = 128, chunk 64): products inside a
 *     chunk use fp16 matrix-core operands with fp32 accumulation; the state,
 *     the decays and all outputs are fp32.  Every value rounded to an fp16
 *     operand is first checked against the fp16 range (|x| < 65504; NaN and
 *     Inf fail too): q and k entries (which must not exceed 32768; unit-length
 *     q and k, as the DeltaNet family uses them, are far inside), the gated
 *     Gram matrix M, the UT transform T and the WY factor W per chunk, and
 *     beta*v, the per-token corrections and the state per chain.  A (sequence,
 *     head, 16-column value block) chain that meets a value outside the range
 *     is recomputed in the same call by the fp32 chunked evaluation (fp32
 *     accuracy, at that path's speed), so there is no range limit beyond
 *     fp32's.  Decays of any strength are exact up to rounding: a
 *     chunk in which some channel decays by more than e^10 over 8 tokens sums
 *     its diagonal 16x16 Gram tiles in fp32 with one exponential per token
 *     pair, which costs that chunk extra time.  The fp32 path has no such
 *     limits.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad cu_seqlens count, ... */
    KDA_ERR_UNSUPPORTED = -2, /* (dtype, d_k, d_v, chunk) combination not implemented */
    KDA_ERR_MISALIGNED = -3,  /* a pointer is not aligned as required (see Conventions) */
    KDA_ERR_ALIAS = -4,       /* outputs overlap inputs, or state_out partially overlaps state_in */
    KDA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than kda_workspace_size() */
    KDA_ERR_HIP = -6          /* the HIP runtime reported an error (message in kda_last_error) */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

typedef enum { KDA_OP_PREFILL = 0, KDA_OP_APPEND = 1, KDA_OP_DECODE = 2, KDA_OP_BACKWARD = 3 } kda_op;

/*
 * Chunked prefill of B equal-length sequences of T tokens.
 *   q, k       [B, T, H, d_k]   dtype
 *   v          [B, T, H, d_v]   dtype
 *   g          [B, T, H, d_k]   float, log of the per-channel forget gate alpha
 *   beta       [B, T, H]        dtype, write strength
 *   state_in   [B, H, d_k, d_v] float, or NULL for a zero initial state
 *   out        [B, T, H, d_v]   float
 *   state_out  [B, H, d_k, d_v] float, or NULL; may equal state_in (in place),
 *              must not partially overlap it
 *   chunk      tokens per chunk: 16, 32 or 64 (64 for the bfloat16 d=128 path)
 *   workspace  device scratch of at least kda_workspace_size(KDA_OP_PREFILL, B, T, ...)
 *              bytes (NULL allowed when that size is 0), 256-byte aligned,
 *              overlapping no other argument (KDA_ERR_ALIAS); contents need no
 *              initialisation and are clobbered.
 * T = 0 copies state_in to state_out (zeros when state_in is NULL).
 */
int kda_prefill_chunked(const void* q, const void* k, const void* v, const float* g, const void* beta,
                        const float* state_in, float* out, float* state_out, int64_t B, int64_t T,
                        int32_t H, int32_t d_k, int32_t d_v, int32_t dtype, int32_t chunk,
                        void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Append-prefill of N packed variable-length segments, each continuing from
 * its own carried state (the append-prefill workload: a long new segment on
 * top of a kept history).
 *   q, k, g    [T_total, H, d_k]; v [T_total, H, d_v]; beta [T_total, H]
 *   cu_seqlens DEVICE int32 [N + 1]: cu[0] = 0, non-decreasing, cu[N] = T_total
 *              (segment n is tokens cu[n] .. cu[n+1]-1; checked only with
 *              KDA_DEBUG_CHECK=1, see Conventions)
 *   state_in   [N, H, d_k, d_v] float or NULL (zeros); state_out as in prefill
 *   out        [T_total, H, d_v] float
 * Empty segments pass their state through unchanged.
 */
int kda_append_prefill(const void* q, const void* k, const void* v, const float* g, const void* beta,
                       const int32_t* cu_seqlens, int32_t N, int64_t T_total, const float* state_in,
                       float* out, float* state_out, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype,
                       int32_t chunk, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * One decode step: one new token for each of N sequences.
 *   q, k, g    [N, H, d_k]; v [N, H, d_v]; beta [N, H]
 *   state_in   [N, H, d_k, d_v] float (required)
 *   state_out  [N, H, d_k, d_v] float (required); may equal state_in for an
 *              in-place update, must not partially overlap it
 *   out        [N, H, d_v] float
 * Each state element is read once and written once.
 */
int kda_decode_step(const void* q, const void* k, const void* v, const float* g, const void* beta,
                    const float* state_in, float* state_out, float* out, int32_t N, int32_t H,
                    int32_t d_k, int32_t d_v, int32_t dtype, void* hip_stream);

/*
 * Extended calls: the same operations with options.
 *
 * Gate kind ("Kimi K3, explained", "How Kimi Delta Attention works, step by
 * step" and the comparison with Gated DeltaNet, whose forget gate is one
 * scalar per head and token rather than one value per key channel):
 *   KDA_GATE_CHANNEL  g has one log-decay per key channel: [..., H, d_k]
 *                     (KDA; the plain calls always use this).
 *   KDA_GATE_HEAD     g has one log-decay per token and head: [..., H], and
 *                     alpha_t = exp(g_t) multiplies every key channel (Gated
 *                     DeltaNet; g = 0 gives the plain delta rule).
 *
 * State snapshots ("Kimi K3 changed the memory math for agentic AI": keeping
 * the fixed-size state at checkpoints of a long context so that a session can
 * resume from one).  With snapshot_every = E > 0 (prefill and append only),
 * the state after every E * chunk tokens of a sequence is written, counted
 * from the start of the call's tokens for that sequence: snapshot m (m = 0,
 * 1, ...) is the state after the first (m + 1) * E * chunk tokens, for every
 * such count that does not exceed the sequence's length.  The final state
 * still goes to state_out.
 *   prefill: snapshots [B, T / (E * chunk), H, d_k, d_v] float (integer division)
 *   append:  snapshots [snapshot_cu[N], H, d_k, d_v] float, sequence n at rows
 *            snapshot_cu[n] .. snapshot_cu[n+1]-1; snapshot_cu is a DEVICE
 *            int32 [N + 1] with snapshot_cu[0] = 0 and snapshot_cu[n+1] -
 *            snapshot_cu[n] = (cu_seqlens[n+1] - cu_seqlens[n]) / (E * chunk)
 *            (a caller contract, not checked on the device).
 * snapshots must be 4-byte aligned and overlap no other argument.
 *
 * Fused input prologue ("Kimi K3, explained", "How Kimi Delta Attention
 * works, step by step": in the DeltaNet family queries and keys are
 * L2-normalised; beta is a write strength in (0, 1) and alpha a forget gate in
 * (0, 1)).  With prologue = 1 the inputs are the raw projections and the
 * kernels apply, per token and head:
 *   q <- q / ||q||,  k <- k / ||k||       (a zero vector stays zero)
 *   beta <- sigmoid(beta)                 (beta holds logits)
 *   g <- -gate_scale * softplus(g)        (g holds the raw gate input a, per
 *                                          key channel or per head)
 * so that no separate elementwise pass (and no extra round trip through
 * memory) is needed.  gate_scale must be finite and > 0.
 *
 * A NULL options pointer means { KDA_GATE_CHANNEL, 0, NULL, NULL, 0, 0 }.
 */
typedef enum { KDA_GATE_CHANNEL = 0, KDA_GATE_HEAD = 1 } kda_gate;

typedef struct kda_options {
    int32_t gate;               /* kda_gate */
    int32_t snapshot_every;     /* chunks between state snapshots; 0 = none (must be 0 for decode) */
    float* snapshots;           /* see above; NULL when snapshot_every = 0 */
    const int32_t* snapshot_cu; /* append only; NULL otherwise */
    int32_t prologue;           /* 1: raw q, k, beta logits and gate inputs (see above); 0: as stored */
    float gate_scale;           /* prologue only: g = -gate_scale * softplus(a) */
} kda_options;

int kda_prefill_chunked_ex(const void* q, const void* k, const void* v, const float* g, const void* beta,
                           const float* state_in, float* out, float* state_out, int64_t B, int64_t T,
                           int32_t H, int32_t d_k, int32_t d_v, int32_t dtype, int32_t chunk,
                           void* workspace, size_t workspace_bytes, const kda_options* options,
                           void* hip_stream);

int kda_append_prefill_ex(const void* q, const void* k, const void* v, const float* g, const void* beta,
                          const int32_t* cu_seqlens, int32_t N, int64_t T_total, const float* state_in,
                          float* out, float* state_out, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype,
                          int32_t chunk, void* workspace, size_t workspace_bytes, const kda_options* options,
                          void* hip_stream);

int kda_decode_step_ex(const void* q, const void* k, const void* v, const float* g, const void* beta,
                       const float* state_in, float* state_out, float* out, int32_t N, int32_t H,
                       int32_t d_k, int32_t d_v, int32_t dtype, const kda_options* options, void* hip_stream);

/*
 * kda_append_prefill_noalloc — kda_append_prefill_ex without a workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * results and errors as kda_append_prefill_ex with a workspace (the same
 * kernels), except:
 *   - The scratch the matrix-core path needs (kda_workspace_size(KDA_OP_APPEND,
 *     ...) bytes) comes from a fixed array of KDA_NOALLOC_SCRATCH_BYTES bytes
 *     in device memory that the library holds on each GPU it runs on, from
 *     its first use there until the process ends.  A call that needs more
 *     returns KDA_ERR_WORKSPACE before any launch; 128 MiB covers, e.g.,
 *     H = 32 with T_total / 64 + N <= 62 (one segment of up to 3,904 tokens).
 *     Shapes served by the fp32 kernel need no scratch.
 *   - The call allocates and frees nothing (no hipMalloc, hipFree or
 *     allocating library routine).  Its first call on a device looks up the
 *     array's address on that device once (hipGetSymbolAddress).
 *   - Every call on one GPU shares that GPU's array, which keeps the previous
 *     call's contents (nothing in it needs clearing: every word a call reads
 *     it has written first).  Calls that overlap in time on one GPU (several
 *     streams, or several host threads) race on it: serialise them, e.g. on
 *     one stream.
 *   - KDA_DEBUG_CHECK=1 (see Conventions) synchronises and copies through host
 *     memory, so it is for debugging only, not for the callers above.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

int kda_append_prefill_noalloc(const void* q, const void* k, const void* v, const float* g, const void* beta,
                               const int32_t* cu_seqlens, int32_t N, int64_t T_total, const float* state_in,
                               float* out, float* state_out, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype,
                               int32_t chunk, const kda_options* options, void* hip_stream);

/*
 * kda_chunked_backward — gradients of the chunked prefill (training).
 *
 * "Kimi K3, explained" ("How is KDA trained efficiently if it is a
 * recurrence?"; "Training in chunks") states that training runs the same
 * recurrence in chunks; it prints no gradient equations.  This call returns
 * the derivative of the recurrence of kda_append_prefill (same inputs, same
 * packed layout) with respect to every input, given the gradients of a loss L
 * with respect to its outputs:
 *   d_out        [T_total, H, d_v] float   dL/do (required when T_total > 0)
 *   d_state_out  [N, H, d_k, d_v] float    dL/dS_T, or NULL (zero)
 * and writes (all float, caller-owned, overlapping no input):
 *   dq, dk       [T_total, H, d_k]         dL/dq, dL/dk
 *   dv           [T_total, H, d_v]         dL/dv
 *   dg           [T_total, H, d_k]         dL/dg (g = log alpha); [T_total, H]
 *                                          with options->gate = KDA_GATE_HEAD
 *   dbeta        [T_total, H]              dL/dbeta
 *   d_state_in   [N, H, d_k, d_v]          dL/dS_0, or NULL (not wanted)
 * q, k, v, g, beta, cu_seqlens, state_in, dtype and chunk are as for
 * kda_append_prefill (a batch of B equal sequences is cu_seqlens = 0, T, 2T,
 * ...).  Accumulation is fp32 whatever dtype is; with KDA_BF16 at d = 128,
 * chunk 64 the chain and state-side products multiply split-bf16 operands
 * (each fp32 value as bf16 hi plus bf16 lo, three bf16 matrix-core steps per
 * product, within about 2^-16 of the fp32 product), the rest fp32 operands.
 * Supported shapes:
 * d_k = d_v in {16, 32, 64, 128}, chunk in {16, 32, 64}.  options may be NULL;
 * only options->gate is honoured, and snapshot_every and prologue must be 0
 * (KDA_ERR_UNSUPPORTED otherwise).  workspace: at least
 * kda_workspace_size(KDA_OP_BACKWARD, N, T_total, H, d_k, d_v, dtype, chunk)
 * bytes, 256-byte aligned, overlapping no argument; it holds the per-chunk
 * factors, the states entering each chunk and the state gradients leaving it.
 * That grows with T_total (about 545 KB per chunk and head at d = 128, chunk
 * 64); when it would exceed 20 GiB (or the byte count in the environment
 * variable KDA_BWD_WORKSPACE_CAP, read by both kda_workspace_size and the
 * call, which must agree), the chunks are taken in windows of a fixed number
 * of chunks of every sequence: the factors and the forward state chain run
 * twice (a forward sweep keeping the states at window boundaries, then a
 * reverse sweep that rebuilds each window from its checkpoint), and the
 * workspace is one window's records plus the checkpoints.  The results are
 * bitwise those of the one-pass evaluation.
 * The gradient outputs must not overlap one another either (KDA_ERR_ALIAS).
 * Repeated calls on the same inputs give bitwise equal results (no atomics).
 * Asynchronous on hip_stream; errors as for the other calls.
 */
int kda_chunked_backward(const void* q, const void* k, const void* v, const float* g, const void* beta,
                         const int32_t* cu_seqlens, int32_t N, int64_t T_total, const float* state_in,
                         const float* d_out, const float* d_state_out, float* dq, float* dk, float* dv,
                         float* dg, float* dbeta, float* d_state_in, int32_t H, int32_t d_k, int32_t d_v,
                         int32_t dtype, int32_t chunk, void* workspace, size_t workspace_bytes,
                         const kda_options* options, void* hip_stream);

/*
 * Host-side validators of the device-resident contract (the checks that
 * KDA_DEBUG_CHECK=1 applies to a call's data after copying it to the host).
 * Every pointer here is a HOST pointer; nothing is launched.  Each returns
 * KDA_OK, or KDA_ERR_INVALID_ARG with a message in kda_last_error().
 *   kda_validate_cu_seqlens   cu [N + 1]: cu[0] = 0, cu[n] <= cu[n+1],
 *                             cu[N] = T_total (the append-prefill layout).
 *   kda_validate_snapshot_cu  snapshot_cu [N + 1]: snapshot_cu[0] = 0 and
 *                             snapshot_cu[n+1] - snapshot_cu[n] =
 *                             (cu[n+1] - cu[n]) / (snapshot_every * chunk).
 *   kda_validate_gates        g [n_g] finite and <= 0 (alpha = exp(g) in
 *                             (0, 1]); beta [n_beta] finite and in [0, 1]
 *                             ("Kimi K3, explained", "How Kimi Delta
 *                             Attention works, step by step": both gates lie
 *                             in (0, 1)).  raw = 1 (fused prologue inputs):
 *                             finite only.  beta is given as float.
 */
int kda_validate_cu_seqlens(const int32_t* cu, int32_t N, int64_t T_total);
int kda_validate_snapshot_cu(const int32_t* cu, const int32_t* snapshot_cu, int32_t N, int32_t snapshot_every,
                             int32_t chunk);
int kda_validate_gates(const float* g, int64_t n_g, const float* beta, int64_t n_beta, int32_t raw);

/* Workspace bytes an op needs (B_or_N sequences, T tokens per sequence for
 * KDA_OP_PREFILL or T_total for KDA_OP_APPEND and KDA_OP_BACKWARD).  0 for
 * KDA_OP_DECODE.
 * Returns (size_t)-1 for an unsupported or invalid combination. */
size_t kda_workspace_size(int32_t op, int64_t B_or_N, int64_t T, int32_t H, int32_t d_k, int32_t d_v,
                          int32_t dtype, int32_t chunk);

/* 1 if (op, dtype, d_k, d_v, chunk) is implemented, else 0. */
int kda_is_supported(int32_t op, int32_t dtype, int32_t d_k, int32_t d_v, int32_t chunk);

/* Static description of a kda_status value. */
const char* kda_status_string(int status);

/* Message describing the last failed call on the calling thread ("" if none). */
const char* kda_last_error(void);

/* Library version string. */
const char* kda_version(void);

/*
 * Diagnostics: per-kernel timing with HIP events (the library's own tracing).
 * kda_timing_begin() starts recording, for calls made on the calling thread,
 * a HIP event immediately before and after every kernel the library launches,
 * on that call's stream.  kda_timing_end() stops recording, waits for the
 * recorded events, and writes up to max_records (kernel id, milliseconds)
 * pairs in launch order into kernel_ids / ms (either may be NULL to only
 * count).  Returns the number of kernels recorded, or a negative kda_status
 * (KDA_ERR_HIP if an event failed).  Event objects are created on first use and
 * reused; no device memory is allocated.  Kernel ids are kda_kernel values.
 */
typedef enum {
    KDA_KERNEL_PREP = 1,      /* chunk-parallel prep of the matrix-core prefill */
    KDA_KERNEL_STATE = 2,     /* sequential state pass of the matrix-core prefill */
    KDA_KERNEL_CHUNK_F32 = 3, /* fp32 chunked prefill */
    KDA_KERNEL_DECODE = 4,    /* decode step */
    KDA_KERNEL_BWD_FACTORS = 5,    /* backward: per-chunk factors */
    KDA_KERNEL_BWD_FWD_CHAIN = 6,  /* backward: states entering each chunk */
    KDA_KERNEL_BWD_REV_CHAIN = 7,  /* backward: state gradients, chunks in reverse */
    KDA_KERNEL_BWD_GRAD_STATE = 8, /* backward: products over the value axis */
    KDA_KERNEL_BWD_GRAD_CHUNK = 9  /* backward: in-chunk gradients */
} kda_kernel;

int kda_timing_begin(void);
int kda_timing_end(int32_t* kernel_ids, float* ms, int32_t max_records);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
