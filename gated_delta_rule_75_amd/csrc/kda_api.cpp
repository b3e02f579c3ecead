// C ABI of the KDA library: argument validation, kernel selection, launch and
// status reporting.  Declarations and contracts: include/kda.h.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "kda_internal.h"

// ---------------------------------------------------------------------------------------
// per-kernel event timing (diagnostics), per calling thread
// ---------------------------------------------------------------------------------------
namespace {
struct TimingState {
    bool on = false;
    bool failed = false;
    struct Rec {
        int id;
        hipEvent_t start, stop;
    };
    std::vector<Rec> recs;
    std::vector<hipEvent_t> pool;
    size_t used = 0;

    hipEvent_t take() {
        if (used == pool.size()) {
            hipEvent_t e = nullptr;
            if (hipEventCreate(&e) != hipSuccess) {
                failed = true;
                return nullptr;
            }
            pool.push_back(e);
        }
        return pool[used++];
    }
};
thread_local TimingState g_timing;
}  // namespace

namespace kda {
bool timing_on() { return g_timing.on; }
void timed_begin(int kernel_id, hipStream_t s) {
    TimingState::Rec r{kernel_id, g_timing.take(), g_timing.take()};
    if (!r.start || !r.stop || hipEventRecord(r.start, s) != hipSuccess) {
        g_timing.failed = true;
        return;
    }
    g_timing.recs.push_back(r);
}
void timed_end(hipStream_t s) {
    if (g_timing.recs.empty() || hipEventRecord(g_timing.recs.back().stop, s) != hipSuccess) g_timing.failed = true;
}
}  // namespace kda

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return KDA_OK;
}

bool env_flag(const char* name) {
    const char* v = std::getenv(name);
    return v && v[0] && std::strcmp(v, "0") != 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Span {
    const void* p;
    size_t bytes;
};

bool overlap(Span a, Span b) {
    if (!a.p || !b.p || !a.bytes || !b.bytes) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

int check_hip(hipError_t e, hipStream_t s, const char* what) {
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    if (env_flag("KDA_DEBUG_SYNC")) {
        e = hipStreamSynchronize(s);
        if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s (debug sync): %s", what, hipGetErrorString(e));
    }
    return ok();
}

// Host-side stand-in for a launch failure, for tests of the error path only.
bool injected_launch_failure() { return env_flag("KDA_TEST_FAIL_LAUNCH"); }

// ---------------------------------------------------------------------------------------
// Debug checks of device-resident data (KDA_DEBUG_CHECK=1): the offsets and gates are
// copied to the host, after the caller's stream has drained, and validated before any
// launch.  Off by default: the calls then never synchronise.
// ---------------------------------------------------------------------------------------
bool debug_check() { return env_flag("KDA_DEBUG_CHECK"); }

template <typename T>
int fetch(const void* dev, size_t count, hipStream_t s, std::vector<T>& out, const char* name) {
    out.resize(count);
    if (!count) return KDA_OK;
    hipError_t e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipMemcpy(out.data(), dev, count * sizeof(T), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s (debug check): %s", name, hipGetErrorString(e));
    return KDA_OK;
}

float bf16_bits_to_float(uint16_t b) {
    const uint32_t u = static_cast<uint32_t>(b) << 16;
    float f;
    std::memcpy(&f, &u, sizeof(f));
    return f;
}

// cu_seqlens (and snapshot_cu when every > 0) of an append or backward call
int debug_check_offsets(const int32_t* cu, int32_t N, int64_t T_total, const int32_t* snap_cu, int32_t every,
                        int32_t chunk, hipStream_t s, const char* name) {
    std::vector<int32_t> h, hs;
    if (int rc = fetch(cu, (size_t)N + 1, s, h, name)) return rc;
    if (int rc = kda_validate_cu_seqlens(h.data(), N, T_total)) return rc;
    if (every > 0 && snap_cu) {
        if (int rc = fetch(snap_cu, (size_t)N + 1, s, hs, name)) return rc;
        if (int rc = kda_validate_snapshot_cu(h.data(), hs.data(), N, every, chunk)) return rc;
    }
    return KDA_OK;
}

// g (ng floats) and beta (nb values of dtype); raw prologue inputs are only checked to be finite
int debug_check_gates(const float* g, size_t ng, const void* beta, size_t nb, int32_t dtype, bool prologue,
                      hipStream_t s, const char* name) {
    std::vector<float> hg, hb(nb);
    if (int rc = fetch(g, ng, s, hg, name)) return rc;
    if (dtype == KDA_BF16) {
        std::vector<uint16_t> raw;
        if (int rc = fetch(beta, nb, s, raw, name)) return rc;
        for (size_t i = 0; i < nb; ++i) hb[i] = bf16_bits_to_float(raw[i]);
    } else if (int rc = fetch(beta, nb, s, hb, name)) {
        return rc;
    }
    return kda_validate_gates(hg.data(), (int64_t)ng, hb.data(), (int64_t)nb, prologue ? 1 : 0);
}

bool valid_dtype(int32_t d) { return d == KDA_F32 || d == KDA_BF16; }

// Which chunked implementation serves (dtype, dk, dv, chunk): 2 = matrix cores, 1 = fp32, 0 = none.
int prefill_path(int32_t dtype, int32_t dk, int32_t dv, int32_t chunk) {
    if (kda::chunk_mfma_supported(dtype == KDA_BF16, dk, dv, chunk)) return 2;
    if (kda::chunk_f32_supported(dk, dv, chunk)) return 1;
    return 0;
}

size_t ws_size(int32_t op, int64_t N, int64_t T, int32_t H, int32_t dk, int32_t dv, int32_t dtype, int32_t chunk) {
    if (op == KDA_OP_DECODE) return 0;
    if (op == KDA_OP_BACKWARD) return kda::chunk_bwd_workspace(N, T, H, dk, dv, chunk);
    if (prefill_path(dtype, dk, dv, chunk) != 2) return 0;
    const bool fixed = op == KDA_OP_PREFILL;
    const int64_t T_total = fixed ? N * T : T;
    return kda::chunk_mfma_workspace(N, fixed ? T : 0, T_total, fixed, H, chunk);
}

int run_prefill(const kda::PrefillArgs& a, int32_t dtype, hipStream_t s, const char* name) {
    const int path = prefill_path(dtype, a.dk, a.dv, a.chunk);
    if (injected_launch_failure()) return fail(KDA_ERR_HIP, "%s: injected launch failure (KDA_TEST_FAIL_LAUNCH)", name);
    hipError_t e = path == 2 ? kda::launch_chunk_mfma(a, s) : kda::launch_chunk_f32(a, s);
    return check_hip(e, s, name);
}

// Alignment: q, k and g are read with 16-byte vector loads by the prefill kernels
// (qkg_align = 16); every other tensor only needs its element alignment.
int validate_common(const void* q, const void* k, const void* v, const float* g, const void* beta, int64_t tokens,
                    int32_t H, int32_t dk, int32_t dv, int32_t dtype, size_t qkg_align, bool gate_head) {
    if (H <= 0 || dk <= 0 || dv <= 0) return fail(KDA_ERR_INVALID_ARG, "H, d_k, d_v must be positive");
    // the kernels address one chunk's rows (up to 64 tokens of H heads) with 32-bit byte offsets
    if ((int64_t)H * (dk > dv ? dk : dv) >= ((int64_t)1 << 23))
        return fail(KDA_ERR_INVALID_ARG, "H * max(d_k, d_v) must be below 2^23");
    if (!valid_dtype(dtype)) return fail(KDA_ERR_INVALID_ARG, "dtype must be KDA_F32 or KDA_BF16");
    if (tokens > 0 && (!q || !k || !v || !g || !beta))
        return fail(KDA_ERR_INVALID_ARG, "q, k, v, g and beta are required");
    const size_t esz = dtype == KDA_BF16 ? 2 : 4;
    const size_t qa = qkg_align > esz ? qkg_align : esz;
    if (!aligned_to(q, qa) || !aligned_to(k, qa) || !aligned_to(g, gate_head || qkg_align < 4 ? 4 : qkg_align))
        return fail(KDA_ERR_MISALIGNED, "q and k must be %zu-byte aligned, g %zu-byte aligned", qa,
                    gate_head || qkg_align < 4 ? (size_t)4 : qkg_align);
    if (!aligned_to(v, esz) || !aligned_to(beta, esz))
        return fail(KDA_ERR_MISALIGNED, "v and beta must be aligned to their element size");
    return KDA_OK;
}

// Options of the extended calls (NULL: defaults).
struct Opts {
    bool gate_head = false;
    int every = 0;
    float* snaps = nullptr;
    const int32_t* snap_cu = nullptr;
    bool prologue = false;
    float gate_scale = 0.f;
};

int read_options(const kda_options* o, int op, const char* name, Opts& out) {
    out = Opts{};
    if (!o) return KDA_OK;
    if (o->gate != KDA_GATE_CHANNEL && o->gate != KDA_GATE_HEAD)
        return fail(KDA_ERR_INVALID_ARG, "%s: options.gate must be KDA_GATE_CHANNEL or KDA_GATE_HEAD", name);
    if (o->snapshot_every < 0) return fail(KDA_ERR_INVALID_ARG, "%s: options.snapshot_every must be >= 0", name);
    if (op == KDA_OP_DECODE && (o->snapshot_every || o->snapshots || o->snapshot_cu))
        return fail(KDA_ERR_INVALID_ARG, "%s: a decode step takes no snapshots", name);
    if (o->snapshot_every > 0) {
        if (!o->snapshots) return fail(KDA_ERR_INVALID_ARG, "%s: options.snapshots is required", name);
        if (op == KDA_OP_APPEND && !o->snapshot_cu)
            return fail(KDA_ERR_INVALID_ARG, "%s: options.snapshot_cu is required", name);
        if (!aligned_to(o->snapshots, 4) || !aligned_to(o->snapshot_cu, 4))
            return fail(KDA_ERR_MISALIGNED, "%s: snapshots and snapshot_cu must be 4-byte aligned", name);
    }
    if (o->prologue != 0 && o->prologue != 1)
        return fail(KDA_ERR_INVALID_ARG, "%s: options.prologue must be 0 or 1", name);
    if (o->prologue && !(o->gate_scale > 0.f && o->gate_scale < 3.4e38f))
        return fail(KDA_ERR_INVALID_ARG, "%s: options.gate_scale must be finite and > 0", name);
    out.prologue = o->prologue == 1;
    out.gate_scale = o->prologue ? o->gate_scale : 0.f;
    out.gate_head = o->gate == KDA_GATE_HEAD;
    out.every = o->snapshot_every;
    out.snaps = o->snapshot_every > 0 ? o->snapshots : nullptr;
    out.snap_cu = o->snapshot_every > 0 ? o->snapshot_cu : nullptr;
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_validate_cu_seqlens(const int32_t* cu, int32_t N, int64_t T_total) {
    if (!cu || N < 0) return fail(KDA_ERR_INVALID_ARG, "kda_validate_cu_seqlens: cu must be non-NULL and N >= 0");
    if (cu[0] != 0) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens[0] = %d, expected 0", cu[0]);
    for (int32_t n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n])
            return fail(KDA_ERR_INVALID_ARG, "cu_seqlens decreases at %d: %d > %d", n, cu[n], cu[n + 1]);
    if ((int64_t)cu[N] != T_total)
        return fail(KDA_ERR_INVALID_ARG, "cu_seqlens[%d] = %d, expected T_total = %lld", N, cu[N], (long long)T_total);
    return ok();
}

int kda_validate_snapshot_cu(const int32_t* cu, const int32_t* snapshot_cu, int32_t N, int32_t snapshot_every,
                             int32_t chunk) {
    if (!cu || !snapshot_cu || N < 0 || snapshot_every <= 0 || chunk <= 0)
        return fail(KDA_ERR_INVALID_ARG, "kda_validate_snapshot_cu: bad arguments");
    if (snapshot_cu[0] != 0) return fail(KDA_ERR_INVALID_ARG, "snapshot_cu[0] = %d, expected 0", snapshot_cu[0]);
    const int64_t interval = (int64_t)snapshot_every * chunk;
    for (int32_t n = 0; n < N; ++n) {
        const int64_t want = ((int64_t)cu[n + 1] - cu[n]) / interval;
        if ((int64_t)snapshot_cu[n + 1] - snapshot_cu[n] != want)
            return fail(KDA_ERR_INVALID_ARG, "snapshot_cu[%d] - snapshot_cu[%d] = %d, expected %lld", n + 1, n,
                        snapshot_cu[n + 1] - snapshot_cu[n], (long long)want);
    }
    return ok();
}

int kda_validate_gates(const float* g, int64_t n_g, const float* beta, int64_t n_beta, int32_t raw) {
    if ((n_g > 0 && !g) || (n_beta > 0 && !beta) || n_g < 0 || n_beta < 0)
        return fail(KDA_ERR_INVALID_ARG, "kda_validate_gates: bad arguments");
    for (int64_t i = 0; i < n_g; ++i) {
        const float x = g[i];
        if (!std::isfinite(x) || (!raw && x > 0.f))
            return fail(KDA_ERR_INVALID_ARG, "g[%lld] = %g: %s", (long long)i, (double)x,
                        raw ? "not finite" : "a log-decay must be finite and <= 0");
    }
    for (int64_t i = 0; i < n_beta; ++i) {
        const float x = beta[i];
        if (!std::isfinite(x) || (!raw && (x < 0.f || x > 1.f)))
            return fail(KDA_ERR_INVALID_ARG, "beta[%lld] = %g: %s", (long long)i, (double)x,
                        raw ? "not finite" : "must lie in [0, 1]");
    }
    return ok();
}

const char* kda_version(void) { return "kda-mi355x 0.2.0 (gfx950)"; }

int kda_timing_begin(void) {
    g_timing.on = true;
    g_timing.failed = false;
    g_timing.recs.clear();
    g_timing.used = 0;
    return ok();
}

int kda_timing_end(int32_t* kernel_ids, float* ms, int32_t max_records) {
    g_timing.on = false;
    if (g_timing.failed) return fail(KDA_ERR_HIP, "kda_timing_end: an event could not be created or recorded");
    int32_t n = 0;
    for (const auto& r : g_timing.recs) {
        float t = 0.f;
        hipError_t e = hipEventSynchronize(r.stop);
        if (e == hipSuccess) e = hipEventElapsedTime(&t, r.start, r.stop);
        if (e != hipSuccess) return fail(KDA_ERR_HIP, "kda_timing_end: %s", hipGetErrorString(e));
        if (n < max_records) {
            if (kernel_ids) kernel_ids[n] = r.id;
            if (ms) ms[n] = t;
        }
        ++n;
    }
    g_timing.recs.clear();
    g_timing.used = 0;
    ok();
    return n;
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

const char* kda_status_string(int status) {
    switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID_ARG: return "invalid argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported shape, dtype or chunk size";
    case KDA_ERR_MISALIGNED: return "pointer not aligned as required";
    case KDA_ERR_ALIAS: return "output buffers overlap inputs";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

int kda_is_supported(int32_t op, int32_t dtype, int32_t d_k, int32_t d_v, int32_t chunk) {
    if (!valid_dtype(dtype)) return 0;
    if (op == KDA_OP_DECODE) return kda::decode_supported(d_k, d_v) ? 1 : 0;
    if (op == KDA_OP_PREFILL || op == KDA_OP_APPEND) return prefill_path(dtype, d_k, d_v, chunk) ? 1 : 0;
    if (op == KDA_OP_BACKWARD) return kda::chunk_bwd_supported(d_k, d_v, chunk) ? 1 : 0;
    return 0;
}

size_t kda_workspace_size(int32_t op, int64_t B_or_N, int64_t T, int32_t H, int32_t d_k, int32_t d_v,
                          int32_t dtype, int32_t chunk) {
    if (B_or_N < 0 || T < 0 || H <= 0 || !kda_is_supported(op, dtype, d_k, d_v, chunk)) return (size_t)-1;
    return ws_size(op, B_or_N, T, H, d_k, d_v, dtype, chunk);
}

int kda_prefill_chunked_ex(const void* q, const void* k, const void* v, const float* g, const void* beta,
                           const float* state_in, float* out, float* state_out, int64_t B, int64_t T, int32_t H,
                           int32_t d_k, int32_t d_v, int32_t dtype, int32_t chunk, void* workspace,
                           size_t workspace_bytes, const kda_options* options, void* hip_stream) {
    static const char* name = "kda_prefill_chunked";
    Opts op;
    if (int rc = read_options(options, KDA_OP_PREFILL, name, op)) return rc;
    if (B < 0 || T < 0) return fail(KDA_ERR_INVALID_ARG, "%s: B and T must be >= 0", name);
    if (int rc = validate_common(q, k, v, g, beta, B * T, H, d_k, d_v, dtype, 16, op.gate_head)) return rc;
    if (!prefill_path(dtype, d_k, d_v, chunk))
        return fail(KDA_ERR_UNSUPPORTED, "%s: dtype=%d d_k=%d d_v=%d chunk=%d not implemented", name, dtype, d_k, d_v,
                    chunk);
    if (B * T > 0 && !out) return fail(KDA_ERR_INVALID_ARG, "%s: out is required", name);
    if (!aligned_to(out, 4) || !aligned_to(state_in, 4) || !aligned_to(state_out, 4) || !aligned_to(workspace, 256))
        return fail(KDA_ERR_MISALIGNED, "%s: out and states must be 4-byte, workspace 256-byte aligned", name);
    const size_t esz = dtype == KDA_BF16 ? 2 : 4;
    const size_t tokens = (size_t)(B * T);
    const size_t sbytes = (size_t)B * H * d_k * d_v * 4;
    const Span sin{state_in, state_in ? sbytes : 0}, sout{state_out, state_out ? sbytes : 0};
    const Span o{out, tokens * H * d_v * 4};
    const int64_t snap_per_seq = op.every > 0 ? T / ((int64_t)op.every * chunk) : 0;
    const Span snp{op.snaps, (size_t)(B * snap_per_seq) * H * d_k * d_v * 4};
    const Span ins[] = {{q, tokens * H * d_k * esz}, {k, tokens * H * d_k * esz}, {v, tokens * H * d_v * esz},
                        {g, tokens * H * (op.gate_head ? 1 : d_k) * 4}, {beta, tokens * H * esz}, sin};
    for (const Span& in : ins)
        if (overlap(o, in) || (overlap(sout, in) && in.p != state_in) || overlap(snp, in))
            return fail(KDA_ERR_ALIAS, "%s: out/state_out/snapshots overlap an input", name);
    if (overlap(o, sout) || overlap(snp, o) || overlap(snp, sout))
        return fail(KDA_ERR_ALIAS, "%s: out, state_out and snapshots overlap", name);
    if (overlap(sin, sout) && state_in != state_out)
        return fail(KDA_ERR_ALIAS, "%s: state_out partially overlaps state_in", name);
    const size_t need = ws_size(KDA_OP_PREFILL, B, T, H, d_k, d_v, dtype, chunk);
    if (need && (!workspace || workspace_bytes < need))
        return fail(KDA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", name, need,
                    workspace ? workspace_bytes : (size_t)0);
    const Span wsp{workspace, need};
    for (const Span& in : ins)
        if (overlap(wsp, in)) return fail(KDA_ERR_ALIAS, "%s: the workspace overlaps an input", name);
    if (overlap(wsp, o) || overlap(wsp, sout) || overlap(wsp, snp))
        return fail(KDA_ERR_ALIAS, "%s: the workspace overlaps out, state_out or snapshots", name);
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (debug_check())
        if (int rc = debug_check_gates(g, tokens * H * (op.gate_head ? 1 : d_k), beta, tokens * H, dtype, op.prologue,
                                       stream, name))
            return rc;
    kda::PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.s0 = state_in; a.o = out; a.sT = state_out;
    a.cu = nullptr; a.N = B; a.T_fixed = T; a.T_total = B * T;
    a.H = H; a.dk = d_k; a.dv = d_v; a.chunk = chunk; a.bf16 = dtype == KDA_BF16;
    a.ws = workspace; a.ws_bytes = workspace_bytes;
    a.gate_head = op.gate_head; a.snap = snap_per_seq > 0 ? op.snaps : nullptr; a.snap_every = op.every;
    a.snap_cu = nullptr; a.snap_per_seq = snap_per_seq;
    a.prologue = op.prologue; a.gate_scale = op.gate_scale;
    return run_prefill(a, dtype, stream, name);
}

int kda_prefill_chunked(const void* q, const void* k, const void* v, const float* g, const void* beta,
                        const float* state_in, float* out, float* state_out, int64_t B, int64_t T, int32_t H,
                        int32_t d_k, int32_t d_v, int32_t dtype, int32_t chunk, void* workspace,
                        size_t workspace_bytes, void* hip_stream) {
    return kda_prefill_chunked_ex(q, k, v, g, beta, state_in, out, state_out, B, T, H, d_k, d_v, dtype, chunk,
                                  workspace, workspace_bytes, nullptr, hip_stream);
}

}  // extern "C"

namespace {

// Append-prefill with a caller workspace (noalloc = false), or with the library's fixed device
// scratch in place of one (noalloc = true: workspace must be NULL and 0).
int append_impl(const void* q, const void* k, const void* v, const float* g, const void* beta,
                const int32_t* cu_seqlens, int32_t N, int64_t T_total, const float* state_in, float* out,
                float* state_out, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype, int32_t chunk, void* workspace,
                size_t workspace_bytes, const kda_options* options, void* hip_stream, bool noalloc) {
    const char* name = noalloc ? "kda_append_prefill_noalloc" : "kda_append_prefill";
    Opts op;
    if (int rc = read_options(options, KDA_OP_APPEND, name, op)) return rc;
    if (N < 0 || T_total < 0) return fail(KDA_ERR_INVALID_ARG, "%s: N and T_total must be >= 0", name);
    if (!cu_seqlens) return fail(KDA_ERR_INVALID_ARG, "%s: cu_seqlens is required", name);
    if (int rc = validate_common(q, k, v, g, beta, T_total, H, d_k, d_v, dtype, 16, op.gate_head)) return rc;
    if (!prefill_path(dtype, d_k, d_v, chunk))
        return fail(KDA_ERR_UNSUPPORTED, "%s: dtype=%d d_k=%d d_v=%d chunk=%d not implemented", name, dtype, d_k, d_v,
                    chunk);
    if (T_total > 0 && !out) return fail(KDA_ERR_INVALID_ARG, "%s: out is required", name);
    if (!aligned_to(out, 4) || !aligned_to(state_in, 4) || !aligned_to(state_out, 4) || !aligned_to(workspace, 256))
        return fail(KDA_ERR_MISALIGNED, "%s: out and states must be 4-byte, workspace 256-byte aligned", name);
    const size_t esz = dtype == KDA_BF16 ? 2 : 4;
    const size_t tokens = (size_t)T_total;
    const size_t sbytes = (size_t)N * H * d_k * d_v * 4;
    const Span sin{state_in, state_in ? sbytes : 0}, sout{state_out, state_out ? sbytes : 0};
    const Span o{out, tokens * H * d_v * 4};
    // the snapshot rows are on the device (snapshot_cu); only the first row is checked here
    const Span snp{op.snaps, (size_t)H * d_k * d_v * 4};
    const Span ins[] = {{q, tokens * H * d_k * esz}, {k, tokens * H * d_k * esz}, {v, tokens * H * d_v * esz},
                        {g, tokens * H * (op.gate_head ? 1 : d_k) * 4}, {beta, tokens * H * esz},
                        {cu_seqlens, (size_t)(N + 1) * 4}, {op.snap_cu, op.snap_cu ? (size_t)(N + 1) * 4 : 0}, sin};
    for (const Span& in : ins)
        if (overlap(o, in) || (overlap(sout, in) && in.p != state_in) || overlap(snp, in))
            return fail(KDA_ERR_ALIAS, "%s: out/state_out/snapshots overlap an input", name);
    if (overlap(o, sout) || overlap(snp, o) || overlap(snp, sout))
        return fail(KDA_ERR_ALIAS, "%s: out, state_out and snapshots overlap", name);
    if (overlap(sin, sout) && state_in != state_out)
        return fail(KDA_ERR_ALIAS, "%s: state_out partially overlaps state_in", name);
    const size_t need = ws_size(KDA_OP_APPEND, N, T_total, H, d_k, d_v, dtype, chunk);
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (noalloc) {
        // the library's own scratch; it overlaps no caller buffer
        if (need > kda::noalloc_scratch_bytes())
            return fail(KDA_ERR_WORKSPACE, "%s: this call needs %zu bytes of scratch, beyond the fixed maximum of %zu",
                        name, need, kda::noalloc_scratch_bytes());
        workspace = nullptr;
        workspace_bytes = 0;
        if (need) {
            hipError_t e = kda::noalloc_scratch(stream, &workspace);
            if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: scratch address: %s", name, hipGetErrorString(e));
            workspace_bytes = kda::noalloc_scratch_bytes();
        }
    } else {
        if (need && (!workspace || workspace_bytes < need))
            return fail(KDA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", name, need,
                        workspace ? workspace_bytes : (size_t)0);
        const Span wsp{workspace, need};
        for (const Span& in : ins)
            if (overlap(wsp, in)) return fail(KDA_ERR_ALIAS, "%s: the workspace overlaps an input", name);
        if (overlap(wsp, o) || overlap(wsp, sout) || overlap(wsp, snp))
            return fail(KDA_ERR_ALIAS, "%s: the workspace overlaps out, state_out or snapshots", name);
    }
    if (debug_check()) {
        if (int rc = debug_check_offsets(cu_seqlens, N, T_total, op.snap_cu, op.every, chunk, stream, name)) return rc;
        if (int rc = debug_check_gates(g, tokens * H * (op.gate_head ? 1 : d_k), beta, tokens * H, dtype, op.prologue,
                                       stream, name))
            return rc;
    }
    kda::PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.s0 = state_in; a.o = out; a.sT = state_out;
    a.cu = cu_seqlens; a.N = N; a.T_fixed = 0; a.T_total = T_total;
    a.H = H; a.dk = d_k; a.dv = d_v; a.chunk = chunk; a.bf16 = dtype == KDA_BF16;
    a.ws = workspace; a.ws_bytes = workspace_bytes;
    a.gate_head = op.gate_head; a.snap = op.snaps; a.snap_every = op.every; a.snap_cu = op.snap_cu;
    a.snap_per_seq = 0;
    a.prologue = op.prologue; a.gate_scale = op.gate_scale;
    return run_prefill(a, dtype, stream, name);
}

}  // namespace

extern "C" {

int kda_append_prefill_ex(const void* q, const void* k, const void* v, const float* g, const void* beta,
                          const int32_t* cu_seqlens, int32_t N, int64_t T_total, const float* state_in, float* out,
                          float* state_out, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype, int32_t chunk,
                          void* workspace, size_t workspace_bytes, const kda_options* options, void* hip_stream) {
    return append_impl(q, k, v, g, beta, cu_seqlens, N, T_total, state_in, out, state_out, H, d_k, d_v, dtype, chunk,
                       workspace, workspace_bytes, options, hip_stream, false);
}

int kda_append_prefill_noalloc(const void* q, const void* k, const void* v, const float* g, const void* beta,
                               const int32_t* cu_seqlens, int32_t N, int64_t T_total, const float* state_in,
                               float* out, float* state_out, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype,
                               int32_t chunk, const kda_options* options, void* hip_stream) {
    return append_impl(q, k, v, g, beta, cu_seqlens, N, T_total, state_in, out, state_out, H, d_k, d_v, dtype, chunk,
                       nullptr, 0, options, hip_stream, true);
}

int kda_append_prefill(const void* q, const void* k, const void* v, const float* g, const void* beta,
                       const int32_t* cu_seqlens, int32_t N, int64_t T_total, const float* state_in, float* out,
                       float* state_out, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype, int32_t chunk,
                       void* workspace, size_t workspace_bytes, void* hip_stream) {
    return kda_append_prefill_ex(q, k, v, g, beta, cu_seqlens, N, T_total, state_in, out, state_out, H, d_k, d_v,
                                 dtype, chunk, workspace, workspace_bytes, nullptr, hip_stream);
}

int kda_chunked_backward(const void* q, const void* k, const void* v, const float* g, const void* beta,
                         const int32_t* cu_seqlens, int32_t N, int64_t T_total, const float* state_in,
                         const float* d_out, const float* d_state_out, float* dq, float* dk, float* dv,
                         float* dg, float* dbeta, float* d_state_in, int32_t H, int32_t d_k, int32_t d_v,
                         int32_t dtype, int32_t chunk, void* workspace, size_t workspace_bytes,
                         const kda_options* options, void* hip_stream) {
    static const char* name = "kda_chunked_backward";
    Opts op;
    if (int rc = read_options(options, KDA_OP_APPEND, name, op)) return rc;
    if (op.every || op.prologue)
        return fail(KDA_ERR_UNSUPPORTED, "%s: snapshots and the fused prologue are not part of the backward", name);
    if (N < 0 || T_total < 0) return fail(KDA_ERR_INVALID_ARG, "%s: N and T_total must be >= 0", name);
    if (!cu_seqlens) return fail(KDA_ERR_INVALID_ARG, "%s: cu_seqlens is required", name);
    if (int rc = validate_common(q, k, v, g, beta, T_total, H, d_k, d_v, dtype, 1, op.gate_head)) return rc;
    if (!kda::chunk_bwd_supported(d_k, d_v, chunk))
        return fail(KDA_ERR_UNSUPPORTED, "%s: d_k=%d d_v=%d chunk=%d not implemented", name, d_k, d_v, chunk);
    if (T_total > 0 && (!d_out || !dq || !dk || !dv || !dg || !dbeta))
        return fail(KDA_ERR_INVALID_ARG, "%s: d_out, dq, dk, dv, dg and dbeta are required", name);
    const void* fl[] = {state_in, d_out, d_state_out, dq, dk, dv, dg, dbeta, d_state_in};
    for (const void* p : fl)
        if (!aligned_to(p, 4)) return fail(KDA_ERR_MISALIGNED, "%s: float buffers must be 4-byte aligned", name);
    if (!aligned_to(workspace, 256)) return fail(KDA_ERR_MISALIGNED, "%s: workspace must be 256-byte aligned", name);
    const size_t esz = dtype == KDA_BF16 ? 2 : 4, tokens = (size_t)T_total;
    const size_t sbytes = (size_t)N * H * d_k * d_v * 4, gk = op.gate_head ? 1 : (size_t)d_k;
    const Span ins[] = {{q, tokens * H * d_k * esz},
                        {k, tokens * H * d_k * esz},
                        {v, tokens * H * d_v * esz},
                        {g, tokens * H * gk * 4},
                        {beta, tokens * H * esz},
                        {cu_seqlens, (size_t)(N + 1) * 4},
                        {state_in, state_in ? sbytes : 0},
                        {d_out, tokens * H * d_v * 4},
                        {d_state_out, d_state_out ? sbytes : 0}};
    const Span outs[] = {{dq, tokens * H * d_k * 4}, {dk, tokens * H * d_k * 4}, {dv, tokens * H * d_v * 4},
                         {dg, tokens * H * gk * 4},  {dbeta, tokens * H * 4},    {d_state_in, d_state_in ? sbytes : 0}};
    const size_t need = ws_size(KDA_OP_BACKWARD, N, T_total, H, d_k, d_v, dtype, chunk);
    const Span ws{workspace, need};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const Span& in : ins)
            if (overlap(outs[i], in)) return fail(KDA_ERR_ALIAS, "%s: a gradient output overlaps an input", name);
        for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
            if (overlap(outs[i], outs[j])) return fail(KDA_ERR_ALIAS, "%s: gradient outputs overlap", name);
        if (overlap(outs[i], ws)) return fail(KDA_ERR_ALIAS, "%s: a gradient output overlaps the workspace", name);
    }
    for (const Span& in : ins)
        if (overlap(ws, in)) return fail(KDA_ERR_ALIAS, "%s: the workspace overlaps an input", name);
    if (need && (!workspace || workspace_bytes < need))
        return fail(KDA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", name, need,
                    workspace ? workspace_bytes : (size_t)0);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    if (debug_check()) {
        if (int rc = debug_check_offsets(cu_seqlens, N, T_total, nullptr, 0, chunk, s, name)) return rc;
        if (int rc = debug_check_gates(g, tokens * H * gk, beta, tokens * H, dtype, false, s, name)) return rc;
    }
    if (injected_launch_failure()) return fail(KDA_ERR_HIP, "%s: injected launch failure (KDA_TEST_FAIL_LAUNCH)", name);
    kda::BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.cu = cu_seqlens; a.N = N; a.T_total = T_total;
    a.H = H; a.dk = d_k; a.dv = d_v; a.chunk = chunk; a.bf16 = dtype == KDA_BF16; a.gate_head = op.gate_head;
    a.s0 = state_in; a.dO = d_out; a.dsT = d_state_out;
    a.gq = dq; a.gk = dk; a.gv = dv; a.gg = dg; a.gbeta = dbeta; a.gs0 = d_state_in;
    a.ws = static_cast<float*>(workspace);
    return check_hip(kda::launch_chunk_bwd(a, s), s, name);
}

int kda_decode_step_ex(const void* q, const void* k, const void* v, const float* g, const void* beta,
                       const float* state_in, float* state_out, float* out, int32_t N, int32_t H, int32_t d_k,
                       int32_t d_v, int32_t dtype, const kda_options* options, void* hip_stream) {
    static const char* name = "kda_decode_step";
    Opts op;
    if (int rc = read_options(options, KDA_OP_DECODE, name, op)) return rc;
    if (N < 0) return fail(KDA_ERR_INVALID_ARG, "%s: N must be >= 0", name);
    if (int rc = validate_common(q, k, v, g, beta, N, H, d_k, d_v, dtype, 1, op.gate_head)) return rc;
    if (!kda::decode_supported(d_k, d_v))
        return fail(KDA_ERR_UNSUPPORTED, "%s: d_k=%d d_v=%d not implemented", name, d_k, d_v);
    if (N > 0 && (!state_in || !state_out || !out))
        return fail(KDA_ERR_INVALID_ARG, "%s: state_in, state_out and out are required", name);
    if (!aligned_to(out, 4) || !aligned16(state_in) || !aligned16(state_out))
        return fail(KDA_ERR_MISALIGNED, "%s: states must be 16-byte aligned, out 4-byte aligned", name);
    const size_t esz = dtype == KDA_BF16 ? 2 : 4;
    const size_t sbytes = (size_t)N * H * d_k * d_v * 4;
    const Span sin{state_in, sbytes}, sout{state_out, sbytes}, o{out, (size_t)N * H * d_v * 4};
    const Span ins[] = {{q, (size_t)N * H * d_k * esz}, {k, (size_t)N * H * d_k * esz}, {v, (size_t)N * H * d_v * esz},
                        {g, (size_t)N * H * (op.gate_head ? 1 : d_k) * 4}, {beta, (size_t)N * H * esz}, sin};
    for (const Span& in : ins)
        if (overlap(o, in) || (overlap(sout, in) && in.p != state_in))
            return fail(KDA_ERR_ALIAS, "%s: out/state_out overlap an input", name);
    if (overlap(o, sout)) return fail(KDA_ERR_ALIAS, "%s: out overlaps state_out", name);
    if (overlap(sin, sout) && state_in != state_out)
        return fail(KDA_ERR_ALIAS, "%s: state_out partially overlaps state_in", name);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    if (debug_check())
        if (int rc = debug_check_gates(g, (size_t)N * H * (op.gate_head ? 1 : d_k), beta, (size_t)N * H, dtype,
                                       op.prologue, s, name))
            return rc;
    if (injected_launch_failure()) return fail(KDA_ERR_HIP, "%s: injected launch failure (KDA_TEST_FAIL_LAUNCH)", name);
    kda::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.s_in = state_in; a.s_out = state_out; a.o = out;
    a.N = N; a.H = H; a.dk = d_k; a.dv = d_v; a.bf16 = dtype == KDA_BF16; a.gate_head = op.gate_head;
    a.prologue = op.prologue; a.gate_scale = op.gate_scale;
    return check_hip(kda::launch_decode(a, s), s, name);
}

int kda_decode_step(const void* q, const void* k, const void* v, const float* g, const void* beta,
                    const float* state_in, float* state_out, float* out, int32_t N, int32_t H, int32_t d_k,
                    int32_t d_v, int32_t dtype, void* hip_stream) {
    return kda_decode_step_ex(q, k, v, g, beta, state_in, state_out, out, N, H, d_k, d_v, dtype, nullptr,
                              hip_stream);
}

}  // extern "C"
