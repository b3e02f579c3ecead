/*
 * Seeded, counter-based synthetic input generator for the KDA workloads.
 *
 * This file holds no arithmetic of the method itself: it only draws the
 * tensors the method consumes (queries, keys, values, write strengths,
 * log-decays, carried states, segment lengths).  Both the GPU path and the
 * CPU oracle are fed from these bits; neither is implemented here.
 *
 * Random numbers: SplitMix64's output mixer (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014, with the
 * 64-bit finaliser constants used by its published implementation) applied to
 * a counter.  Element i of a tensor depends only on (seed, tensor id, i), so
 * any slice can be regenerated without producing the rest, and the result does
 * not depend on the number of threads.
 *
 *   key(seed, id)   = mix(seed * G + mix(id + K0))
 *   uniform(key, c) = ((mix(key + (c + 1) * G) >> 11) + 0.5) * 2^-53   in (0, 1)
 *   normal(key, i)  = sqrt(-2 ln u0) * cos(2 pi u1),  u0 = uniform(key, 2i),
 *                     u1 = uniform(key, 2i + 1)        (Box-Muller, one output)
 *
 * Values are produced in fp64, then rounded once to fp32 (round to nearest
 * even), and from fp32 to bfloat16 (round to nearest even) when asked.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t id) {
    return mix64(seed * GOLDEN + mix64(id + 0x632BE59BD9B4E019ULL));
}

static inline double uniform01(uint64_t key, uint64_t ctr) {
    uint64_t z = mix64(key + (ctr + 1) * GOLDEN);
    return ((double)(z >> 11) + 0.5) * 0x1.0p-53;
}

static inline double normal01(uint64_t key, uint64_t idx) {
    double u0 = uniform01(key, 2 * idx), u1 = uniform01(key, 2 * idx + 1);
    return sqrt(-2.0 * log(u0)) * cos(2.0 * M_PI * u1);
}

static inline double softplus(double x) {
    return x > 0 ? x + log1p(exp(-x)) : log1p(exp(x));
}

/* fp32 -> bfloat16 bits, round to nearest even (NaN kept quiet). */
static inline uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

enum { K_NORMAL = 0, K_UNIT_ROWS = 1, K_SIGMOID_NORMAL = 2, K_LOGDECAY_SOFTPLUS = 3,
       K_LOGDECAY_RATE = 4, K_UNIFORM = 5, K_UNIFORM_INT = 6 };
enum { OUT_F64 = 0, OUT_F32 = 1, OUT_BF16 = 2, OUT_I32 = 3 };

typedef struct {
    int kind, out_dtype;
    uint64_t key, key2;
    int64_t count, row_len, heads, offset;
    double p0, p1, p2, p3;
    void* out;
    int64_t lo, hi; /* element range [lo, hi) of this worker */
} job_t;

static void store(const job_t* j, int64_t i, double x) {
    switch (j->out_dtype) {
    case OUT_F64: ((double*)j->out)[i] = x; break;
    case OUT_F32: ((float*)j->out)[i] = (float)x; break;
    case OUT_BF16: ((uint16_t*)j->out)[i] = f32_to_bf16((float)x); break;
    case OUT_I32: ((int32_t*)j->out)[i] = (int32_t)x; break;
    }
}

static void* worker(void* arg) {
    const job_t* j = (const job_t*)arg;
    if (j->kind == K_UNIT_ROWS) {
        /* lo/hi are row indices here */
        double* row = (double*)malloc(sizeof(double) * (size_t)j->row_len);
        for (int64_t r = j->lo; r < j->hi; ++r) {
            int64_t base = (j->offset + r * j->row_len);
            double ss = 0;
            for (int64_t c = 0; c < j->row_len; ++c) {
                row[c] = normal01(j->key, (uint64_t)(base + c));
                ss += row[c] * row[c];
            }
            double inv = 1.0 / sqrt(ss);
            for (int64_t c = 0; c < j->row_len; ++c) store(j, r * j->row_len + c, row[c] * inv);
        }
        free(row);
        return NULL;
    }
    for (int64_t i = j->lo; i < j->hi; ++i) {
        uint64_t gi = (uint64_t)(j->offset + i);
        double x = 0;
        switch (j->kind) {
        case K_NORMAL: x = j->p1 + j->p0 * normal01(j->key, gi); break;
        case K_SIGMOID_NORMAL: x = 1.0 / (1.0 + exp(-normal01(j->key, gi))); break;
        case K_LOGDECAY_SOFTPLUS: x = -j->p0 * softplus(normal01(j->key, gi)); break;
        case K_LOGDECAY_RATE: {
            /* per-(head, channel) rate r ~ U(p0, p1) from its own stream */
            int64_t c = (int64_t)(gi % (uint64_t)j->row_len);
            int64_t h = (int64_t)((gi / (uint64_t)j->row_len) % (uint64_t)j->heads);
            double r = j->p0 + (j->p1 - j->p0) * uniform01(j->key2, (uint64_t)(h * j->row_len + c));
            x = -softplus(normal01(j->key, gi)) * r;
            break;
        }
        case K_UNIFORM: x = j->p0 + (j->p1 - j->p0) * uniform01(j->key, gi); break;
        case K_UNIFORM_INT: {
            double span = j->p1 - j->p0 + 1.0;
            double v = floor(uniform01(j->key, gi) * span);
            if (v > span - 1) v = span - 1;
            x = j->p0 + v;
            break;
        }
        }
        store(j, i, x);
    }
    return NULL;
}

/*
 * Fill `out` with `count` elements of the recipe `kind`, as elements
 * offset .. offset+count-1 of the tensor (seed, tensor_id).
 *   K_NORMAL            p0 = std, p1 = mean
 *   K_UNIT_ROWS         N(0,1) rows of length row_len, each scaled to unit L2 norm in fp64
 *   K_SIGMOID_NORMAL    1 / (1 + exp(-N(0,1)))
 *   K_LOGDECAY_SOFTPLUS -p0 * softplus(N(0,1))
 *   K_LOGDECAY_RATE     -softplus(N(0,1)) * r[h, c], r ~ U(p0, p1) drawn once per (head, channel)
 *                        from stream (seed, tensor_id2); row_len = channels, heads = H
 *   K_UNIFORM           U(p0, p1)
 *   K_UNIFORM_INT       integer uniform on [p0, p1] inclusive
 * Returns 0 on success, -1 on a bad argument.
 */
int synth_fill(int kind, uint64_t seed, uint64_t tensor_id, uint64_t tensor_id2, int64_t offset,
               int64_t count, int64_t row_len, int64_t heads, double p0, double p1, int out_dtype,
               void* out, int nthreads) {
    if (count < 0 || offset < 0 || !out || out_dtype < 0 || out_dtype > 3) return -1;
    if ((kind == K_UNIT_ROWS || kind == K_LOGDECAY_RATE) && row_len <= 0) return -1;
    if (kind == K_UNIT_ROWS && (count % row_len || offset % row_len)) return -1;
    if (kind == K_LOGDECAY_RATE && heads <= 0) return -1;
    if (count == 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    int64_t units = kind == K_UNIT_ROWS ? count / row_len : count;
    if (units < 4096 * (int64_t)nthreads) nthreads = (int)(units / 4096) + 1;
    pthread_t th[256];
    job_t jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        job_t* j = &jobs[t];
        memset(j, 0, sizeof(*j));
        j->kind = kind;
        j->out_dtype = out_dtype;
        j->key = stream_key(seed, tensor_id);
        j->key2 = stream_key(seed, tensor_id2);
        j->count = count;
        j->row_len = row_len;
        j->heads = heads;
        j->offset = offset;
        j->p0 = p0;
        j->p1 = p1;
        j->out = out;
        j->lo = units * t / nthreads;
        j->hi = units * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, worker, &jobs[t]);
    worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    return 0;
}

/* Raw uniform draws, exposed so that tests can check the mixer against its definition. */
void synth_uniform_raw(uint64_t seed, uint64_t tensor_id, uint64_t start, int64_t count, double* out) {
    uint64_t key = stream_key(seed, tensor_id);
    for (int64_t i = 0; i < count; ++i) out[i] = uniform01(key, start + (uint64_t)i);
}

uint64_t synth_mix64(uint64_t z) { return mix64(z); }
