/*
 * fp64 CPU oracle for the Kimi Delta Attention (KDA) gated delta rule.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU path never calls,
 * links or includes it, and it shares no code with the GPU path.
 *
 * Sources ("Kimi K3, explained", vibeengines.com):
 *   - "How Kimi Delta Attention works, step by step": decay each key channel
 *     by alpha_t, erase a beta_t share of what the decayed state returns for
 *     k_t, write beta_t * (value) * (key), read with the query from the updated
 *     state.
 *   - "The math", the gated delta rule equation, written there for a state of
 *     size d_v x d_k.  This file keeps the transposed state S in R^{d_k x d_v}
 *     (row = key channel, column = value channel, value index contiguous):
 *         S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *         o_t = S_t^T q_t
 *     which is the page's equation transposed.
 *   - "Training in chunks" / "How is KDA trained efficiently if it is a
 *     recurrence?": the chunked form only reorganises the same product of
 *     per-token transitions, so its result is the recurrence's.
 *
 * alpha_t is passed as its natural log g_t = log(alpha_t) (one value per key
 * channel), so alpha_t = exp(g_t).  All arithmetic is fp64.
 *
 * Layouts (row-major, contiguous):
 *   q, k  [T_total, H, dk]    v [T_total, H, dv]    g [T_total, H, dk]
 *   beta  [T_total, H]        s0, sT [N, H, dk, dv] o [T_total, H, dv]
 *   cu    [N + 1] token offsets of the N packed sequences (cu[0] = 0).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *g, *beta, *s0;
    const int64_t* cu;
    double *o, *sT;
    int64_t snap_every;      /* tokens between state snapshots (0: none) */
    const int64_t* snap_cu;  /* first snapshot row of each sequence */
    double* snaps;           /* [snap_cu[N], H, dk, dv] */
    /* reverse mode (O3): upstream gradients in, input gradients out */
    const double *dO, *dsT;
    double *dq, *dk_, *dv_, *dg, *dbeta, *ds0;
    int64_t N, H, dk, dv, chunk;
    int64_t vcols; /* value columns per work unit */
    int64_t nunits;
    int64_t next;  /* shared work counter */
    pthread_mutex_t mu;
    int err;
} ctx_t;

static int64_t take_unit(ctx_t* c) {
    pthread_mutex_lock(&c->mu);
    int64_t u = c->next < c->nunits ? c->next++ : -1;
    pthread_mutex_unlock(&c->mu);
    return u;
}

/*
 * O1 — one (sequence n, head h, value columns [j0, j1)) unit of the token
 * recurrence.  Value columns evolve independently (each column j of S only
 * ever meets column j of v), so splitting them across threads changes nothing.
 */
static void recurrence_unit(ctx_t* c, int64_t n, int64_t h, int64_t j0, int64_t j1) {
    const int64_t H = c->H, dk = c->dk, dv = c->dv, w = j1 - j0;
    double* S = (double*)calloc((size_t)(dk * w), sizeof(double));
    double* a = (double*)malloc(sizeof(double) * (size_t)dk);
    if (!S || !a) { c->err = 1; free(S); free(a); return; }
    if (c->s0)
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < w; ++j) S[i * w + j] = c->s0[((n * H + h) * dk + i) * dv + j0 + j];
    for (int64_t t = c->cu[n]; t < c->cu[n + 1]; ++t) {
        const double* qt = c->q + (t * H + h) * dk;
        const double* kt = c->k + (t * H + h) * dk;
        const double* vt = c->v + (t * H + h) * dv;
        const double* gt = c->g + (t * H + h) * dk;
        const double bt = c->beta[t * H + h];
        /* decay: multiply the state by Diag(alpha_t) along the key dimension */
        for (int64_t i = 0; i < dk; ++i) a[i] = exp(gt[i]);
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < w; ++j) S[i * w + j] *= a[i];
        for (int64_t j = 0; j < w; ++j) {
            /* erase: what the decayed state returns for k_t, in column j */
            double u = 0;
            for (int64_t i = 0; i < dk; ++i) u += kt[i] * S[i * w + j];
            /* erase a beta_t share of it and write beta_t * v_t under k_t */
            double d = bt * (vt[j0 + j] - u);
            for (int64_t i = 0; i < dk; ++i) S[i * w + j] += kt[i] * d;
            /* read the updated state with the query */
            double o = 0;
            for (int64_t i = 0; i < dk; ++i) o += qt[i] * S[i * w + j];
            c->o[(t * H + h) * dv + j0 + j] = o;
        }
        /* snapshot: the state after every snap_every tokens of the sequence */
        const int64_t done = t - c->cu[n] + 1;
        if (c->snaps && done % c->snap_every == 0) {
            double* dst = c->snaps + ((c->snap_cu[n] + done / c->snap_every - 1) * H + h) * dk * dv;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < w; ++j) dst[i * dv + j0 + j] = S[i * w + j];
        }
    }
    if (c->sT)
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < w; ++j) c->sT[((n * H + h) * dk + i) * dv + j0 + j] = S[i * w + j];
    free(S);
    free(a);
}

/*
 * O2 — the chunked form in fp64, used only to check that the chunk algebra
 * reaches the recurrence's result.  Within a chunk of L tokens (rows r, s),
 * with G[r] = sum_{s<=r} g_s (per key channel, restarting at the chunk) and
 * S0 the state entering the chunk:
 *   A[r,s]  = beta_r sum_c k_rc k_sc exp(G_rc - G_sc)   (s < r)
 *   M[r,s]  =        sum_c q_rc k_sc exp(G_rc - G_sc)   (s <= r)
 *   T       = (I + A)^{-1}                              (forward substitution)
 *   D       = T Diag(beta) (V - K+ S0),  K+[r,c] = k_rc exp(G_rc)
 *   O       = Q+ S0 + M D,               Q+[r,c] = q_rc exp(G_rc)
 *   S_next  = Diag(exp(G_L)) S0 + K'^T D, K'[s,c] = k_sc exp(G_Lc - G_sc)
 * The pairwise exponentials are evaluated directly, one per (r, s, c).
 */
static void chunked_unit(ctx_t* c, int64_t n, int64_t h) {
    const int64_t H = c->H, dk = c->dk, dv = c->dv, C = c->chunk;
    double* S = (double*)calloc((size_t)(dk * dv), sizeof(double));
    double* G = (double*)malloc(sizeof(double) * (size_t)(C * dk));
    double* A = (double*)malloc(sizeof(double) * (size_t)(C * C));
    double* M = (double*)malloc(sizeof(double) * (size_t)(C * C));
    double* Tm = (double*)malloc(sizeof(double) * (size_t)(C * C));
    double* R = (double*)malloc(sizeof(double) * (size_t)(C * dv));
    double* D = (double*)malloc(sizeof(double) * (size_t)(C * dv));
    double* Sn = (double*)malloc(sizeof(double) * (size_t)(dk * dv));
    if (!S || !G || !A || !M || !Tm || !R || !D || !Sn) { c->err = 1; goto done; }
    if (c->s0) memcpy(S, c->s0 + (n * H + h) * dk * dv, sizeof(double) * (size_t)(dk * dv));
    for (int64_t t0 = c->cu[n]; t0 < c->cu[n + 1]; t0 += C) {
        int64_t L = c->cu[n + 1] - t0 < C ? c->cu[n + 1] - t0 : C;
#define Q_(r, i) c->q[((t0 + (r)) * H + h) * dk + (i)]
#define K_(r, i) c->k[((t0 + (r)) * H + h) * dk + (i)]
#define V_(r, j) c->v[((t0 + (r)) * H + h) * dv + (j)]
#define B_(r) c->beta[(t0 + (r)) * H + h]
        for (int64_t i = 0; i < dk; ++i) {
            double acc = 0;
            for (int64_t r = 0; r < L; ++r) {
                acc += c->g[((t0 + r) * H + h) * dk + i];
                G[r * dk + i] = acc;
            }
        }
        for (int64_t r = 0; r < L; ++r)
            for (int64_t s = 0; s < L; ++s) {
                double a = 0, m = 0;
                if (s <= r)
                    for (int64_t i = 0; i < dk; ++i) {
                        double e = exp(G[r * dk + i] - G[s * dk + i]);
                        a += K_(r, i) * K_(s, i) * e;
                        m += Q_(r, i) * K_(s, i) * e;
                    }
                A[r * C + s] = s < r ? B_(r) * a : 0.0;
                M[r * C + s] = s <= r ? m : 0.0;
            }
        /* T = (I + A)^{-1}: unit lower triangular, column by column */
        for (int64_t j = 0; j < L; ++j)
            for (int64_t r = 0; r < L; ++r) {
                if (r < j) { Tm[r * C + j] = 0; continue; }
                if (r == j) { Tm[r * C + j] = 1; continue; }
                double acc = 0;
                for (int64_t s = j; s < r; ++s) acc += A[r * C + s] * Tm[s * C + j];
                Tm[r * C + j] = -acc;
            }
        /* R = Diag(beta) (V - K+ S0) */
        for (int64_t r = 0; r < L; ++r)
            for (int64_t j = 0; j < dv; ++j) {
                double ks = 0;
                for (int64_t i = 0; i < dk; ++i) ks += K_(r, i) * exp(G[r * dk + i]) * S[i * dv + j];
                R[r * dv + j] = B_(r) * (V_(r, j) - ks);
            }
        /* D = T R */
        for (int64_t r = 0; r < L; ++r)
            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0;
                for (int64_t s = 0; s <= r; ++s) acc += Tm[r * C + s] * R[s * dv + j];
                D[r * dv + j] = acc;
            }
        /* O = Q+ S0 + M D */
        for (int64_t r = 0; r < L; ++r)
            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0;
                for (int64_t i = 0; i < dk; ++i) acc += Q_(r, i) * exp(G[r * dk + i]) * S[i * dv + j];
                for (int64_t s = 0; s <= r; ++s) acc += M[r * C + s] * D[s * dv + j];
                c->o[((t0 + r) * H + h) * dv + j] = acc;
            }
        /* S_next = Diag(exp(G_L)) S0 + K'^T D */
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) {
                double acc = exp(G[(L - 1) * dk + i]) * S[i * dv + j];
                for (int64_t s = 0; s < L; ++s)
                    acc += K_(s, i) * exp(G[(L - 1) * dk + i] - G[s * dk + i]) * D[s * dv + j];
                Sn[i * dv + j] = acc;
            }
        memcpy(S, Sn, sizeof(double) * (size_t)(dk * dv));
#undef Q_
#undef K_
#undef V_
#undef B_
    }
    if (c->sT) memcpy(c->sT + (n * H + h) * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
done:
    free(S); free(G); free(A); free(M); free(Tm); free(R); free(D); free(Sn);
}

/*
 * One token of O1 on a whole state (rows i < dk, columns j < dv), keeping what
 * the reverse sweep needs: X = Diag(alpha_t) S_{t-1}, u = X^T k_t and
 * delta = beta_t (v_t - u).  S is advanced to S_t in place.
 */
static void step_token(const ctx_t* c, int64_t t, int64_t h, double* S, double* X, double* u, double* delta) {
    const int64_t H = c->H, dk = c->dk, dv = c->dv;
    const double* kt = c->k + (t * H + h) * dk;
    const double* vt = c->v + (t * H + h) * dv;
    const double* gt = c->g + (t * H + h) * dk;
    const double bt = c->beta[t * H + h];
    for (int64_t i = 0; i < dk; ++i) {
        const double a = exp(gt[i]);
        for (int64_t j = 0; j < dv; ++j) X[i * dv + j] = a * S[i * dv + j];
    }
    for (int64_t j = 0; j < dv; ++j) {
        double acc = 0;
        for (int64_t i = 0; i < dk; ++i) acc += kt[i] * X[i * dv + j];
        u[j] = acc;
        delta[j] = bt * (vt[j] - acc);
    }
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) S[i * dv + j] = X[i * dv + j] + kt[i] * delta[j];
}

/*
 * O3 — reverse-mode derivative of O1 for one (sequence n, head h).  Given the
 * upstream gradients dL/do_t (dO) and dL/dS_T (dsT, NULL = 0), it returns
 * dL/dq, dL/dk, dL/dv, dL/dg (g = log alpha), dL/dbeta and dL/dS_0.  Written
 * from the four lines of one token, taken backwards (S the state after the
 * token, dS its gradient):
 *   o = S^T q             dq = S do;           dS += q do^T
 *   S = X + k delta^T     dk += dS delta;      ddelta = dS^T k;   dX = dS
 *   delta = beta (v - u)  dbeta = ddelta.(v - u); dv = beta ddelta; du = -beta ddelta
 *   u = X^T k             dk += X du;          dX += k du^T
 *   X = Diag(alpha) S'    dg_i = sum_j dX_ij X_ij;  dS' = Diag(alpha) dX
 * The states S_{t-1} come from a forward sweep that keeps the state at the
 * start of every block of `blk` tokens and re-steps each block when the
 * reverse sweep reaches it (the same arithmetic, so the same states).
 */
static void backward_unit(ctx_t* c, int64_t n, int64_t h) {
    const int64_t H = c->H, dk = c->dk, dv = c->dv, t0 = c->cu[n], L = c->cu[n + 1] - t0;
    const int64_t blk = 64, nblk = (L + blk - 1) / blk, sz = dk * dv;
    double* ck = (double*)malloc(sizeof(double) * (size_t)((nblk > 0 ? nblk : 1) * sz));
    double* st = (double*)malloc(sizeof(double) * (size_t)(blk * sz)); /* S_{t-1} of each token of a block */
    double* S = (double*)calloc((size_t)sz, sizeof(double));
    double* X = (double*)malloc(sizeof(double) * (size_t)sz);
    double* dS = (double*)calloc((size_t)sz, sizeof(double));
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    double* delta = (double*)malloc(sizeof(double) * (size_t)dv);
    double* dd = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!ck || !st || !S || !X || !dS || !u || !delta || !dd) { c->err = 1; goto done; }
    if (c->s0) memcpy(S, c->s0 + (n * H + h) * sz, sizeof(double) * (size_t)sz);
    for (int64_t b = 0; b < nblk; ++b) {
        memcpy(ck + b * sz, S, sizeof(double) * (size_t)sz);
        for (int64_t t = t0 + b * blk; t < t0 + L && t < t0 + (b + 1) * blk; ++t) step_token(c, t, h, S, X, u, delta);
    }
    if (c->dsT) memcpy(dS, c->dsT + (n * H + h) * sz, sizeof(double) * (size_t)sz);
    for (int64_t b = nblk - 1; b >= 0; --b) {
        const int64_t ta = t0 + b * blk, tb = ta + blk < t0 + L ? ta + blk : t0 + L;
        memcpy(S, ck + b * sz, sizeof(double) * (size_t)sz);
        for (int64_t t = ta; t < tb; ++t) {
            memcpy(st + (t - ta) * sz, S, sizeof(double) * (size_t)sz);
            step_token(c, t, h, S, X, u, delta);
        }
        for (int64_t t = tb - 1; t >= ta; --t) {
            /* recompute this token from S_{t-1}: S becomes S_t, X, u and delta as in the forward */
            memcpy(S, st + (t - ta) * sz, sizeof(double) * (size_t)sz);
            step_token(c, t, h, S, X, u, delta);
            const double* qt = c->q + (t * H + h) * dk;
            const double* kt = c->k + (t * H + h) * dk;
            const double* vt = c->v + (t * H + h) * dv;
            const double* gt = c->g + (t * H + h) * dk;
            const double* dot = c->dO + (t * H + h) * dv;
            const double bt = c->beta[t * H + h];
            double* dqt = c->dq + (t * H + h) * dk;
            double* dkt = c->dk_ + (t * H + h) * dk;
            double* dvt = c->dv_ + (t * H + h) * dv;
            double* dgt = c->dg + (t * H + h) * dk;
            /* read: o = S_t^T q */
            for (int64_t i = 0; i < dk; ++i) {
                double acc = 0;
                for (int64_t j = 0; j < dv; ++j) {
                    acc += S[i * dv + j] * dot[j];
                    dS[i * dv + j] += qt[i] * dot[j];
                }
                dqt[i] = acc;
            }
            /* write: S_t = X + k delta^T */
            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0;
                for (int64_t i = 0; i < dk; ++i) acc += kt[i] * dS[i * dv + j];
                dd[j] = acc;
            }
            for (int64_t i = 0; i < dk; ++i) {
                double acc = 0;
                for (int64_t j = 0; j < dv; ++j) acc += dS[i * dv + j] * delta[j];
                dkt[i] = acc;
            }
            /* erase: delta = beta (v - u) */
            double db = 0;
            for (int64_t j = 0; j < dv; ++j) {
                db += dd[j] * (vt[j] - u[j]);
                dvt[j] = bt * dd[j];
                dd[j] = -bt * dd[j]; /* now du */
            }
            c->dbeta[t * H + h] = db;
            /* u = X^T k: into dk and into dX (held in dS) */
            for (int64_t i = 0; i < dk; ++i) {
                double acc = 0;
                for (int64_t j = 0; j < dv; ++j) {
                    acc += X[i * dv + j] * dd[j];
                    dS[i * dv + j] += kt[i] * dd[j];
                }
                dkt[i] += acc;
            }
            /* decay: X = Diag(alpha) S_{t-1} */
            for (int64_t i = 0; i < dk; ++i) {
                const double a = exp(gt[i]);
                double acc = 0;
                for (int64_t j = 0; j < dv; ++j) {
                    acc += dS[i * dv + j] * X[i * dv + j];
                    dS[i * dv + j] *= a;
                }
                dgt[i] = acc;
            }
        }
    }
    if (c->ds0) memcpy(c->ds0 + (n * H + h) * sz, dS, sizeof(double) * (size_t)sz);
done:
    free(ck); free(st); free(S); free(X); free(dS); free(u); free(delta); free(dd);
}

static void* backward_worker(void* arg) {
    ctx_t* c = (ctx_t*)arg;
    for (int64_t u; (u = take_unit(c)) >= 0;) backward_unit(c, u / c->H, u % c->H);
    return NULL;
}

static void* recurrence_worker(void* arg) {
    ctx_t* c = (ctx_t*)arg;
    const int64_t nvb = (c->dv + c->vcols - 1) / c->vcols;
    for (int64_t u; (u = take_unit(c)) >= 0;) {
        int64_t vb = u % nvb, nh = u / nvb;
        int64_t j0 = vb * c->vcols, j1 = j0 + c->vcols < c->dv ? j0 + c->vcols : c->dv;
        recurrence_unit(c, nh / c->H, nh % c->H, j0, j1);
    }
    return NULL;
}

static void* chunked_worker(void* arg) {
    ctx_t* c = (ctx_t*)arg;
    for (int64_t u; (u = take_unit(c)) >= 0;) chunked_unit(c, u / c->H, u % c->H);
    return NULL;
}

static int run(ctx_t* c, void* (*fn)(void*), int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 512) nthreads = 512;
    if (nthreads > c->nunits) nthreads = (int)(c->nunits > 0 ? c->nunits : 1);
    pthread_mutex_init(&c->mu, NULL);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, fn, c);
    fn(c);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
    pthread_mutex_destroy(&c->mu);
    return c->err ? -2 : 0;
}

static int check(const int64_t* cu, int64_t N, int64_t H, int64_t dk, int64_t dv) {
    if (!cu || N < 0 || H <= 0 || dk <= 0 || dv <= 0 || cu[0] != 0) return -1;
    for (int64_t n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n]) return -1;
    return 0;
}

/*
 * Token-by-token recurrence (the oracle).  s0 may be NULL (zero state), sT may
 * be NULL.  vcols > 0 splits value columns into work units of that width for
 * threading (0 = whole rows).  Returns 0, -1 on a bad argument, -2 on OOM.
 */
/*
 * O1 with state snapshots: snaps receives the state after every snap_every
 * tokens of each sequence (snapshot m of sequence n, the state after its first
 * (m + 1) * snap_every tokens, at row snap_cu[n] + m); snap_every = 0 or
 * snaps = NULL: no snapshots.
 */
int kda_oracle_recurrence_snap(const double* q, const double* k, const double* v, const double* g,
                               const double* beta, const int64_t* cu, int64_t N, const double* s0, double* o,
                               double* sT, int64_t H, int64_t dk, int64_t dv, int64_t vcols, int nthreads,
                               int64_t snap_every, const int64_t* snap_cu, double* snaps) {
    if (check(cu, N, H, dk, dv) || (cu[N] > 0 && (!q || !k || !v || !g || !beta || !o))) return -1;
    if (snap_every < 0 || (snap_every > 0 && snaps && !snap_cu)) return -1;
    ctx_t c;
    memset(&c, 0, sizeof(c));
    c.q = q; c.k = k; c.v = v; c.g = g; c.beta = beta; c.s0 = s0; c.cu = cu; c.o = o; c.sT = sT;
    c.snap_every = snap_every; c.snap_cu = snap_cu; c.snaps = snap_every > 0 ? snaps : NULL;
    c.N = N; c.H = H; c.dk = dk; c.dv = dv;
    c.vcols = vcols > 0 && vcols < dv ? vcols : dv;
    c.nunits = N * H * ((dv + c.vcols - 1) / c.vcols);
    return run(&c, recurrence_worker, nthreads);
}

int kda_oracle_recurrence(const double* q, const double* k, const double* v, const double* g,
                          const double* beta, const int64_t* cu, int64_t N, const double* s0, double* o,
                          double* sT, int64_t H, int64_t dk, int64_t dv, int64_t vcols, int nthreads) {
    return kda_oracle_recurrence_snap(q, k, v, g, beta, cu, N, s0, o, sT, H, dk, dv, vcols, nthreads, 0, NULL,
                                      NULL);
}

/* Chunked fp64 algebra (check of the chunked form only).  chunk >= 1. */
int kda_oracle_chunked(const double* q, const double* k, const double* v, const double* g,
                       const double* beta, const int64_t* cu, int64_t N, const double* s0, double* o,
                       double* sT, int64_t H, int64_t dk, int64_t dv, int64_t chunk, int nthreads) {
    if (check(cu, N, H, dk, dv) || chunk < 1 || (cu[N] > 0 && (!q || !k || !v || !g || !beta || !o))) return -1;
    ctx_t c;
    memset(&c, 0, sizeof(c));
    c.q = q; c.k = k; c.v = v; c.g = g; c.beta = beta; c.s0 = s0; c.cu = cu; c.o = o; c.sT = sT;
    c.N = N; c.H = H; c.dk = dk; c.dv = dv; c.chunk = chunk;
    c.nunits = N * H;
    return run(&c, chunked_worker, nthreads);
}

/*
 * O3: gradients of the recurrence.  dO [T_total, H, dv] is required; dsT
 * [N, H, dk, dv] may be NULL (zero).  dq, dk, dg [T_total, H, dk], dv
 * [T_total, H, dv] and dbeta [T_total, H] are written; ds0 [N, H, dk, dv] may
 * be NULL.  s0 may be NULL (zero initial state).
 */
int kda_oracle_backward(const double* q, const double* k, const double* v, const double* g, const double* beta,
                        const int64_t* cu, int64_t N, const double* s0, const double* dO, const double* dsT,
                        double* dq, double* dk, double* dv_out, double* dg, double* dbeta, double* ds0, int64_t H,
                        int64_t dk_dim, int64_t dv, int nthreads) {
    if (check(cu, N, H, dk_dim, dv) ||
        (cu[N] > 0 && (!q || !k || !v || !g || !beta || !dO || !dq || !dk || !dv_out || !dg || !dbeta)))
        return -1;
    ctx_t c;
    memset(&c, 0, sizeof(c));
    c.q = q; c.k = k; c.v = v; c.g = g; c.beta = beta; c.s0 = s0; c.cu = cu;
    c.dO = dO; c.dsT = dsT; c.dq = dq; c.dk_ = dk; c.dv_ = dv_out; c.dg = dg; c.dbeta = dbeta; c.ds0 = ds0;
    c.N = N; c.H = H; c.dk = dk_dim; c.dv = dv;
    c.nunits = N * H;
    return run(&c, backward_worker, nthreads);
}

/*
 * Contrast only ("The delta: overwrite, don't accumulate"): plain linear
 * attention, S <- S + k v^T and o = S^T q, for one head of T tokens.  It has
 * no erase, so two writes under one key read back their sum.
 */
int kda_oracle_linear_attention(const double* q, const double* k, const double* v, int64_t T, int64_t dk,
                                int64_t dv, const double* s0, double* o, double* sT) {
    if (T < 0 || dk <= 0 || dv <= 0 || (T > 0 && (!q || !k || !v || !o))) return -1;
    double* S = (double*)calloc((size_t)(dk * dv), sizeof(double));
    if (!S) return -2;
    if (s0) memcpy(S, s0, sizeof(double) * (size_t)(dk * dv));
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += k[t * dk + i] * v[t * dv + j];
        for (int64_t j = 0; j < dv; ++j) {
            double acc = 0;
            for (int64_t i = 0; i < dk; ++i) acc += q[t * dk + i] * S[i * dv + j];
            o[t * dv + j] = acc;
        }
    }
    if (sT) memcpy(sT, S, sizeof(double) * (size_t)(dk * dv));
    free(S);
    return 0;
}
