/*
 * kda_oracle.c -- plain, slow, CPU reference for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * HIP path.
 *
 * Everything is computed in fp64, token by token, in the order the source
 * pages state it.  Page labels used in the citations below:
 *   [kda.rs]   "atlas_core/kimi_k3/kda.rs" (Kimi K3 KDA CPU reference page):
 *              module doc "Recurrence", conv_update, softplus, bounded_gate,
 *              l2norm_rows, kda_recurrent_step, kda_decode_token, and its tests.
 *   [api.py]   "K3/kda/ops/api.py" (training-facing chunk_kda boundary page):
 *              chunk_kda argument list, flag semantics and gate formulas.
 *   [Primus]   "KDA <=> FLA Parity in Primus": section "What changed and why",
 *              table A (in-kernel gate fused with its cumulative sum).
 *   [kda.rs] also gives full_rank_output_gate, the per-head gated RMS norm
 *              of the output; "memra-engine kda_fixture_gpu.rs" gives its eps.
 *
 * Parity status of every function is given in its comment; all of them are
 * pinned by the CPU tests (hand-worked recurrence, closed forms, invariants,
 * naive-vs-chunked agreement and central finite differences).
 *
 * Layouts (row-major, last index fastest):
 *   q, k, g [rows, H, K]   v, o [rows, H, V]   beta [rows, H]
 *   state   [N, H, K, V]   (key index major: S[kk*V + vv])
 * "rows" is B*T for dense input (sequence n occupies rows n*T .. n*T+T-1) or
 * the packed token count for variable-length input (sequence n occupies rows
 * cu_seqlens[n] .. cu_seqlens[n+1]-1).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_GATE_LOGDECAY = 0, OR_GATE_SAFE = 1, OR_GATE_SOFTPLUS = 2 };

typedef struct {
    int B, T, H, K, V;
    const int32_t *cu_seqlens; /* host, [N+1] or NULL */
    int N;
    const double *q, *k, *v, *g, *beta;
    const double *A_log;   /* [H] or NULL */
    const double *dt_bias; /* [H*K] or NULL */
    double scale;
    double lower_bound;
    int gate_mode;
    int use_qk_l2norm;
    int use_beta_sigmoid;
    double l2_eps;
    const double *initial_state; /* [N,H,K,V] or NULL */
} or_problem;

/* ------------------------------------------------------------------ */
/* Dense vector / matrix primitives (row-major, K x V matrices S with   */
/* S[kk * V + vv]), so that the recurrence below reads as its matrix     */
/* equations.                                                           */
/* ------------------------------------------------------------------ */
static double la_dot(int n, const double *x, const double *y) {
    double acc = 0.0;
    for (int i = 0; i < n; ++i) acc += x[i] * y[i];
    return acc;
}

/* out = a * x (out may be x) */
static void la_scale(int n, double a, const double *x, double *out) {
    for (int i = 0; i < n; ++i) out[i] = a * x[i];
}

/* out = S^T x  (S is K x V, x has K entries, out has V) */
static void la_tmatvec(int K, int V, const double *S, const double *x, double *out) {
    for (int vv = 0; vv < V; ++vv) out[vv] = 0.0;
    for (int kk = 0; kk < K; ++kk)
        for (int vv = 0; vv < V; ++vv) out[vv] += S[kk * V + vv] * x[kk];
}

/* S = diag(d) S: row kk of S times d[kk] */
static void la_diag_rows(int K, int V, const double *d, double *S) {
    for (int kk = 0; kk < K; ++kk) la_scale(V, d[kk], S + (size_t)kk * V, S + (size_t)kk * V);
}

/* S = S + a b^T */
static void la_rank1(int K, int V, const double *a, const double *b, double *S) {
    for (int kk = 0; kk < K; ++kk)
        for (int vv = 0; vv < V; ++vv) S[kk * V + vv] += a[kk] * b[vv];
}

/* ------------------------------------------------------------------ */
/* Scalar pieces of the prologue                                       */
/* ------------------------------------------------------------------ */

/* Logistic function 1 / (1 + e^-x). */
static double or_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* softplus(x) = log(1 + e^x) ([kda.rs] `softplus`, which evaluates it in an
 * overflow-free form).  Here: for x > 0, log(1 + e^x) = x + log(1 + e^-x); for
 * x <= 0 it is log(1 + e^x) directly; both log1p arguments are in (0, 1]. */
static double or_softplus(double x) { return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x)); }

/* x / ||x||_eps with ||x||_eps = sqrt(x . x + eps): the L2 normalisation of
 * [kda.rs] `l2norm_rows` with the in-kernel eps 1e-6. */
static void or_l2norm(const double *x, int d, double eps, double *out) {
    la_scale(d, 1.0 / sqrt(la_dot(d, x, x) + eps), x, out);
}

/* Per-channel log-decay of head h from the raw gate input x (one token):
 * with the pre-activation z = x + dt_bias (dt_bias indexed [h*K + c], NULL
 * meaning 0, as [api.py] views it with g's trailing shape) and the rate
 * a = exp(A_log_h),
 *   LOGDECAY: g = x                       ([api.py] default path: the decay
 *                                          is passed in log space)
 *   SAFE:     g = lower_bound * sigma(a z) ([kda.rs] bounded_gate with a bound;
 *                                          [api.py] safe_gate branch)
 *   SOFTPLUS: g = -a * softplus(z)        ([kda.rs] bounded_gate without one;
 *                                          [api.py] unbounded branch) */
static void or_gate(const or_problem *P, int h, const double *x, double *g) {
    const int K = P->K;
    if (P->gate_mode == OR_GATE_LOGDECAY) {
        memcpy(g, x, sizeof(double) * K);
        return;
    }
    const double a = exp(P->A_log[h]);
    const double *bias = P->dt_bias ? P->dt_bias + (size_t)h * K : NULL;
    for (int c = 0; c < K; ++c) {
        const double z = x[c] + (bias ? bias[c] : 0.0);
        g[c] = P->gate_mode == OR_GATE_SAFE ? P->lower_bound * or_sigmoid(a * z) : -a * or_softplus(z);
    }
}

static void or_seq_bounds(const or_problem *P, int n, int64_t *start, int64_t *len) {
    if (P->cu_seqlens) {
        *start = P->cu_seqlens[n];
        *len = (int64_t)P->cu_seqlens[n + 1] - P->cu_seqlens[n];
    } else {
        *start = (int64_t)n * P->T;
        *len = P->T;
    }
}

/* Prologue of one token-head: normalised q and k, effective beta and log-decay.
 * [api.py] chunk_kda applies, in this order, the q/k normalisation, the beta
 * sigmoid and the gate transform before the recurrence. */
static void or_prologue(const or_problem *P, int64_t row, int h, double *qh, double *kh,
                        double *b, double *gt) {
    int H = P->H, K = P->K;
    const double *qr = P->q + (row * H + h) * K;
    const double *kr = P->k + (row * H + h) * K;
    if (P->use_qk_l2norm) {
        or_l2norm(qr, K, P->l2_eps, qh);
        or_l2norm(kr, K, P->l2_eps, kh);
    } else {
        memcpy(qh, qr, sizeof(double) * K);
        memcpy(kh, kr, sizeof(double) * K);
    }
    double bb = P->beta[row * H + h];
    *b = P->use_beta_sigmoid ? or_sigmoid(bb) : bb;
    or_gate(P, h, P->g + (row * H + h) * K, gt);
}

/* ------------------------------------------------------------------ */
/* One token of the recurrence, written as the matrix equations of the  */
/* [kda.rs] module doc "Recurrence" (its kda_recurrent_step evaluates   */
/* the same step):                                                      */
/*   S~ = diag(exp(g)) S        the decay acts on the key axis (rows)   */
/*   d  = beta (v - S~^T k)     the delta against the prediction for k  */
/*   S  = S~ + k d^T            the rank-1 write                         */
/*   o  = scale S^T q           the read-out after the write            */
/* p receives S~^T k and d the delta (both kept for the backward).      */
/* ------------------------------------------------------------------ */
static void or_step(int K, int V, double *S, const double *qh, const double *kh,
                    const double *vt, double b, const double *gt, double scale,
                    double *p, double *d, double *o) {
    double *decay = (double *)malloc(sizeof(double) * K);
    for (int kk = 0; kk < K; ++kk) decay[kk] = exp(gt[kk]);
    la_diag_rows(K, V, decay, S);
    free(decay);
    la_tmatvec(K, V, S, kh, p);
    for (int vv = 0; vv < V; ++vv) d[vv] = b * (vt[vv] - p[vv]);
    la_rank1(K, V, kh, d, S);
    if (o) {
        la_tmatvec(K, V, S, qh, o);
        la_scale(V, scale, o, o);
    }
}

/* ------------------------------------------------------------------ */
/* Thread pool over independent (sequence, head) units                 */
/* ------------------------------------------------------------------ */
typedef struct {
    int n_units;
    int next;
    pthread_mutex_t mu;
    void (*fn)(void *ctx, int unit);
    void *ctx;
} or_pool;

static void *or_worker(void *arg) {
    or_pool *pl = (or_pool *)arg;
    for (;;) {
        pthread_mutex_lock(&pl->mu);
        int u = pl->next++;
        pthread_mutex_unlock(&pl->mu);
        if (u >= pl->n_units) break;
        pl->fn(pl->ctx, u);
    }
    return NULL;
}

static void or_parallel(int n_units, int threads, void (*fn)(void *, int), void *ctx) {
    if (threads < 1) threads = 1;
    if (threads > n_units) threads = n_units;
    if (threads <= 1) {
        for (int u = 0; u < n_units; ++u) fn(ctx, u);
        return;
    }
    or_pool pl;
    pl.n_units = n_units;
    pl.next = 0;
    pl.fn = fn;
    pl.ctx = ctx;
    pthread_mutex_init(&pl.mu, NULL);
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * threads);
    for (int i = 0; i < threads; ++i) pthread_create(&tid[i], NULL, or_worker, &pl);
    for (int i = 0; i < threads; ++i) pthread_join(tid[i], NULL);
    free(tid);
    pthread_mutex_destroy(&pl.mu);
}

/* ------------------------------------------------------------------ */
/* Forward, token by token (the definition)                            */
/* ------------------------------------------------------------------ */
typedef struct {
    const or_problem *P;
    double *o;           /* [rows, H, V] */
    double *final_state; /* [N, H, K, V] or NULL */
} or_fwd_ctx;

static void or_fwd_unit(void *vctx, int unit) {
    or_fwd_ctx *C = (or_fwd_ctx *)vctx;
    const or_problem *P = C->P;
    int H = P->H, K = P->K, V = P->V;
    int n = unit / H, h = unit % H;
    int64_t start, len;
    or_seq_bounds(P, n, &start, &len);
    double *S = (double *)calloc((size_t)K * V, sizeof(double));
    double *buf = (double *)malloc(sizeof(double) * (3 * K + 3 * V));
    double *qh = buf, *kh = buf + K, *gt = buf + 2 * K;
    double *p = buf + 3 * K, *d = p + V, *ot = d + V;
    if (P->initial_state) memcpy(S, P->initial_state + ((size_t)n * H + h) * K * V, sizeof(double) * K * V);
    for (int64_t t = 0; t < len; ++t) {
        int64_t row = start + t;
        double b;
        or_prologue(P, row, h, qh, kh, &b, gt);
        or_step(K, V, S, qh, kh, P->v + (row * H + h) * V, b, gt, P->scale, p, d, ot);
        memcpy(C->o + (row * H + h) * V, ot, sizeof(double) * V);
    }
    if (C->final_state) memcpy(C->final_state + ((size_t)n * H + h) * K * V, S, sizeof(double) * K * V);
    free(buf);
    free(S);
}

/* Full forward of chunk_kda's operator boundary ([api.py] chunk_kda: q, k, v,
 * g, beta, A_log, dt_bias, scale, initial_state, output_final_state and the
 * in-kernel flags), computed as the plain recurrence.  Rows that belong to no
 * sequence are left untouched in o. */
int or_chunk_fwd(const or_problem *P, double *o, double *final_state, int threads) {
    or_fwd_ctx C = {P, o, final_state};
    int N = P->cu_seqlens ? P->N : P->B;
    or_parallel(N * P->H, threads, or_fwd_unit, &C);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Forward in chunkwise (WY/UT) form -- an independent second          */
/* derivation used only to pin the recurrence above.                   */
/* [api.py] warns that the chunkwise form relies on (I + tril(A_kk*beta))  */
/* being invertible with unit-norm keys; the form below follows that:  */
/*   G  = inclusive cumulative sum of g inside the chunk               */
/*   A  = beta_i * sum_c k_i k_j exp(G_i - G_j), strictly lower        */
/*   T  = (I + A)^{-1}                                                 */
/*   u  = T (beta v),  w = T (beta k exp(G))                           */
/*   D  = u - w S                                                      */
/*   O  = scale * ((q exp(G)) S + Mqk D),  Mqk lower incl. diagonal    */
/*   S' = diag(exp(G_last)) S + (k exp(G_last - G))^T D                */
/* Exponents are formed pairwise, so every factor is <= 1.             */
/* ------------------------------------------------------------------ */
typedef struct {
    const or_problem *P;
    int chunk;
    double *o;
    double *final_state;
} or_chk_ctx;

static void or_chunked_unit(void *vctx, int unit) {
    or_chk_ctx *C = (or_chk_ctx *)vctx;
    const or_problem *P = C->P;
    int H = P->H, K = P->K, V = P->V, CS = C->chunk;
    int n = unit / H, h = unit % H;
    int64_t start, len;
    or_seq_bounds(P, n, &start, &len);
    size_t KV = (size_t)K * V;
    double *S = (double *)calloc(KV, sizeof(double));
    double *qh = (double *)malloc(sizeof(double) * CS * K);
    double *kh = (double *)malloc(sizeof(double) * CS * K);
    double *G = (double *)malloc(sizeof(double) * CS * K);
    double *gt = (double *)malloc(sizeof(double) * K);
    double *bt = (double *)malloc(sizeof(double) * CS);
    double *A = (double *)malloc(sizeof(double) * CS * CS);
    double *Mq = (double *)malloc(sizeof(double) * CS * CS);
    double *Tm = (double *)malloc(sizeof(double) * CS * CS);
    double *u = (double *)malloc(sizeof(double) * CS * V);
    double *w = (double *)malloc(sizeof(double) * CS * K);
    double *D = (double *)malloc(sizeof(double) * CS * V);
    double *X = (double *)malloc(sizeof(double) * CS * (K > V ? K : V));
    double *Sn = (double *)malloc(sizeof(double) * KV);
    if (P->initial_state) memcpy(S, P->initial_state + ((size_t)n * H + h) * KV, sizeof(double) * KV);

    for (int64_t c0 = 0; c0 < len; c0 += CS) {
        int L = (int)((len - c0) < CS ? (len - c0) : CS);
        for (int i = 0; i < L; ++i) {
            int64_t row = start + c0 + i;
            or_prologue(P, row, h, qh + i * K, kh + i * K, &bt[i], gt);
            for (int c = 0; c < K; ++c) G[i * K + c] = (i ? G[(i - 1) * K + c] : 0.0) + gt[c];
        }
        /* A (strictly lower, beta-scaled) and Mqk (lower incl. diagonal). */
        for (int i = 0; i < L; ++i)
            for (int j = 0; j < L; ++j) {
                double a = 0.0, m = 0.0;
                if (j <= i)
                    for (int c = 0; c < K; ++c) {
                        double e = exp(G[i * K + c] - G[j * K + c]);
                        a += kh[i * K + c] * kh[j * K + c] * e;
                        m += qh[i * K + c] * kh[j * K + c] * e;
                    }
                A[i * CS + j] = (j < i) ? bt[i] * a : 0.0;
                Mq[i * CS + j] = (j <= i) ? m : 0.0;
            }
        /* T = (I + A)^{-1} by forward substitution, column by column. */
        for (int j = 0; j < L; ++j)
            for (int i = 0; i < L; ++i) {
                if (i < j) { Tm[i * CS + j] = 0.0; continue; }
                double acc = (i == j) ? 1.0 : 0.0;
                for (int m = j; m < i; ++m) acc -= A[i * CS + m] * Tm[m * CS + j];
                Tm[i * CS + j] = acc;
            }
        /* u = T (beta v) */
        for (int i = 0; i < L; ++i)
            for (int vv = 0; vv < V; ++vv) X[i * V + vv] = bt[i] * P->v[((start + c0 + i) * H + h) * V + vv];
        for (int i = 0; i < L; ++i)
            for (int vv = 0; vv < V; ++vv) {
                double acc = 0.0;
                for (int m = 0; m <= i; ++m) acc += Tm[i * CS + m] * X[m * V + vv];
                u[i * V + vv] = acc;
            }
        /* w = T (beta k exp(G)) */
        for (int i = 0; i < L; ++i)
            for (int c = 0; c < K; ++c) X[i * K + c] = bt[i] * kh[i * K + c] * exp(G[i * K + c]);
        for (int i = 0; i < L; ++i)
            for (int c = 0; c < K; ++c) {
                double acc = 0.0;
                for (int m = 0; m <= i; ++m) acc += Tm[i * CS + m] * X[m * K + c];
                w[i * K + c] = acc;
            }
        /* D = u - w S */
        for (int i = 0; i < L; ++i)
            for (int vv = 0; vv < V; ++vv) {
                double acc = 0.0;
                for (int c = 0; c < K; ++c) acc += w[i * K + c] * S[c * V + vv];
                D[i * V + vv] = u[i * V + vv] - acc;
            }
        /* O = scale * ((q exp(G)) S + Mqk D) */
        for (int i = 0; i < L; ++i)
            for (int vv = 0; vv < V; ++vv) {
                double acc = 0.0;
                for (int c = 0; c < K; ++c) acc += qh[i * K + c] * exp(G[i * K + c]) * S[c * V + vv];
                for (int m = 0; m <= i; ++m) acc += Mq[i * CS + m] * D[m * V + vv];
                C->o[((start + c0 + i) * H + h) * V + vv] = P->scale * acc;
            }
        /* S' = diag(exp(G_last)) S + (k exp(G_last - G))^T D */
        const double *Gl = G + (L - 1) * K;
        for (int c = 0; c < K; ++c)
            for (int vv = 0; vv < V; ++vv) {
                double acc = exp(Gl[c]) * S[c * V + vv];
                for (int i = 0; i < L; ++i) acc += kh[i * K + c] * exp(Gl[c] - G[i * K + c]) * D[i * V + vv];
                Sn[c * V + vv] = acc;
            }
        memcpy(S, Sn, sizeof(double) * KV);
    }
    if (C->final_state) memcpy(C->final_state + ((size_t)n * H + h) * KV, S, sizeof(double) * KV);
    free(S); free(qh); free(kh); free(G); free(gt); free(bt); free(A); free(Mq); free(Tm);
    free(u); free(w); free(D); free(X); free(Sn);
}

int or_chunk_fwd_chunked(const or_problem *P, int chunk, double *o, double *final_state, int threads) {
    if (chunk < 1) return 1;
    or_chk_ctx C = {P, chunk, o, final_state};
    int N = P->cu_seqlens ? P->N : P->B;
    or_parallel(N * P->H, threads, or_chunked_unit, &C);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Backward: reverse-mode through the token recurrence (BPTT).         */
/* The pages give no backward; this is the adjoint of or_step, derived */
/* by hand and pinned by central finite differences in the tests.      */
/* Per token, walking t from last to first with the running dS:        */
/*   dS += s q dO^T;  dq = s S_t dO                                     */
/*   dk  = dS d;      dd = dS^T k                                       */
/*   dv  = beta dd;   dbeta = dd . (v - p);   dp = -beta dd            */
/*   dS~ = dS + k dp^T;  dk += S~ dp;  dg_c = sum_v dS~[c,v] S~[c,v]    */
/*   dS  = diag(exp(g)) dS~                                             */
/* then the prologue chain rule (normalisation, sigmoid, gate).        */
/* States are re-derived from checkpoints kept every 64 tokens.        */
/* ------------------------------------------------------------------ */
typedef struct {
    const or_problem *P;
    const double *dO;       /* [rows, H, V] */
    const double *dS_final; /* [N, H, K, V] or NULL */
    double *dq, *dk, *dv, *dg, *dbeta; /* gradients w.r.t. the tensors as passed */
    double *dh0;            /* [N, H, K, V] or NULL */
    double *dA_part;        /* [N*H] per-unit partial of dA_log */
    double *ddt_part;       /* [N*H, K] per-unit partial of ddt_bias */
} or_bwd_ctx;

#define OR_CKPT 64

static void or_bwd_unit(void *vctx, int unit) {
    or_bwd_ctx *C = (or_bwd_ctx *)vctx;
    const or_problem *P = C->P;
    int H = P->H, K = P->K, V = P->V;
    int n = unit / H, h = unit % H;
    int64_t start, len;
    or_seq_bounds(P, n, &start, &len);
    size_t KV = (size_t)K * V;
    double *S = (double *)calloc(KV, sizeof(double));
    if (P->initial_state) memcpy(S, P->initial_state + ((size_t)n * H + h) * KV, sizeof(double) * KV);
    int64_t nck = (len + OR_CKPT - 1) / OR_CKPT;
    /* ckpt[b] = state entering token b*OR_CKPT */
    double *ckpt = (double *)malloc(sizeof(double) * KV * (nck > 0 ? nck : 1));
    double *qh = (double *)malloc(sizeof(double) * K), *kh = (double *)malloc(sizeof(double) * K);
    double *gt = (double *)malloc(sizeof(double) * K);
    double *p = (double *)malloc(sizeof(double) * V), *d = (double *)malloc(sizeof(double) * V);
    for (int64_t t = 0; t < len; ++t) {
        if (t % OR_CKPT == 0) memcpy(ckpt + (t / OR_CKPT) * KV, S, sizeof(double) * KV);
        double b;
        or_prologue(P, start + t, h, qh, kh, &b, gt);
        or_step(K, V, S, qh, kh, P->v + ((start + t) * H + h) * V, b, gt, P->scale, p, d, NULL);
    }
    double *dS = (double *)calloc(KV, sizeof(double));
    if (C->dS_final) memcpy(dS, C->dS_final + ((size_t)n * H + h) * KV, sizeof(double) * KV);

    /* per-token saved states inside one checkpoint block: entry (S_prev) of each token */
    double *blk = (double *)malloc(sizeof(double) * KV * OR_CKPT);
    double *St = (double *)malloc(sizeof(double) * KV);
    double *Sd = (double *)malloc(sizeof(double) * KV);
    double *dqh = (double *)malloc(sizeof(double) * K), *dkh = (double *)malloc(sizeof(double) * K);
    double *dgt = (double *)malloc(sizeof(double) * K), *dd = (double *)malloc(sizeof(double) * V);
    double dA_acc = 0.0;
    double *ddt_acc = C->ddt_part + (size_t)unit * K;
    for (int c = 0; c < K; ++c) ddt_acc[c] = 0.0;

    for (int64_t bi = nck - 1; bi >= 0; --bi) {
        int64_t t0 = bi * OR_CKPT;
        int64_t t1 = (t0 + OR_CKPT < len) ? t0 + OR_CKPT : len;
        memcpy(St, ckpt + bi * KV, sizeof(double) * KV);
        for (int64_t t = t0; t < t1; ++t) {
            memcpy(blk + (t - t0) * KV, St, sizeof(double) * KV);
            double b;
            or_prologue(P, start + t, h, qh, kh, &b, gt);
            or_step(K, V, St, qh, kh, P->v + ((start + t) * H + h) * V, b, gt, P->scale, p, d, NULL);
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
            int64_t row = start + t;
            const double *vt = P->v + (row * H + h) * V;
            const double *dOt = C->dO + (row * H + h) * V;
            double b;
            or_prologue(P, row, h, qh, kh, &b, gt);
            /* S~ = diag(exp(g)) S_prev; p, d; S_t = S~ + k d^T */
            const double *Sp = blk + (t - t0) * KV;
            for (int kk = 0; kk < K; ++kk) {
                double e = exp(gt[kk]);
                for (int vv = 0; vv < V; ++vv) Sd[kk * V + vv] = e * Sp[kk * V + vv];
            }
            for (int vv = 0; vv < V; ++vv) {
                double acc = 0.0;
                for (int kk = 0; kk < K; ++kk) acc += Sd[kk * V + vv] * kh[kk];
                p[vv] = acc;
                d[vv] = b * (vt[vv] - acc);
            }
            for (int kk = 0; kk < K; ++kk)
                for (int vv = 0; vv < V; ++vv) St[kk * V + vv] = Sd[kk * V + vv] + kh[kk] * d[vv];
            /* o = s S_t^T q */
            for (int kk = 0; kk < K; ++kk) {
                double acc = 0.0;
                for (int vv = 0; vv < V; ++vv) {
                    dS[kk * V + vv] += P->scale * qh[kk] * dOt[vv];
                    acc += St[kk * V + vv] * dOt[vv];
                }
                dqh[kk] = P->scale * acc;
            }
            /* S_t = S~ + k d^T */
            for (int kk = 0; kk < K; ++kk) {
                double acc = 0.0;
                for (int vv = 0; vv < V; ++vv) acc += dS[kk * V + vv] * d[vv];
                dkh[kk] = acc;
            }
            for (int vv = 0; vv < V; ++vv) {
                double acc = 0.0;
                for (int kk = 0; kk < K; ++kk) acc += dS[kk * V + vv] * kh[kk];
                dd[vv] = acc;
            }
            /* d = beta (v - p) */
            double dbeta = 0.0;
            for (int vv = 0; vv < V; ++vv) {
                C->dv[(row * H + h) * V + vv] = b * dd[vv];
                dbeta += dd[vv] * (vt[vv] - p[vv]);
                dd[vv] = -b * dd[vv]; /* now dp */
            }
            /* p = S~^T k: dS~ = dS + k dp^T, dk += S~ dp */
            for (int kk = 0; kk < K; ++kk) {
                double acc = 0.0;
                for (int vv = 0; vv < V; ++vv) {
                    acc += Sd[kk * V + vv] * dd[vv];
                    dS[kk * V + vv] += kh[kk] * dd[vv];
                }
                dkh[kk] += acc;
            }
            /* S~ = diag(exp(g)) S_prev */
            for (int kk = 0; kk < K; ++kk) {
                double acc = 0.0, e = exp(gt[kk]);
                for (int vv = 0; vv < V; ++vv) {
                    acc += dS[kk * V + vv] * Sd[kk * V + vv];
                    dS[kk * V + vv] *= e;
                }
                dgt[kk] = acc;
            }
            /* prologue chain rule */
            const double *qr = P->q + (row * H + h) * K;
            const double *kr = P->k + (row * H + h) * K;
            double *dq_out = C->dq + (row * H + h) * K;
            double *dk_out = C->dk + (row * H + h) * K;
            if (P->use_qk_l2norm) {
                /* x^ = x r, r = (sum x^2 + eps)^{-1/2}: dx = r (dx^ - x^ (x^ . dx^)) */
                double ssq = 0.0, ssk = 0.0, dotq = 0.0, dotk = 0.0;
                for (int c = 0; c < K; ++c) { ssq += qr[c] * qr[c]; ssk += kr[c] * kr[c]; }
                double rq = 1.0 / sqrt(ssq + P->l2_eps), rk = 1.0 / sqrt(ssk + P->l2_eps);
                for (int c = 0; c < K; ++c) { dotq += qh[c] * dqh[c]; dotk += kh[c] * dkh[c]; }
                for (int c = 0; c < K; ++c) {
                    dq_out[c] = rq * (dqh[c] - qh[c] * dotq);
                    dk_out[c] = rk * (dkh[c] - kh[c] * dotk);
                }
            } else {
                memcpy(dq_out, dqh, sizeof(double) * K);
                memcpy(dk_out, dkh, sizeof(double) * K);
            }
            C->dbeta[row * H + h] = P->use_beta_sigmoid ? dbeta * b * (1.0 - b) : dbeta;
            double *dg_out = C->dg + (row * H + h) * K;
            const double *xr = P->g + (row * H + h) * K;
            if (P->gate_mode == OR_GATE_LOGDECAY) {
                memcpy(dg_out, dgt, sizeof(double) * K);
            } else {
                double rate = exp(P->A_log[h]);
                for (int c = 0; c < K; ++c) {
                    double z = xr[c] + (P->dt_bias ? P->dt_bias[h * K + c] : 0.0);
                    double dx, dA;
                    if (P->gate_mode == OR_GATE_SAFE) {
                        /* g = lb sig(rate z): dg/dx = lb sig (1-sig) rate, dg/dA_log = lb sig (1-sig) rate z */
                        double sg = or_sigmoid(rate * z);
                        double base = P->lower_bound * sg * (1.0 - sg);
                        dx = base * rate;
                        dA = base * rate * z;
                    } else {
                        /* g = -rate softplus(z): dg/dx = -rate sig(z), dg/dA_log = g */
                        dx = -rate * or_sigmoid(z);
                        dA = -rate * or_softplus(z);
                    }
                    dg_out[c] = dgt[c] * dx;
                    ddt_acc[c] += dgt[c] * dx;
                    dA_acc += dgt[c] * dA;
                }
            }
        }
    }
    C->dA_part[unit] = dA_acc;
    if (C->dh0) memcpy(C->dh0 + ((size_t)n * H + h) * KV, dS, sizeof(double) * KV);
    free(S); free(ckpt); free(qh); free(kh); free(gt); free(p); free(d); free(dS); free(blk);
    free(St); free(Sd); free(dqh); free(dkh); free(dgt); free(dd);
}

/* Gradients of L = <o, dO> + <final_state, dS_final> with respect to every
 * input as passed: q, k, v, the raw gate input g (log-decay in LOGDECAY mode),
 * beta (logit when the sigmoid flag is set), initial_state, A_log and dt_bias
 * (the last two only in the SAFE / SOFTPLUS modes; sums over every token and,
 * for A_log, over the key channels too).  Unit partials are reduced serially
 * so the result does not depend on the thread count. */
int or_chunk_bwd(const or_problem *P, const double *dO, const double *dS_final, double *dq,
                 double *dk, double *dv, double *dg, double *dbeta, double *dh0, double *dA_log,
                 double *ddt_bias, int threads) {
    int N = P->cu_seqlens ? P->N : P->B;
    int U = N * P->H;
    or_bwd_ctx C;
    C.P = P; C.dO = dO; C.dS_final = dS_final;
    C.dq = dq; C.dk = dk; C.dv = dv; C.dg = dg; C.dbeta = dbeta; C.dh0 = dh0;
    C.dA_part = (double *)calloc(U > 0 ? U : 1, sizeof(double));
    C.ddt_part = (double *)calloc((size_t)(U > 0 ? U : 1) * P->K, sizeof(double));
    or_parallel(U, threads, or_bwd_unit, &C);
    if (dA_log)
        for (int h = 0; h < P->H; ++h) {
            double acc = 0.0;
            for (int n = 0; n < N; ++n) acc += C.dA_part[n * P->H + h];
            dA_log[h] = acc;
        }
    if (ddt_bias)
        for (int h = 0; h < P->H; ++h)
            for (int c = 0; c < P->K; ++c) {
                double acc = 0.0;
                for (int n = 0; n < N; ++n) acc += C.ddt_part[((size_t)n * P->H + h) * P->K + c];
                ddt_bias[h * P->K + c] = acc;
            }
    free(C.dA_part);
    free(C.ddt_part);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Decode: one token per sequence with the short-conv update.          */
/* [kda.rs] kda_decode_token = conv_update over the 3*H*D [q|k|v]       */
/* channels, then kda_recurrent_step on the conv output.                */
/* conv_update: shift the window left by one (slot 0 leaves), write x  */
/* into the last slot, y = SiLU(sum_j w[c,j] * window[c,j]).            */
/* ------------------------------------------------------------------ */
/* SiLU(x) = x sigma(x). */
static double or_silu(double x) { return x * or_sigmoid(x); }

/* The causal depthwise convolution at the newest token x of one channel:
 * sum_j w[j] u[j] over the W most recent inputs u, oldest first (u = the
 * W - 1 newest entries of the window `win`, then x): [kda.rs] conv_update's
 * output, no bias. */
static double or_conv_tap(int W, const double *w, const double *win, double x) {
    return la_dot(W - 1, w, win + 1) + w[W - 1] * x;
}

/* The window after x enters: the oldest entry leaves, x becomes the newest. */
static void or_window_push(int W, double *win, double x) {
    memmove(win, win + 1, sizeof(double) * (W - 1));
    win[W - 1] = x;
}

typedef struct {
    int N, H, D, W;
    const double *x;       /* [N, 3*H*D] */
    const double *conv_w;  /* [3*H*D, W] */
    double *conv_state;    /* [N, 3*H*D, W] in/out */
    const double *g;       /* [N, H*D] raw gate input */
    const double *beta;    /* [N, H] */
    const double *A_log, *dt_bias;
    double lower_bound;
    int gate_mode, use_qk_l2norm, use_beta_sigmoid;
    double scale, l2_eps;
    double *state;         /* [N, H, D, D] in/out */
    double *o;             /* [N, H*D] */
} or_decode;

static void or_decode_seq(void *vctx, int n) {
    or_decode *Dp = (or_decode *)vctx;
    int H = Dp->H, D = Dp->D, W = Dp->W, CH = 3 * H * D;
    double *y = (double *)malloc(sizeof(double) * CH);
    const double *xn = Dp->x + (size_t)n * CH;
    double *cs = Dp->conv_state + (size_t)n * CH * W;
    for (int c = 0; c < CH; ++c) {
        double *win = cs + (size_t)c * W;  /* the last W inputs, oldest first */
        y[c] = or_silu(or_conv_tap(W, Dp->conv_w + (size_t)c * W, win, xn[c]));
        or_window_push(W, win, xn[c]);
    }
    /* the recurrent step on the post-conv [q|k|v] */
    or_problem P;
    memset(&P, 0, sizeof(P));
    P.B = 1; P.T = 1; P.H = H; P.K = D; P.V = D;
    P.q = y; P.k = y + H * D; P.v = y + 2 * H * D;
    P.g = Dp->g + (size_t)n * H * D;
    P.beta = Dp->beta + (size_t)n * H;
    P.A_log = Dp->A_log; P.dt_bias = Dp->dt_bias;
    P.scale = Dp->scale; P.lower_bound = Dp->lower_bound; P.gate_mode = Dp->gate_mode;
    P.use_qk_l2norm = Dp->use_qk_l2norm; P.use_beta_sigmoid = Dp->use_beta_sigmoid;
    P.l2_eps = Dp->l2_eps;
    double *qh = (double *)malloc(sizeof(double) * D), *kh = (double *)malloc(sizeof(double) * D);
    double *gt = (double *)malloc(sizeof(double) * D);
    double *p = (double *)malloc(sizeof(double) * D), *d = (double *)malloc(sizeof(double) * D);
    for (int h = 0; h < H; ++h) {
        double b;
        or_prologue(&P, 0, h, qh, kh, &b, gt);
        double *S = Dp->state + ((size_t)n * H + h) * D * D;
        or_step(D, D, S, qh, kh, P.v + h * D, b, gt, Dp->scale, p, d, Dp->o + (size_t)n * H * D + h * D);
    }
    free(y); free(qh); free(kh); free(gt); free(p); free(d);
}

int or_decode_step(or_decode *Dp, int threads) {
    or_parallel(Dp->N, threads, or_decode_seq, Dp);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Stateful conv prefill: [kda.rs] conv_update applied to each row of a */
/* sequence in order, starting from the sequence's conv state (zeros    */
/* when conv_state is NULL) and leaving the window after its last row   */
/* in it, so that a stateful prime continues exactly in the decode step */
/* ("memra-engine kda_fixture_gpu.rs" page, GATE 2 and GATE 3).         */
/* x, y [rows, C]; conv_w [C, W]; conv_state [N, C, W] in/out or NULL.  */
/* cu NULL: N = B sequences of T rows each.                              */
/* ------------------------------------------------------------------ */
int or_conv_prefill(int B, int T, int C, int W, const int32_t *cu, int N, const double *x,
                    const double *conv_w, double *conv_state, double *y) {
    /* Per sequence and channel, the inputs extended on the left by the W
     * entries of the incoming window: u = [window ; x_0 .. x_{L-1}], so that
     * y_t = SiLU(sum_j w[j] u[t + 1 + j]) and the outgoing window is the last
     * W entries of u. */
    int nseq = cu ? N : B;
    for (int n = 0; n < nseq; ++n) {
        long start = cu ? cu[n] : (long)n * T;
        long len = cu ? (long)cu[n + 1] - cu[n] : T;
        double *u = (double *)malloc(sizeof(double) * (size_t)(W + len));
        for (int c = 0; c < C; ++c) {
            double *st = conv_state ? conv_state + ((size_t)n * C + c) * W : NULL;
            for (int j = 0; j < W; ++j) u[j] = st ? st[j] : 0.0;
            for (long t = 0; t < len; ++t) u[W + t] = x[(size_t)(start + t) * C + c];
            for (long t = 0; t < len; ++t)
                y[(size_t)(start + t) * C + c] = or_silu(la_dot(W, conv_w + (size_t)c * W, u + t + 1));
            if (st) memcpy(st, u + len, sizeof(double) * W);
        }
        free(u);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Full-rank output gate: [kda.rs] full_rank_output_gate.  For each of  */
/* the n_vec = rows*H vectors of length V (one head of one row):        */
/*     ms = (1/V) sum_v o[v]^2,   r = 1 / sqrt(ms + eps),               */
/*     y[v] = sigmoid(g[v]) * o[v] * r.                                 */
/* eps is that of the gated output norm ("memra-engine                  */
/* kda_fixture_gpu.rs" page: 1e-5), supplied by the caller.             */
/* ------------------------------------------------------------------ */
int or_output_gate(int64_t n_vec, int V, const double *o, const double *g, double eps, double *y) {
    for (int64_t i = 0; i < n_vec; ++i) {
        const double *oi = o + i * V, *gi = g + i * V;
        double *yi = y + i * V;
        /* RMS normalisation of the head's vector, then the elementwise gate */
        la_scale(V, 1.0 / sqrt(la_dot(V, oi, oi) / V + eps), oi, yi);
        for (int v = 0; v < V; ++v) yi[v] *= or_sigmoid(gi[v]);
    }
    return 0;
}

/* Reverse mode of or_output_gate (chain rule written out; no page prints */
/* it).  With a = sigmoid(g), r as above and the upstream dy:            */
/*     dg[v] = dy[v] * o[v] * r * a[v] (1 - a[v])                         */
/*     do[v] = r a[v] dy[v]  +  o[v] * dr/dms * (2/V) * sum_u a[u] dy[u] o[u] */
/* where dr/dms = -r^3 / 2, so the second term is                         */
/*     -(r^3 / V) * o[v] * sum_u a[u] dy[u] o[u].                          */
int or_output_gate_bwd(int64_t n_vec, int V, const double *o, const double *g, double eps,
                       const double *dy, double *dO, double *dg) {
    for (int64_t i = 0; i < n_vec; ++i) {
        const double *oi = o + i * V, *gi = g + i * V, *di = dy + i * V;
        double ss = 0.0, sa = 0.0;
        for (int v = 0; v < V; ++v) {
            ss += oi[v] * oi[v];
            sa += or_sigmoid(gi[v]) * di[v] * oi[v];
        }
        const double r = 1.0 / sqrt(ss / V + eps);
        const double dr_dms = -0.5 * r * r * r;
        for (int v = 0; v < V; ++v) {
            const double a = or_sigmoid(gi[v]);
            dg[i * V + v] = di[v] * oi[v] * r * a * (1.0 - a);
            dO[i * V + v] = r * a * di[v] + oi[v] * dr_dms * (2.0 / V) * sa;
        }
    }
    return 0;
}

/* Exposed scalar pieces, for the closed-form pins. */
void or_gate_values(int gate_mode, int H, int K, const double *x, const double *A_log,
                    const double *dt_bias, double lower_bound, double *g_out) {
    or_problem P;
    memset(&P, 0, sizeof(P));
    P.H = H; P.K = K; P.gate_mode = gate_mode; P.A_log = A_log; P.dt_bias = dt_bias;
    P.lower_bound = lower_bound;
    for (int h = 0; h < H; ++h) or_gate(&P, h, x + h * K, g_out + h * K);
}

void or_l2norm_rows(const double *x, int rows, int d, double eps, double *out) {
    for (int r = 0; r < rows; ++r) or_l2norm(x + (size_t)r * d, d, eps, out + (size_t)r * d);
}
