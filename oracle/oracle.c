/*
 * oracle.c -- plain, slow, fp64 CPU reference for linear attention with the
 * elu(x)+1 feature map.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the HIP library under linear_attention_02_amd/.
 *
 * Every function follows a definition printed on the pages:
 *   [WRA]  "Why Replace Attention? The Softmax Bottleneck and the Path to
 *           Linear Time" (prathamp.com/blog/attention-why-replace)
 *   [KN]   "Transformers Are RNNs: Linear Attention" knowledge note
 *           (zhongzhoutan-coder.github.io/algorithms/attention/linear/)
 *   [PR]   "[Paper Review] Transformers are RNNs ..." (velog.io/@jmsong62)
 *
 * Conventions (readings of the pages where they leave a point open):
 *   - phi(x) = elu(x) + 1 with alpha = 1: x + 1 for x > 0, exp(x) otherwise
 *     ([WRA] §5.3, boxed formula and the elu definition under it).
 *   - causal sums are inclusive, j <= i ([WRA] §7.1).
 *   - the recurrence updates S and z first, then reads them ([WRA] §7.2,
 *     steps 2-4; [KN] "Turn Causal Attention into a Recurrence").
 *   - no epsilon in the denominator; a non-positive denominator is reported
 *     through the return code instead (positivity: [WRA] §5.4, [PR] §3.3).
 *
 * Layouts: Q, K are [units][N][C], V is [units][N][M] (units = B*H), all
 * contiguous row-major; outputs are double [units][N][M].  Input element
 * types: ORACLE_F64, ORACLE_F32, ORACLE_BF16 (raw 16-bit patterns).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F64 = 0, ORACLE_F32 = 1, ORACLE_BF16 = 2 };

/* Return codes. */
enum { ORACLE_OK = 0, ORACLE_NONPOSITIVE_DEN = 1, ORACLE_BAD_ARG = 2, ORACLE_NO_MEMORY = 3 };

/* bfloat16 is the upper half of an IEEE binary32 pattern; widening it is the
 * bit shift below followed by an exact float -> double conversion. */
double oracle_bf16_to_double(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double elem(const void *p, int dtype, size_t i) {
    switch (dtype) {
    case ORACLE_F64: return ((const double *)p)[i];
    case ORACLE_F32: return (double)((const float *)p)[i];
    default: return oracle_bf16_to_double(((const uint16_t *)p)[i]);
    }
}

/* [WRA] §5.3: phi(x) = elu(x) + 1, elu(x) = x for x > 0 and e^x - 1 for x <= 0.
 * For x <= 0, (e^x - 1) + 1 is written as e^x, the same number without the
 * cancellation. */
double oracle_phi(double x) { return x > 0.0 ? x + 1.0 : exp(x); }

/* ---------------------------------------------------------------------------
 * A minimal parallel-for over the B*H independent (batch, head) units.
 * ------------------------------------------------------------------------- */
typedef void (*unit_fn)(void *ctx, long unit);

typedef struct {
    unit_fn fn;
    void *ctx;
    long units;
    long first;
    long stride;
} worker_arg;

static void *worker_main(void *p) {
    worker_arg *a = (worker_arg *)p;
    for (long u = a->first; u < a->units; u += a->stride) a->fn(a->ctx, u);
    return NULL;
}

static void parallel_units(unit_fn fn, void *ctx, long units, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > units) nthreads = (int)(units > 0 ? units : 1);
    if (nthreads == 1) {
        for (long u = 0; u < units; ++u) fn(ctx, u);
        return;
    }
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    worker_arg *args = (worker_arg *)malloc(sizeof(worker_arg) * (size_t)nthreads);
    int started = 0;
    for (int t = 0; th && args && t < nthreads; ++t) {
        args[t].fn = fn;
        args[t].ctx = ctx;
        args[t].units = units;
        args[t].first = t;
        args[t].stride = nthreads;
        if (pthread_create(&th[t], NULL, worker_main, &args[t]) != 0) break;
        ++started;
    }
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    /* Units of threads that could not be started run here. */
    if (started < nthreads) {
        for (int t = started; t < nthreads; ++t)
            for (long u = t; u < units; u += nthreads) fn(ctx, u);
    }
    free(th);
    free(args);
}

/* ---------------------------------------------------------------------------
 * Shared argument block for the forward forms.
 * ------------------------------------------------------------------------- */
typedef struct {
    const void *Q, *K, *V;
    int dtype;
    long N, C, M;
    int causal;
    int absv;             /* use |v| instead of v: the magnitude companion */
    double *O;
    const double *S0;     /* optional initial state [units][C][M] */
    const double *z0;     /* optional initial normaliser [units][C] */
    double *S_out;        /* optional final state */
    double *z_out;
    volatile int bad;     /* set when some denominator is <= 0 */
} fwd_ctx;

static double vval(const fwd_ctx *x, size_t idx) {
    double v = elem(x->V, x->dtype, idx);
    return x->absv ? fabs(v) : v;
}

/* O1 -- the definition ([WRA] §5.7 and §7.1):
 *   w_ij = phi(q_i)^T phi(k_j) for j in J(i),
 *   o_i  = sum_j w_ij v_j / sum_j w_ij,
 * with J(i) = {0..i} when causal and {0..N-1} otherwise.  O(N^2 (C+M)). */
static void quadratic_unit(void *vctx, long u) {
    fwd_ctx *x = (fwd_ctx *)vctx;
    const long N = x->N, C = x->C, M = x->M;
    const size_t qk0 = (size_t)u * (size_t)N * (size_t)C;
    const size_t v0 = (size_t)u * (size_t)N * (size_t)M;
    double *num = (double *)malloc(sizeof(double) * (size_t)M);
    if (!num) { x->bad = 1; return; }
    for (long i = 0; i < N; ++i) {
        const long jmax = x->causal ? i : N - 1;
        double den = 0.0;
        for (long m = 0; m < M; ++m) num[m] = 0.0;
        for (long j = 0; j <= jmax; ++j) {
            double w = 0.0;
            for (long c = 0; c < C; ++c)
                w += oracle_phi(elem(x->Q, x->dtype, qk0 + (size_t)i * C + c)) *
                     oracle_phi(elem(x->K, x->dtype, qk0 + (size_t)j * C + c));
            den += w;
            for (long m = 0; m < M; ++m) num[m] += w * vval(x, v0 + (size_t)j * M + m);
        }
        if (!(den > 0.0)) x->bad = 1;
        for (long m = 0; m < M; ++m) x->O[v0 + (size_t)i * M + m] = num[m] / den;
    }
    free(num);
}

/* O2 -- the causal recurrence ([WRA] §7.2; [KN] "Turn Causal Attention into a
 * Recurrence"): S_0 = 0, z_0 = 0 (or a given initial state), and per token i
 *   S_i = S_{i-1} + phi(k_i) v_i^T,  z_i = z_{i-1} + phi(k_i),
 *   o_i = phi(q_i)^T S_i / phi(q_i)^T z_i.
 * The non-causal linear form ([WRA] §6.2) is run by the same function with
 * causal = 0: S and z are summed over every token first, then read. */
static void recurrent_unit(void *vctx, long u) {
    fwd_ctx *x = (fwd_ctx *)vctx;
    const long N = x->N, C = x->C, M = x->M;
    const size_t qk0 = (size_t)u * (size_t)N * (size_t)C;
    const size_t v0 = (size_t)u * (size_t)N * (size_t)M;
    double *S = (double *)calloc((size_t)(C * M), sizeof(double));
    double *z = (double *)calloc((size_t)C, sizeof(double));
    double *pk = (double *)malloc(sizeof(double) * (size_t)C);
    double *pq = (double *)malloc(sizeof(double) * (size_t)C);
    if (!S || !z || !pk || !pq) { x->bad = 1; free(S); free(z); free(pk); free(pq); return; }
    if (x->S0) memcpy(S, x->S0 + (size_t)u * C * M, sizeof(double) * (size_t)(C * M));
    if (x->z0) memcpy(z, x->z0 + (size_t)u * C, sizeof(double) * (size_t)C);

    if (!x->causal) {
        /* S = sum_j phi(k_j) v_j^T, z = sum_j phi(k_j) ([WRA] §6.2). */
        for (long j = 0; j < N; ++j) {
            for (long c = 0; c < C; ++c) pk[c] = oracle_phi(elem(x->K, x->dtype, qk0 + (size_t)j * C + c));
            for (long c = 0; c < C; ++c) {
                z[c] += pk[c];
                for (long m = 0; m < M; ++m) S[c * M + m] += pk[c] * vval(x, v0 + (size_t)j * M + m);
            }
        }
    }
    for (long i = 0; i < N; ++i) {
        if (x->causal) {
            for (long c = 0; c < C; ++c) pk[c] = oracle_phi(elem(x->K, x->dtype, qk0 + (size_t)i * C + c));
            for (long c = 0; c < C; ++c) {
                z[c] += pk[c];
                for (long m = 0; m < M; ++m) S[c * M + m] += pk[c] * vval(x, v0 + (size_t)i * M + m);
            }
        }
        for (long c = 0; c < C; ++c) pq[c] = oracle_phi(elem(x->Q, x->dtype, qk0 + (size_t)i * C + c));
        double den = 0.0;
        for (long c = 0; c < C; ++c) den += pq[c] * z[c];
        if (!(den > 0.0)) x->bad = 1;
        for (long m = 0; m < M; ++m) {
            double num = 0.0;
            for (long c = 0; c < C; ++c) num += pq[c] * S[c * M + m];
            x->O[v0 + (size_t)i * M + m] = num / den;
        }
    }
    if (x->S_out) memcpy(x->S_out + (size_t)u * C * M, S, sizeof(double) * (size_t)(C * M));
    if (x->z_out) memcpy(x->z_out + (size_t)u * C, z, sizeof(double) * (size_t)C);
    free(S); free(z); free(pk); free(pq);
}

static int check_dims(const void *Q, const void *K, const void *V, const double *O, int dtype,
                      long units, long N, long C, long M) {
    if (units < 0 || N < 0 || C < 1 || M < 1) return 0;
    if (dtype != ORACLE_F64 && dtype != ORACLE_F32 && dtype != ORACLE_BF16) return 0;
    if (units > 0 && N > 0 && (!Q || !K || !V || !O)) return 0;
    return 1;
}

/* O1: quadratic definition.  causal selects J(i). */
int oracle_forward_quadratic(const void *Q, const void *K, const void *V, int dtype, long units,
                             long N, long C, long M, int causal, int absv, double *O, int nthreads) {
    if (!check_dims(Q, K, V, O, dtype, units, N, C, M)) return ORACLE_BAD_ARG;
    fwd_ctx x = {Q, K, V, dtype, N, C, M, causal != 0, absv != 0, O, NULL, NULL, NULL, NULL, 0};
    parallel_units(quadratic_unit, &x, units, nthreads);
    return x.bad ? ORACLE_NONPOSITIVE_DEN : ORACLE_OK;
}

/* O2 (causal = 1) and O3 (causal = 0).  S0/z0 (may be NULL) seed the state;
 * S_out/z_out (may be NULL) receive the state after the last token. */
int oracle_forward_recurrent(const void *Q, const void *K, const void *V, int dtype, long units,
                             long N, long C, long M, int causal, int absv, const double *S0,
                             const double *z0, double *O, double *S_out, double *z_out,
                             int nthreads) {
    if (!check_dims(Q, K, V, O, dtype, units, N, C, M)) return ORACLE_BAD_ARG;
    fwd_ctx x = {Q, K, V, dtype, N, C, M, causal != 0, absv != 0, O, S0, z0, S_out, z_out, 0};
    parallel_units(recurrent_unit, &x, units, nthreads);
    return x.bad ? ORACLE_NONPOSITIVE_DEN : ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * O4 -- one decode step on an fp64 state, in place ([WRA] §7.2, steps 1-4):
 * for each of the units independent heads,
 *   S += phi(k) v^T; z += phi(k); o = phi(q)^T S / phi(q)^T z.
 * q, k are [units][C]; v is [units][M]; S is [units][C][M]; z is [units][C];
 * o is double [units][M].
 * ------------------------------------------------------------------------- */
typedef struct {
    double *S, *z;
    const void *q, *k, *v;
    int dtype;
    long C, M;
    int absv;
    double *o;
    volatile int bad;
} dec_ctx;

static void decode_unit(void *vctx, long u) {
    dec_ctx *x = (dec_ctx *)vctx;
    const long C = x->C, M = x->M;
    double *S = x->S + (size_t)u * C * M;
    double *z = x->z + (size_t)u * C;
    for (long c = 0; c < C; ++c) {
        const double pk = oracle_phi(elem(x->k, x->dtype, (size_t)u * C + c));
        z[c] += pk;
        for (long m = 0; m < M; ++m) {
            double v = elem(x->v, x->dtype, (size_t)u * M + m);
            if (x->absv) v = fabs(v);
            S[c * M + m] += pk * v;
        }
    }
    double den = 0.0;
    for (long c = 0; c < C; ++c) den += oracle_phi(elem(x->q, x->dtype, (size_t)u * C + c)) * z[c];
    if (!(den > 0.0)) x->bad = 1;
    for (long m = 0; m < M; ++m) {
        double num = 0.0;
        for (long c = 0; c < C; ++c)
            num += oracle_phi(elem(x->q, x->dtype, (size_t)u * C + c)) * S[c * M + m];
        x->o[(size_t)u * M + m] = num / den;
    }
}

int oracle_decode_step(double *S, double *z, const void *q, const void *k, const void *v, int dtype,
                       long units, long C, long M, int absv, double *o, int nthreads) {
    if (units < 0 || C < 1 || M < 1) return ORACLE_BAD_ARG;
    if (dtype != ORACLE_F64 && dtype != ORACLE_F32 && dtype != ORACLE_BF16) return ORACLE_BAD_ARG;
    if (units > 0 && (!S || !z || !q || !k || !v || !o)) return ORACLE_BAD_ARG;
    dec_ctx x = {S, z, q, k, v, dtype, C, M, absv != 0, o, 0};
    parallel_units(decode_unit, &x, units, nthreads);
    return x.bad ? ORACLE_NONPOSITIVE_DEN : ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Gradients.  The pages state that the causal gradients can themselves be
 * written as cumulative sums, so training stays linear in time and memory
 * ([PR] §3.5 "Gradient Computation"; [KN] "Turn Causal Attention into a
 * Recurrence"), but print no formula.  What follows is the chain rule applied
 * to the definition O1.  For a loss L with G = dL/dO (rows g_i), per token i
 * with J(i) as in O1:
 *   den_i = sum_{j in J(i)} w_ij,   o_i = sum_{j in J(i)} w_ij v_j / den_i,
 *   a_i   = g_i / den_i               (dL/dnum_i, an M-vector),
 *   b_i   = -(g_i . o_i) / den_i      (dL/dden_i),
 *   dL/dw_ij = a_i . v_j + b_i,
 * and since w_ij = phi(q_i) . phi(k_j):
 *   dphi(q_i) = sum_{j in J(i)}        (a_i . v_j + b_i) phi(k_j)
 *   dphi(k_j) = sum_{i : j in J(i)}    (a_i . v_j + b_i) phi(q_i)
 *   dv_j      = sum_{i : j in J(i)}    w_ij a_i
 *   dq = dphi(q) * phi'(q),  dk = dphi(k) * phi'(k),
 *   phi'(x) = 1 for x > 0, e^x otherwise (the derivative of elu(x) + 1; both
 *   sides give 1 at x = 0).
 * These are checked against finite differences, exact rational dual numbers
 * and an independent autograd run, not against themselves.
 *
 * Magnitude companion (mode 1): every signed term is replaced by an upper
 * bound of its absolute value -- a_i by |g_i| / den_i, b_i by
 * sum_m |g_im| obar_im / den_i (obar is O1 on |v|, and |o_im| <= obar_im),
 * a_i . v_j by |a_i| . |v_j| -- giving elementwise bounds of |dq|, |dk|, |dv|
 * on which the GPU's rounding error is measured.
 * ------------------------------------------------------------------------- */
double oracle_phi_prime(double x) { return x > 0.0 ? 1.0 : exp(x); }

typedef struct {
    const void *Q, *K, *V, *G;
    int dtype;
    long N, C, M;
    int causal;
    int mode;             /* 0: gradient, 1: magnitude companion */
    double *dQ, *dK, *dV;
    volatile int bad;
} bwd_ctx;

typedef struct {
    double *pq, *pk;      /* phi(Q), phi(K): [N][C] */
    double *v, *g;        /* V (|V| in mode 1), G (|G| in mode 1): [N][M] */
    double *a;            /* a_i: [N][M] */
    double *b;            /* b_i: [N] */
} bwd_unit_arrays;

static void bwd_free(bwd_unit_arrays *w) {
    free(w->pq); free(w->pk); free(w->v); free(w->g); free(w->a); free(w->b);
}

/* Loads one unit's phi(Q), phi(K), V and G (absolute values of V and G in
 * companion mode).  Returns 0 when memory runs out. */
static int bwd_load(const bwd_ctx *x, long u, bwd_unit_arrays *w) {
    const long N = x->N, C = x->C, M = x->M;
    const size_t qk0 = (size_t)u * (size_t)N * (size_t)C, v0 = (size_t)u * (size_t)N * (size_t)M;
    const size_t nc = (size_t)(N > 0 ? N : 1) * (size_t)C, nm = (size_t)(N > 0 ? N : 1) * (size_t)M;
    w->pq = (double *)malloc(sizeof(double) * nc);
    w->pk = (double *)malloc(sizeof(double) * nc);
    w->v = (double *)malloc(sizeof(double) * nm);
    w->g = (double *)malloc(sizeof(double) * nm);
    w->a = (double *)malloc(sizeof(double) * nm);
    w->b = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    if (!w->pq || !w->pk || !w->v || !w->g || !w->a || !w->b) return 0;
    for (size_t e = 0; e < (size_t)N * (size_t)C; ++e) {
        w->pq[e] = oracle_phi(elem(x->Q, x->dtype, qk0 + e));
        w->pk[e] = oracle_phi(elem(x->K, x->dtype, qk0 + e));
    }
    for (size_t e = 0; e < (size_t)N * (size_t)M; ++e) {
        const double v = elem(x->V, x->dtype, v0 + e), g = elem(x->G, x->dtype, v0 + e);
        w->v[e] = x->mode ? fabs(v) : v;
        w->g[e] = x->mode ? fabs(g) : g;
    }
    return 1;
}

/* dq = dphi(q) * phi'(q) and dk likewise, in place on the unit's outputs. */
static void bwd_chain_phi(const bwd_ctx *x, long u) {
    const size_t qk0 = (size_t)u * (size_t)x->N * (size_t)x->C;
    for (size_t e = 0; e < (size_t)x->N * (size_t)x->C; ++e) {
        x->dQ[qk0 + e] *= oracle_phi_prime(elem(x->Q, x->dtype, qk0 + e));
        x->dK[qk0 + e] *= oracle_phi_prime(elem(x->K, x->dtype, qk0 + e));
    }
}

/* Gradient of O1 by its definition: every (i, j) pair with j in J(i) is
 * visited.  O(N^2 (C + M)). */
static void bwd_quadratic_unit(void *vctx, long u) {
    bwd_ctx *x = (bwd_ctx *)vctx;
    const long N = x->N, C = x->C, M = x->M;
    const size_t qk0 = (size_t)u * (size_t)N * (size_t)C, v0 = (size_t)u * (size_t)N * (size_t)M;
    double *dq = x->dQ + qk0, *dk = x->dK + qk0, *dv = x->dV + v0;
    for (size_t e = 0; e < (size_t)N * (size_t)C; ++e) { dq[e] = 0.0; dk[e] = 0.0; }
    for (size_t e = 0; e < (size_t)N * (size_t)M; ++e) dv[e] = 0.0;
    bwd_unit_arrays w = {0};
    if (!bwd_load(x, u, &w)) { x->bad = 1; bwd_free(&w); return; }
    double *o = (double *)malloc(sizeof(double) * (size_t)M);
    if (!o) { x->bad = 1; bwd_free(&w); return; }
    for (long i = 0; i < N; ++i) {
        const long jmax = x->causal ? i : N - 1;
        /* den_i and o_i (obar_i in companion mode: w.v holds |V| there). */
        double den = 0.0;
        for (long m = 0; m < M; ++m) o[m] = 0.0;
        for (long j = 0; j <= jmax; ++j) {
            double wij = 0.0;
            for (long c = 0; c < C; ++c) wij += w.pq[i * C + c] * w.pk[j * C + c];
            den += wij;
            for (long m = 0; m < M; ++m) o[m] += wij * w.v[j * M + m];
        }
        if (!(den > 0.0)) x->bad = 1;
        double go = 0.0;
        for (long m = 0; m < M; ++m) {
            o[m] /= den;
            go += w.g[i * M + m] * o[m];
            w.a[i * M + m] = w.g[i * M + m] / den;
        }
        w.b[i] = x->mode ? go / den : -go / den;
        for (long j = 0; j <= jmax; ++j) {
            double wij = 0.0, coef = w.b[i];
            for (long c = 0; c < C; ++c) wij += w.pq[i * C + c] * w.pk[j * C + c];
            for (long m = 0; m < M; ++m) coef += w.a[i * M + m] * w.v[j * M + m];
            for (long c = 0; c < C; ++c) {
                dq[i * C + c] += coef * w.pk[j * C + c];
                dk[j * C + c] += coef * w.pq[i * C + c];
            }
            for (long m = 0; m < M; ++m) dv[j * M + m] += wij * w.a[i * M + m];
        }
    }
    free(o);
    bwd_free(&w);
    bwd_chain_phi(x, u);
}

/* The same gradients as cumulative sums, O(N C M):
 *   forward sweep with the prefix state S_i, z_i of O2 (all-token totals when
 *   non-causal):  o_i, a_i, b_i as above and dphi(q_i) = S_i a_i + b_i z_i;
 *   backward sweep with the suffix state R_j = sum_{i : j in J(i)} phi(q_i) a_i^T
 *   (C x M) and r_j = sum_{i : j in J(i)} b_i phi(q_i) (C):
 *   dphi(k_j) = R_j v_j + r_j,  dv_j = R_j^T phi(k_j).
 * Only S, z, R, r and the per-token a, b are held -- no per-token state. */
static void bwd_recurrent_unit(void *vctx, long u) {
    bwd_ctx *x = (bwd_ctx *)vctx;
    const long N = x->N, C = x->C, M = x->M;
    const size_t qk0 = (size_t)u * (size_t)N * (size_t)C, v0 = (size_t)u * (size_t)N * (size_t)M;
    double *dq = x->dQ + qk0, *dk = x->dK + qk0, *dv = x->dV + v0;
    bwd_unit_arrays w = {0};
    double *S = (double *)calloc((size_t)(C * M), sizeof(double));
    double *z = (double *)calloc((size_t)C, sizeof(double));
    if (!S || !z || !bwd_load(x, u, &w)) { x->bad = 1; free(S); free(z); bwd_free(&w); return; }
    if (!x->causal)
        for (long j = 0; j < N; ++j)
            for (long c = 0; c < C; ++c) {
                z[c] += w.pk[j * C + c];
                for (long m = 0; m < M; ++m) S[c * M + m] += w.pk[j * C + c] * w.v[j * M + m];
            }
    for (long i = 0; i < N; ++i) {
        if (x->causal)
            for (long c = 0; c < C; ++c) {
                z[c] += w.pk[i * C + c];
                for (long m = 0; m < M; ++m) S[c * M + m] += w.pk[i * C + c] * w.v[i * M + m];
            }
        double den = 0.0, go = 0.0;
        for (long c = 0; c < C; ++c) den += w.pq[i * C + c] * z[c];
        if (!(den > 0.0)) x->bad = 1;
        for (long m = 0; m < M; ++m) {
            double num = 0.0;
            for (long c = 0; c < C; ++c) num += w.pq[i * C + c] * S[c * M + m];
            go += w.g[i * M + m] * (num / den);
            w.a[i * M + m] = w.g[i * M + m] / den;
        }
        w.b[i] = x->mode ? go / den : -go / den;
        for (long c = 0; c < C; ++c) {
            double s = w.b[i] * z[c];
            for (long m = 0; m < M; ++m) s += S[c * M + m] * w.a[i * M + m];
            dq[i * C + c] = s;
        }
    }
    /* Suffix sweep; S and z are reused as R and r. */
    memset(S, 0, sizeof(double) * (size_t)(C * M));
    memset(z, 0, sizeof(double) * (size_t)C);
    if (!x->causal)
        for (long i = 0; i < N; ++i)
            for (long c = 0; c < C; ++c) {
                z[c] += w.b[i] * w.pq[i * C + c];
                for (long m = 0; m < M; ++m) S[c * M + m] += w.pq[i * C + c] * w.a[i * M + m];
            }
    for (long j = N - 1; j >= 0; --j) {
        if (x->causal)
            for (long c = 0; c < C; ++c) {
                z[c] += w.b[j] * w.pq[j * C + c];
                for (long m = 0; m < M; ++m) S[c * M + m] += w.pq[j * C + c] * w.a[j * M + m];
            }
        for (long c = 0; c < C; ++c) {
            double s = z[c];
            for (long m = 0; m < M; ++m) s += S[c * M + m] * w.v[j * M + m];
            dk[j * C + c] = s;
        }
        for (long m = 0; m < M; ++m) {
            double s = 0.0;
            for (long c = 0; c < C; ++c) s += S[c * M + m] * w.pk[j * C + c];
            dv[j * M + m] = s;
        }
    }
    free(S); free(z);
    bwd_free(&w);
    bwd_chain_phi(x, u);
}

static int check_bwd(const void *Q, const void *K, const void *V, const void *G, const double *dQ,
                     const double *dK, const double *dV, int dtype, long units, long N, long C, long M,
                     int mode) {
    if (units < 0 || N < 0 || C < 1 || M < 1 || (mode != 0 && mode != 1)) return 0;
    if (dtype != ORACLE_F64 && dtype != ORACLE_F32 && dtype != ORACLE_BF16) return 0;
    if (units > 0 && N > 0 && (!Q || !K || !V || !G || !dQ || !dK || !dV)) return 0;
    return 1;
}

/* Gradients of O1 (mode 0) or their magnitude companion (mode 1), by the
 * quadratic definition.  Q, K [units][N][C]; V, G [units][N][M]; outputs
 * double, same shapes. */
int oracle_backward_quadratic(const void *Q, const void *K, const void *V, const void *G, int dtype,
                              long units, long N, long C, long M, int causal, int mode, double *dQ,
                              double *dK, double *dV, int nthreads) {
    if (!check_bwd(Q, K, V, G, dQ, dK, dV, dtype, units, N, C, M, mode)) return ORACLE_BAD_ARG;
    bwd_ctx x = {Q, K, V, G, dtype, N, C, M, causal != 0, mode, dQ, dK, dV, 0};
    parallel_units(bwd_quadratic_unit, &x, units, nthreads);
    return x.bad ? ORACLE_NONPOSITIVE_DEN : ORACLE_OK;
}

/* The same, by the cumulative-sum form. */
int oracle_backward_recurrent(const void *Q, const void *K, const void *V, const void *G, int dtype,
                              long units, long N, long C, long M, int causal, int mode, double *dQ,
                              double *dK, double *dV, int nthreads) {
    if (!check_bwd(Q, K, V, G, dQ, dK, dV, dtype, units, N, C, M, mode)) return ORACLE_BAD_ARG;
    bwd_ctx x = {Q, K, V, G, dtype, N, C, M, causal != 0, mode, dQ, dK, dV, 0};
    parallel_units(bwd_recurrent_unit, &x, units, nthreads);
    return x.bad ? ORACLE_NONPOSITIVE_DEN : ORACLE_OK;
}
