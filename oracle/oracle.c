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
