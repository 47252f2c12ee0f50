/*
 * oracle.c -- plain fp64 CPU reference for the attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  The parity tests, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library; the HIP library never
 * does, and the two share no code, header, table or helper.
 *
 * What it computes is the plain definition, not the streaming method that the
 * GPU kernels use:
 *
 *   * three-pass safe softmax: pass 1 takes the maximum, pass 2 sums
 *     exp(x - max), pass 3 divides ('Online Softmax -- the mathematical heart
 *     of FlashAttention' section 1; 'Online softmax in attention -- why and
 *     how', section "The textbook softmax: stable, but two passes");
 *   * attention as softmax over one query's scores applied to the value rows,
 *     A_i = sum_j softmax(s_i)_j V_j with s_ij = scale * q_i . k_j
 *     ('Online Softmax -- the mathematical heart of FlashAttention' section 5;
 *     'Online Softmax & FlashAttention' (interview lesson), Step 2, where the
 *     scores are q K^T times scale with scale = 1/sqrt(d) by default);
 *   * the row log-sum-exp LSE = m + ln l, which is -inf for a row with no
 *     visible key ('Online Softmax & FlashAttention', Step 1 and Step 3).
 *
 * Readings where the pages leave a step open (each listed in the design notes):
 *   * a masked key is left out of the softmax; a row with no visible key has
 *     m = -inf, l = 0, output 0 and LSE = -inf ('Online Softmax & FlashAttention',
 *     Step 1: the fully masked row of the chunking example);
 *   * causal visibility is key j <= query i + (Nk - N): the queries are the last
 *     N positions of the key sequence, which is j <= i for N = Nk
 *     ('Online softmax in attention -- why and how', section "Why this matters
 *     for attention specifically");
 *   * key_lens[b] (clamped to [0, Nk]) hides keys j >= key_lens[b] of batch b
 *     from every query; it combines with the causal rule by AND;
 *   * inputs are the stored fp32 / bf16 values widened exactly to fp64.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared -pthread oracle.c -lm
 * (no fast-math: -inf must stay IEEE -inf).
 *
 * The row-wise softmax (oracle_softmax_rows_f64) is the same three-pass
 * definition applied to every row of a matrix; it checks the streaming
 * softmax / log-sum-exp kernel ('Online Softmax' research-hub page, "Why it
 * matters": the recurrence also streams rows too wide for on-chip memory).
 *
 * The backward pass (oracle_attention_backward_f64) is the exact gradient of
 * the forward above for a loss L = sum dO . O, written out by the chain rule
 * ('Online softmax in attention -- why and how', "Where this is heading":
 * backward recomputes the scores from the cached row statistics; the
 * gradient itself is plain calculus of the same definition):
 *     P = softmax rows of the visible scores, O = P V,
 *     D_i = dO_i . O_i,  dP_ij = dO_i . v_j,  dS_ij = P_ij (dP_ij - D_i),
 *     dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
 *     dV_j = sum_i P_ij dO_i,
 * with masked (query, key) pairs contributing nothing; a row with no visible
 * key has P = 0 and dQ_i = 0.  Pinned by central differences of the forward.
 *
 * Parity pins (tests/test_oracle.py): the worked softmax examples printed on
 * the pages, the chunk-merge invariant of 'Online Softmax & FlashAttention'
 * Step 1, the tiled V1 shapes of its Step 2, closed forms, invariants and a
 * library cross-check.  Every exported function here is pinned.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F64 = 0, ORACLE_F32 = 1, ORACLE_BF16 = 2 };

/* Exact widening of one stored element to fp64. */
static double widen(const void *base, int dtype, size_t idx)
{
    if (dtype == ORACLE_F64)
        return ((const double *)base)[idx];
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    {
        uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
}

/*
 * Three-pass safe softmax of x[0..n).  Entries equal to -inf are masked and
 * get weight 0.  If every entry is masked (or n == 0): m = -inf, l = 0 and
 * y = 0.  Outputs: y[0..n) (may be NULL), *m_out = max, *l_out = sum of
 * exp(x - max).  Returns 0.
 */
int oracle_softmax_f64(const double *x, long n, double *y, double *m_out, double *l_out)
{
    double m = -INFINITY, l = 0.0;
    long j;
    for (j = 0; j < n; ++j)                 /* pass 1: maximum */
        if (x[j] > m)
            m = x[j];
    if (m == -INFINITY) {
        if (y)
            for (j = 0; j < n; ++j)
                y[j] = 0.0;
        *m_out = m;
        *l_out = 0.0;
        return 0;
    }
    for (j = 0; j < n; ++j)                 /* pass 2: normaliser */
        l += exp(x[j] - m);
    if (y)
        for (j = 0; j < n; ++j)             /* pass 3: divide */
            y[j] = exp(x[j] - m) / l;
    *m_out = m;
    *l_out = l;
    return 0;
}

/*
 * Row-wise softmax of a [rows, cols] matrix in fp64: every row goes through
 * the three-pass definition above (-inf entries masked).  X has element type
 * `dtype` (0 = fp64, 1 = fp32, 2 = bf16 bits).  Y: fp64 [rows, cols] or NULL;
 * LSE: fp64 [rows], m + ln l, -inf for a fully masked row.  Returns 0, -1 for
 * invalid arguments, -2 when memory runs out.
 */
int oracle_softmax_rows_f64(const void *X, int dtype, long rows, long cols, double *Y,
                            double *LSE)
{
    double *x, m, l;
    long r, j;
    if (rows < 0 || cols < 0 || dtype < ORACLE_F64 || dtype > ORACLE_BF16 || !LSE)
        return -1;
    if (rows > 0 && cols > 0 && !X)
        return -1;
    x = (double *)malloc(sizeof(double) * (size_t)(cols > 0 ? cols : 1));
    if (!x)
        return -2;
    for (r = 0; r < rows; ++r) {
        for (j = 0; j < cols; ++j)
            x[j] = widen(X, dtype, (size_t)r * cols + j);
        oracle_softmax_f64(x, cols, Y ? Y + (size_t)r * cols : NULL, &m, &l);
        LSE[r] = l > 0.0 ? m + log(l) : -INFINITY;
    }
    free(x);
    return 0;
}

typedef struct {
    const void *Q, *K, *V;
    int dtype;
    long B, H, N, Nk, d;
    double scale;
    int causal;
    const int32_t *key_lens;    /* host int32[B] or NULL */
    long nrows;
    const int64_t *rows;        /* flat indices (b*H + h)*N + i, or NULL = all */
    double *O;                  /* [nrows, d] */
    double *LSE;                /* [nrows] */
} attn_args;

typedef struct {
    const attn_args *a;
    long begin, end;            /* range of output rows */
    int status;
} attn_job;

/* Number of keys visible to query i of batch b: always a prefix [0, n). */
static long visible_keys(const attn_args *a, long b, long i)
{
    long n = a->Nk;
    if (a->key_lens) {
        long kl = a->key_lens[b];
        if (kl < 0)
            kl = 0;
        if (kl > a->Nk)
            kl = a->Nk;
        n = kl;
    }
    if (a->causal) {
        long lim = i + (a->Nk - a->N) + 1;  /* keys j <= i + Nk - N */
        if (lim < 0)
            lim = 0;
        if (lim < n)
            n = lim;
    }
    return n;
}

static void attend_row(const attn_args *a, long out_row, double *s)
{
    long flat = a->rows ? (long)a->rows[out_row] : out_row;
    long bh = flat / a->N, i = flat % a->N, b = bh / a->H;
    long d = a->d, Nk = a->Nk, nvis = visible_keys(a, b, i);
    size_t qoff = ((size_t)bh * a->N + i) * d, kvoff = (size_t)bh * Nk * d;
    double *o = a->O + (size_t)out_row * d;
    double m = -INFINITY, l = 0.0;
    long j, c;

    for (c = 0; c < d; ++c)
        o[c] = 0.0;
    if (nvis == 0) {                        /* fully masked row */
        a->LSE[out_row] = -INFINITY;
        return;
    }
    for (j = 0; j < nvis; ++j) {            /* scores s_j = scale * q . k_j */
        double dot = 0.0;
        for (c = 0; c < d; ++c)
            dot += widen(a->Q, a->dtype, qoff + c) * widen(a->K, a->dtype, kvoff + (size_t)j * d + c);
        s[j] = a->scale * dot;
    }
    for (j = 0; j < nvis; ++j)              /* pass 1: maximum */
        if (s[j] > m)
            m = s[j];
    for (j = 0; j < nvis; ++j)              /* pass 2: normaliser */
        l += exp(s[j] - m);
    for (j = 0; j < nvis; ++j) {            /* pass 3: weighted values / l */
        double p = exp(s[j] - m) / l;
        for (c = 0; c < d; ++c)
            o[c] += p * widen(a->V, a->dtype, kvoff + (size_t)j * d + c);
    }
    a->LSE[out_row] = m + log(l);
}

static void *attend_job(void *arg)
{
    attn_job *job = (attn_job *)arg;
    const attn_args *a = job->a;
    double *s = (double *)malloc(sizeof(double) * (size_t)(a->Nk > 0 ? a->Nk : 1));
    long r;
    if (!s) {
        job->status = -2;
        return NULL;
    }
    for (r = job->begin; r < job->end; ++r)
        attend_row(a, r, s);
    free(s);
    job->status = 0;
    return NULL;
}

/*
 * Attention forward in fp64 for every query row (rows == NULL, nrows must be
 * B*H*N) or for the listed flat rows (b*H + h)*N + i.
 * Q: [B,H,N,d], K and V: [B,H,Nk,d], row-major, element type `dtype`
 * (0 = fp64, 1 = fp32, 2 = bf16 bits).  key_lens: host int32[B] or NULL.
 * O: fp64 [nrows, d]; LSE: fp64 [nrows].  nthreads <= 0 means 1.
 * Returns 0, -1 for invalid arguments, -2 when memory runs out.
 */
int oracle_attention_f64(const void *Q, const void *K, const void *V, int dtype,
                         long B, long H, long N, long Nk, long d, double scale, int causal,
                         const int32_t *key_lens, long nrows, const int64_t *rows,
                         double *O, double *LSE, int nthreads)
{
    attn_args a;
    attn_job *jobs;
    pthread_t *tids;
    char *started;
    long r, per, t;
    int status = 0;

    if (B < 0 || H < 0 || N < 0 || Nk < 0 || d <= 0 || nrows < 0 ||
        dtype < ORACLE_F64 || dtype > ORACLE_BF16 || (causal != 0 && causal != 1))
        return -1;
    if (!rows && nrows != B * H * N)
        return -1;
    if (rows)
        for (r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= B * H * N)
                return -1;
    if (nrows == 0)
        return 0;
    if (!O || !LSE || !Q || (Nk > 0 && (!K || !V)))
        return -1;

    a.Q = Q; a.K = K; a.V = V; a.dtype = dtype;
    a.B = B; a.H = H; a.N = N; a.Nk = Nk; a.d = d;
    a.scale = scale; a.causal = causal; a.key_lens = key_lens;
    a.nrows = nrows; a.rows = rows; a.O = O; a.LSE = LSE;

    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > nrows)
        nthreads = (int)nrows;
    jobs = (attn_job *)calloc((size_t)nthreads, sizeof *jobs);
    tids = (pthread_t *)calloc((size_t)nthreads, sizeof *tids);
    started = (char *)calloc((size_t)nthreads, 1);
    if (!jobs || !tids || !started) {
        free(jobs);
        free(tids);
        free(started);
        return -2;
    }
    per = (nrows + nthreads - 1) / nthreads;
    for (t = 0; t < nthreads; ++t) {
        jobs[t].a = &a;
        jobs[t].begin = t * per < nrows ? t * per : nrows;
        jobs[t].end = (t + 1) * per < nrows ? (t + 1) * per : nrows;
        jobs[t].status = -2;
    }
    for (t = 1; t < nthreads; ++t)
        started[t] = pthread_create(&tids[t], NULL, attend_job, &jobs[t]) == 0;
    attend_job(&jobs[0]);
    for (t = 1; t < nthreads; ++t) {
        if (started[t])
            pthread_join(tids[t], NULL);
        else
            attend_job(&jobs[t]);           /* no thread: run it here */
    }
    for (t = 0; t < nthreads; ++t)
        if (jobs[t].status != 0)
            status = jobs[t].status;
    free(jobs);
    free(tids);
    free(started);
    return status;
}

/* ------------------------------------------------------------- backward */

typedef struct {
    const void *Q, *K, *V, *dO;
    int dtype;
    long B, H, N, Nk, d;
    double scale;
    int causal;
    const int32_t *key_lens;
    const int64_t *heads;       /* flat b*H + h, or NULL = all */
    double *dQ, *dK, *dV;       /* [nheads, N, d], [nheads, Nk, d] x 2 */
} bwd_args;

typedef struct {
    const bwd_args *a;
    long begin, end;            /* range of heads (indices into the head list) */
    int status;
} bwd_job;

/* Gradients of one head: row by row, the row's softmax (three passes), its
 * output, then the chain rule for that row's contributions. */
static void backward_head(const bwd_args *a, long hidx, double *s, double *p, double *o)
{
    long bh = a->heads ? (long)a->heads[hidx] : hidx;
    long b = bh / a->H, d = a->d, N = a->N, Nk = a->Nk, i, j, c;
    size_t qbase = (size_t)bh * N * d, kvbase = (size_t)bh * Nk * d;
    double *dQ = a->dQ + (size_t)hidx * N * d;
    double *dK = a->dK + (size_t)hidx * Nk * d;
    double *dV = a->dV + (size_t)hidx * Nk * d;
    attn_args va;               /* only the fields visible_keys reads */

    memset(&va, 0, sizeof va);
    va.N = N; va.Nk = Nk; va.causal = a->causal; va.key_lens = a->key_lens;
    for (c = 0; c < N * d; ++c)
        dQ[c] = 0.0;
    for (c = 0; c < Nk * d; ++c) {
        dK[c] = 0.0;
        dV[c] = 0.0;
    }
    for (i = 0; i < N; ++i) {
        long nvis = visible_keys(&va, b, i);
        size_t qo = qbase + (size_t)i * d;
        double m = -INFINITY, l = 0.0, D = 0.0;
        if (nvis == 0)
            continue;                       /* P = 0: no gradient through this row */
        for (j = 0; j < nvis; ++j) {        /* scores */
            double dot = 0.0;
            for (c = 0; c < d; ++c)
                dot += widen(a->Q, a->dtype, qo + c) * widen(a->K, a->dtype, kvbase + (size_t)j * d + c);
            s[j] = dot * a->scale;
        }
        for (j = 0; j < nvis; ++j)          /* pass 1 */
            if (s[j] > m)
                m = s[j];
        for (j = 0; j < nvis; ++j)          /* pass 2 */
            l = l + exp(s[j] - m);
        for (c = 0; c < d; ++c)
            o[c] = 0.0;
        for (j = 0; j < nvis; ++j) {        /* pass 3: P and O = P V */
            p[j] = exp(s[j] - m) / l;
            for (c = 0; c < d; ++c)
                o[c] += p[j] * widen(a->V, a->dtype, kvbase + (size_t)j * d + c);
        }
        for (c = 0; c < d; ++c)             /* D_i = dO_i . O_i */
            D += widen(a->dO, a->dtype, qo + c) * o[c];
        for (j = 0; j < nvis; ++j) {
            size_t ko = kvbase + (size_t)j * d;
            double dp = 0.0, ds;
            for (c = 0; c < d; ++c)         /* dP_ij = dO_i . v_j */
                dp += widen(a->dO, a->dtype, qo + c) * widen(a->V, a->dtype, ko + c);
            ds = p[j] * (dp - D);
            for (c = 0; c < d; ++c) {
                dQ[(size_t)i * d + c] += a->scale * ds * widen(a->K, a->dtype, ko + c);
                dK[(size_t)j * d + c] += a->scale * ds * widen(a->Q, a->dtype, qo + c);
                dV[(size_t)j * d + c] += p[j] * widen(a->dO, a->dtype, qo + c);
            }
        }
    }
}

static void *backward_job(void *arg)
{
    bwd_job *job = (bwd_job *)arg;
    const bwd_args *a = job->a;
    size_t nk = (size_t)(a->Nk > 0 ? a->Nk : 1);
    double *s = (double *)malloc(sizeof(double) * nk);
    double *p = (double *)malloc(sizeof(double) * nk);
    double *o = (double *)malloc(sizeof(double) * (size_t)a->d);
    long h;
    if (!s || !p || !o) {
        free(s);
        free(p);
        free(o);
        job->status = -2;
        return NULL;
    }
    for (h = job->begin; h < job->end; ++h)
        backward_head(a, h, s, p, o);
    free(s);
    free(p);
    free(o);
    job->status = 0;
    return NULL;
}

/*
 * Attention backward in fp64: dQ, dK, dV of L = sum dO . O for the forward of
 * oracle_attention_f64 (same masking rules), for every head (heads == NULL,
 * nheads must be B*H) or for the listed flat heads b*H + h.
 * Q, dO: [B,H,N,d]; K, V: [B,H,Nk,d]; element type `dtype` as in the forward.
 * dQ: fp64 [nheads, N, d]; dK, dV: fp64 [nheads, Nk, d].  Returns 0, -1 for
 * invalid arguments, -2 when memory runs out.
 */
int oracle_attention_backward_f64(const void *Q, const void *K, const void *V, const void *dO,
                                  int dtype, long B, long H, long N, long Nk, long d,
                                  double scale, int causal, const int32_t *key_lens,
                                  long nheads, const int64_t *heads,
                                  double *dQ, double *dK, double *dV, int nthreads)
{
    bwd_args a;
    bwd_job *jobs;
    pthread_t *tids;
    char *started;
    long r, per, t;
    int status = 0;

    if (B < 0 || H < 0 || N < 0 || Nk < 0 || d <= 0 || nheads < 0 ||
        dtype < ORACLE_F64 || dtype > ORACLE_BF16 || (causal != 0 && causal != 1))
        return -1;
    if (!heads && nheads != B * H)
        return -1;
    if (heads)
        for (r = 0; r < nheads; ++r)
            if (heads[r] < 0 || heads[r] >= B * H)
                return -1;
    if (nheads == 0)
        return 0;
    if ((N > 0 && (!Q || !dO || !dQ)) || (Nk > 0 && (!K || !V || !dK || !dV)))
        return -1;

    a.Q = Q; a.K = K; a.V = V; a.dO = dO; a.dtype = dtype;
    a.B = B; a.H = H; a.N = N; a.Nk = Nk; a.d = d;
    a.scale = scale; a.causal = causal; a.key_lens = key_lens;
    a.heads = heads; a.dQ = dQ; a.dK = dK; a.dV = dV;

    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > nheads)
        nthreads = (int)nheads;
    jobs = (bwd_job *)calloc((size_t)nthreads, sizeof *jobs);
    tids = (pthread_t *)calloc((size_t)nthreads, sizeof *tids);
    started = (char *)calloc((size_t)nthreads, 1);
    if (!jobs || !tids || !started) {
        free(jobs);
        free(tids);
        free(started);
        return -2;
    }
    per = (nheads + nthreads - 1) / nthreads;
    for (t = 0; t < nthreads; ++t) {
        jobs[t].a = &a;
        jobs[t].begin = t * per < nheads ? t * per : nheads;
        jobs[t].end = (t + 1) * per < nheads ? (t + 1) * per : nheads;
        jobs[t].status = -2;
    }
    for (t = 1; t < nthreads; ++t)
        started[t] = pthread_create(&tids[t], NULL, backward_job, &jobs[t]) == 0;
    backward_job(&jobs[0]);
    for (t = 1; t < nthreads; ++t) {
        if (started[t])
            pthread_join(tids[t], NULL);
        else
            backward_job(&jobs[t]);
    }
    for (t = 0; t < nthreads; ++t)
        if (jobs[t].status != 0)
            status = jobs[t].status;
    free(jobs);
    free(tids);
    free(started);
    return status;
}
