/*
 * FP64 reference for exact scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the attention library calls, links or
 * includes this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the GPU path.
 *
 * What it computes is the plain definition of the attention call that the
 * Stream-CQSA pages describe as a drop-in for PyTorch's
 * scaled_dot_product_attention (stream-cqsa 2.2.0 -> 2.2.2 diff, stream_cqsa/api.py,
 * the attention() docstring): for batch b, query head h, query row i, with
 * g = Hq / Hkv and key/value head h' = floor(h / g),
 *
 *     s_ij  = sigma * sum_t q[b,h,i,t] * k[b,h',j,t]          (sigma: the fp32 scale, widened)
 *     m_i   = max_{j in V(i)} s_ij
 *     l_i   = sum_{j in V(i)} exp(s_ij - m_i)
 *     O_i   = sum_{j in V(i)} exp(s_ij - m_i) * v[b,h',j,:] / l_i
 *     lse_i = m_i + ln(l_i)
 *
 * V(i) is every key when not causal and {j : j <= i + Nk - Nq} when causal
 * (a causal query block sits at the end of the key sequence; with Nq == Nk
 * this is the ordinary lower-triangular mask).  A key range [lo, hi) narrows
 * V(i) further; that is the partial result of one KV chunk, returned as the
 * unnormalised triple (sum_j exp(s_ij - m) v_j, m, l).  The exact merge of two
 * such triples (the log-sum-exp combination the pages rely on to give the
 * monolithic answer from decomposed pieces, stream-cqsa README "Use") is
 * oracle_merge below.
 *
 * Arithmetic: inputs are the exact fp16 / bf16 values widened to double; each
 * product of two such values is exact in double.  Each row is done in two
 * passes (scores and their maximum, then weights), and l and every output
 * coordinate are accumulated with Neumaier's compensated summation
 * (Neumaier, 1974).  Rows are handed out to POSIX threads one small batch at a
 * time; each row's result depends only on the row.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1 };

/* IEEE binary16 bits -> double (exact): sign, 5-bit exponent (bias 15), 10-bit fraction. */
double oracle_f16_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
    } else if (e == 0x1F) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(f | 0x400), e - 25); /* (1024 + f) * 2^(e - 15 - 10) */
    }
    return sign ? -v : v;
}

/* bfloat16 bits -> double (exact): the upper half of a binary32. */
double oracle_bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Every 16-bit pattern of each input format, widened once by the two functions above (whose every
 * output the tests check), so that the inner loops read a table instead of decoding. */
static double g_decode[2][65536];
static pthread_once_t g_decode_once = PTHREAD_ONCE_INIT;

static void fill_decode_tables(void) {
    for (uint32_t u = 0; u < 65536u; ++u) {
        g_decode[0][u] = oracle_f16_to_double((uint16_t)u);
        g_decode[1][u] = oracle_bf16_to_double((uint16_t)u);
    }
}

typedef struct {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    int32_t dtype;       /* ORACLE_F16 or ORACLE_BF16 */
    int32_t causal;
    int64_t B, Hq, Hkv, Nq, Nk, D;
    int64_t q_stride[3]; /* element strides of batch, head, row; the head-dim stride is 1 */
    int64_t k_stride[3];
    int64_t v_stride[3];
    float scale;
} oracle_problem;

typedef struct {
    const oracle_problem* p;
    const int64_t* rows; /* triples (b, h, i) */
    int64_t nrows;
    int64_t* next_row;   /* shared by the workers: the next row not yet taken */
    int64_t key_lo, key_hi;
    int32_t partial;
    double* out_o;       /* [nrows][D] */
    double* out_m;
    double* out_l;
    double* out_lse;
    int32_t status;
} oracle_job;

static inline double elem(const oracle_problem* p, const uint16_t* base, uint64_t off) {
    return g_decode[p->dtype == ORACLE_BF16 ? 1 : 0][base[off]];
}

/* Neumaier: add x to (sum, comp), where comp collects the exact rounding error of every addition.
 * The error is formed by Knuth's TwoSum, which needs no test of which operand is larger in
 * magnitude; Neumaier's formulation branches on |sum| >= |x| instead, and both give the same exact
 * error of a finite sum. */
static inline void nsum(double* sum, double* comp, double x) {
    const double t = *sum + x;
    const double z = t - *sum;
    *comp += (*sum - (t - z)) + (x - z);
    *sum = t;
}

/* Rows in batches of this many go to the next free worker. */
enum { ROW_BATCH = 4 };

static void* row_worker(void* arg) {
    oracle_job* job = (oracle_job*)arg;
    const oracle_problem* p = job->p;
    const int64_t D = p->D;
    const double sigma = (double)p->scale;
    const int64_t g = p->Hq / p->Hkv;
    double* s = (double*)malloc(sizeof(double) * (size_t)(p->Nk > 0 ? p->Nk : 1));
    double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
    double* osum = (double*)malloc(sizeof(double) * (size_t)D);
    double* ocomp = (double*)malloc(sizeof(double) * (size_t)D);
    if (!s || !qrow || !osum || !ocomp) {
        job->status = -2;
        free(s); free(qrow); free(osum); free(ocomp);
        return NULL;
    }
    for (;;) {
      const int64_t r0 = __atomic_fetch_add(job->next_row, (int64_t)ROW_BATCH, __ATOMIC_RELAXED);
      if (r0 >= job->nrows) break;
      const int64_t r1 = r0 + ROW_BATCH < job->nrows ? r0 + ROW_BATCH : job->nrows;
      for (int64_t r = r0; r < r1; ++r) {
        const int64_t b = job->rows[3 * r + 0];
        const int64_t h = job->rows[3 * r + 1];
        const int64_t i = job->rows[3 * r + 2];
        const int64_t hk = h / g;
        /* visible keys: [lo, hi) */
        int64_t lo = job->key_lo < 0 ? 0 : job->key_lo;
        int64_t hi = job->key_hi > p->Nk ? p->Nk : job->key_hi;
        if (p->causal) {
            int64_t last = i + (p->Nk - p->Nq); /* last visible key */
            if (hi > last + 1) hi = last + 1;
        }
        const uint64_t qoff = (uint64_t)(b * p->q_stride[0] + h * p->q_stride[1] + i * p->q_stride[2]);
        for (int64_t t = 0; t < D; ++t) qrow[t] = elem(p, p->q, qoff + (uint64_t)t);

        /* pass 1: scores and their maximum */
        double m = -INFINITY;
        for (int64_t j = lo; j < hi; ++j) {
            const uint64_t koff = (uint64_t)(b * p->k_stride[0] + hk * p->k_stride[1] + j * p->k_stride[2]);
            double dot = 0.0;
            for (int64_t t = 0; t < D; ++t) dot += qrow[t] * elem(p, p->k, koff + (uint64_t)t);
            s[j - lo] = sigma * dot;
            if (s[j - lo] > m) m = s[j - lo];
        }
        /* pass 2: weights, their sum, and the weighted sum of values */
        double lsum = 0.0, lcomp = 0.0;
        for (int64_t t = 0; t < D; ++t) { osum[t] = 0.0; ocomp[t] = 0.0; }
        for (int64_t j = lo; j < hi; ++j) {
            const double w = exp(s[j - lo] - m);
            nsum(&lsum, &lcomp, w);
            const uint64_t voff = (uint64_t)(b * p->v_stride[0] + hk * p->v_stride[1] + j * p->v_stride[2]);
            for (int64_t t = 0; t < D; ++t) nsum(&osum[t], &ocomp[t], w * elem(p, p->v, voff + (uint64_t)t));
        }
        const double l = lsum + lcomp;
        double* o = job->out_o + (size_t)r * (size_t)D;
        if (job->partial) {
            for (int64_t t = 0; t < D; ++t) o[t] = (hi > lo) ? osum[t] + ocomp[t] : 0.0;
            if (job->out_m) job->out_m[r] = m;           /* -inf for an empty key set */
            if (job->out_l) job->out_l[r] = (hi > lo) ? l : 0.0;
        } else {
            for (int64_t t = 0; t < D; ++t) o[t] = (hi > lo) ? (osum[t] + ocomp[t]) / l : NAN;
            if (job->out_lse) job->out_lse[r] = (hi > lo) ? m + log(l) : -INFINITY;
            if (job->out_m) job->out_m[r] = m;
            if (job->out_l) job->out_l[r] = (hi > lo) ? l : 0.0;
        }
      }
    }
    free(s); free(qrow); free(osum); free(ocomp);
    job->status = 0;
    return NULL;
}

/*
 * Attention for a list of rows.  rows: nrows triples (b, h, i).  Keys are
 * restricted to [key_lo, key_hi) intersected with V(i).  partial = 0 gives the
 * normalised output and lse (out_m / out_l optional); partial = 1 gives the
 * unnormalised triple (out_o = sum exp(s - m) v, out_m, out_l), with the
 * identity (0, -inf, 0) for an empty key set.  Returns 0 on success, -1 on a
 * bad argument, -2 when memory runs out.
 */
int oracle_rows(const oracle_problem* p, const int64_t* rows, int64_t nrows, int64_t key_lo, int64_t key_hi,
                int32_t partial, double* out_o, double* out_m, double* out_l, double* out_lse, int32_t nthreads) {
    if (!p || (!rows && nrows > 0) || nrows < 0 || !out_o) return -1;
    if (p->Hkv <= 0 || p->Hq % p->Hkv != 0 || p->D <= 0) return -1;
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= p->B || h < 0 || h >= p->Hq || i < 0 || i >= p->Nq) return -1;
    }
    pthread_once(&g_decode_once, fill_decode_tables);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > nrows) nthreads = (int32_t)(nrows > 0 ? nrows : 1);
    pthread_t th[256];
    int joinable[256];
    oracle_job jobs[256];
    int64_t next_row = 0;
    int njobs = 0;
    for (int t = 0; t < nthreads; ++t) {
        oracle_job* j = &jobs[t];
        j->p = p; j->rows = rows; j->key_lo = key_lo; j->key_hi = key_hi; j->partial = partial;
        j->out_o = out_o; j->out_m = out_m; j->out_l = out_l; j->out_lse = out_lse; j->status = 0;
        j->nrows = nrows;
        j->next_row = &next_row;
        njobs = t + 1;
        joinable[t] = pthread_create(&th[t], NULL, row_worker, j) == 0;
        if (!joinable[t]) row_worker(j); /* no thread available: take rows here */
    }
    int status = 0;
    for (int t = 0; t < njobs; ++t) {
        if (joinable[t]) pthread_join(th[t], NULL);
        if (jobs[t].status != 0) status = jobs[t].status;
    }
    return status;
}

/*
 * Exact merge of two partial triples for nrows rows (the log-sum-exp
 * combination):  m = max(ma, mb),  alpha = exp(ma - m),  beta = exp(mb - m),
 * l = alpha la + beta lb,  O = alpha Oa + beta Ob.  A triple whose m is -inf
 * is the empty set and contributes nothing (its weight is taken as 0, never
 * exp(-inf - -inf)).  Outputs may alias either input.
 */
void oracle_merge(int64_t nrows, int64_t D, const double* oa, const double* ma, const double* la, const double* ob,
                  const double* mb, const double* lb, double* o, double* m, double* l) {
    for (int64_t r = 0; r < nrows; ++r) {
        const double a_m = ma[r], b_m = mb[r];
        const double mm = a_m > b_m ? a_m : b_m;
        const double alpha = (a_m == -INFINITY) ? 0.0 : exp(a_m - mm);
        const double beta = (b_m == -INFINITY) ? 0.0 : exp(b_m - mm);
        const double a_l = la[r], b_l = lb[r];
        for (int64_t t = 0; t < D; ++t) {
            const double x = alpha * oa[r * D + t] + beta * ob[r * D + t];
            o[r * D + t] = x;
        }
        l[r] = alpha * a_l + beta * b_l;
        m[r] = mm;
    }
}

/*
 * Gradients of the same attention for an upstream gradient dO (fp16 / bf16, like q), by the
 * definition (the derivative of softmax(sigma q k^T) v), for the backward the Stream-CQSA pages ship
 * beside the forward (stream-cqsa 2.2.0 -> 2.2.2 diff, README.md, kernel table):
 *
 *     P_ij  = exp(s_ij - m_i) / l_i                        (j in V(i), 0 otherwise)
 *     dV_j  = sum_i P_ij dO_i
 *     dP_ij = dO_i . v_j
 *     D_i   = sum_j P_ij dP_ij
 *     dS_ij = P_ij (dP_ij - D_i)
 *     dQ_i  = sigma sum_j dS_ij k_j
 *     dK_j  = sigma sum_i dS_ij q_i
 *
 * With GQA, dK and dV of key/value head h' sum over the query heads h with floor(h / g) = h'.
 * Two passes: per query row (m_i, l_i, D_i and dQ_i), then per key row (dK_j and dV_j), each spread
 * over threads with no shared accumulator.  Plain double sums (the test sizes keep them far below
 * the tolerances compared against).
 */
typedef struct {
    const oracle_problem* p;
    const uint16_t* dout;
    int64_t do_stride[3];
    double* stats;      /* [B][Hq][Nq][3]: m, l, D */
    double* dq;         /* [B][Hq][Nq][D] */
    double* dk;         /* [B][Hkv][Nk][D] */
    double* dv;
    int64_t begin, end; /* rows of the pass */
    int32_t status;
} oracle_bwd_job;

static double dot_row(const oracle_problem* p, const uint16_t* a, uint64_t ao, const uint16_t* b, uint64_t bo) {
    double d = 0.0;
    for (int64_t t = 0; t < p->D; ++t) d += elem(p, a, ao + (uint64_t)t) * elem(p, b, bo + (uint64_t)t);
    return d;
}

static void visible_keys(const oracle_problem* p, int64_t i, int64_t* hi) {
    *hi = p->Nk;
    if (p->causal) {
        const int64_t last = i + (p->Nk - p->Nq);
        if (*hi > last + 1) *hi = last + 1;
    }
}

/* pass 1: one query row (b, h, i) per step */
static void* bwd_query_worker(void* arg) {
    oracle_bwd_job* job = (oracle_bwd_job*)arg;
    const oracle_problem* p = job->p;
    const int64_t D = p->D, g = p->Hq / p->Hkv;
    const double sigma = (double)p->scale;
    double* s = (double*)malloc(sizeof(double) * (size_t)(p->Nk > 0 ? p->Nk : 1));
    double* dp = (double*)malloc(sizeof(double) * (size_t)(p->Nk > 0 ? p->Nk : 1));
    if (!s || !dp) {
        job->status = -2;
        free(s); free(dp);
        return NULL;
    }
    for (int64_t r = job->begin; r < job->end; ++r) {
        const int64_t i = r % p->Nq, h = (r / p->Nq) % p->Hq, b = r / (p->Nq * p->Hq), hk = h / g;
        int64_t hi;
        visible_keys(p, i, &hi);
        const uint64_t qo = (uint64_t)(b * p->q_stride[0] + h * p->q_stride[1] + i * p->q_stride[2]);
        const uint64_t oo = (uint64_t)(b * job->do_stride[0] + h * job->do_stride[1] + i * job->do_stride[2]);
        double m = -INFINITY;
        for (int64_t j = 0; j < hi; ++j) {
            const uint64_t ko = (uint64_t)(b * p->k_stride[0] + hk * p->k_stride[1] + j * p->k_stride[2]);
            const uint64_t vo = (uint64_t)(b * p->v_stride[0] + hk * p->v_stride[1] + j * p->v_stride[2]);
            s[j] = sigma * dot_row(p, p->q, qo, p->k, ko);
            dp[j] = dot_row(p, job->dout, oo, p->v, vo);
            if (s[j] > m) m = s[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j < hi; ++j) l += exp(s[j] - m);
        double Di = 0.0;
        for (int64_t j = 0; j < hi; ++j) Di += exp(s[j] - m) / l * dp[j];
        double* st = job->stats + 3 * (size_t)r;
        st[0] = m;
        st[1] = l;
        st[2] = Di;
        double* dq = job->dq + (size_t)r * (size_t)D;
        for (int64_t t = 0; t < D; ++t) dq[t] = 0.0;
        for (int64_t j = 0; j < hi; ++j) {
            const double ds = exp(s[j] - m) / l * (dp[j] - Di);
            const uint64_t ko = (uint64_t)(b * p->k_stride[0] + hk * p->k_stride[1] + j * p->k_stride[2]);
            for (int64_t t = 0; t < D; ++t) dq[t] += sigma * ds * elem(p, p->k, ko + (uint64_t)t);
        }
    }
    free(s); free(dp);
    job->status = 0;
    return NULL;
}

/* pass 2: one key row (b, h', j) per step, summing over the group's query heads and rows */
static void* bwd_key_worker(void* arg) {
    oracle_bwd_job* job = (oracle_bwd_job*)arg;
    const oracle_problem* p = job->p;
    const int64_t D = p->D, g = p->Hq / p->Hkv;
    const double sigma = (double)p->scale;
    for (int64_t r = job->begin; r < job->end; ++r) {
        const int64_t j = r % p->Nk, hk = (r / p->Nk) % p->Hkv, b = r / (p->Nk * p->Hkv);
        const uint64_t ko = (uint64_t)(b * p->k_stride[0] + hk * p->k_stride[1] + j * p->k_stride[2]);
        const uint64_t vo = (uint64_t)(b * p->v_stride[0] + hk * p->v_stride[1] + j * p->v_stride[2]);
        double* dk = job->dk + (size_t)r * (size_t)D;
        double* dv = job->dv + (size_t)r * (size_t)D;
        for (int64_t t = 0; t < D; ++t) dk[t] = dv[t] = 0.0;
        for (int64_t h = hk * g; h < (hk + 1) * g; ++h) {
            /* rows that see key j: all, or i >= j - (Nk - Nq) when causal */
            int64_t i0 = 0;
            if (p->causal) i0 = j - (p->Nk - p->Nq) > 0 ? j - (p->Nk - p->Nq) : 0;
            for (int64_t i = i0; i < p->Nq; ++i) {
                const int64_t qr = (b * p->Hq + h) * p->Nq + i;
                const double* st = job->stats + 3 * (size_t)qr;
                const uint64_t qo = (uint64_t)(b * p->q_stride[0] + h * p->q_stride[1] + i * p->q_stride[2]);
                const uint64_t oo = (uint64_t)(b * job->do_stride[0] + h * job->do_stride[1] + i * job->do_stride[2]);
                const double sij = sigma * dot_row(p, p->q, qo, p->k, ko);
                const double P = exp(sij - st[0]) / st[1];
                const double dP = dot_row(p, job->dout, oo, p->v, vo);
                const double ds = P * (dP - st[2]);
                for (int64_t t = 0; t < D; ++t) {
                    dv[t] += P * elem(p, job->dout, oo + (uint64_t)t);
                    dk[t] += sigma * ds * elem(p, p->q, qo + (uint64_t)t);
                }
            }
        }
    }
    job->status = 0;
    return NULL;
}

static int run_pass(void* (*fn)(void*), oracle_bwd_job* base, int64_t n, int32_t nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > n) nthreads = (int32_t)(n > 0 ? n : 1);
    pthread_t th[256];
    int joinable[256];
    oracle_bwd_job jobs[256];
    const int64_t per = (n + nthreads - 1) / nthreads;
    int njobs = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = *base;
        jobs[t].begin = (int64_t)t * per;
        jobs[t].end = jobs[t].begin + per < n ? jobs[t].begin + per : n;
        jobs[t].status = 0;
        if (jobs[t].begin >= jobs[t].end) break;
        njobs = t + 1;
        joinable[t] = pthread_create(&th[t], NULL, fn, &jobs[t]) == 0;
        if (!joinable[t]) fn(&jobs[t]);
    }
    int status = 0;
    for (int t = 0; t < njobs; ++t) {
        if (joinable[t]) pthread_join(th[t], NULL);
        if (jobs[t].status != 0) status = jobs[t].status;
    }
    return status;
}

/*
 * dq [B][Hq][Nq][D], dk and dv [B][Hkv][Nk][D] (contiguous, double) for the problem p and the
 * upstream gradient dout (p's dtype, [B][Hq][Nq][D] with element strides do_stride and a unit
 * head-dim stride).  Causal calls need Nq <= Nk.  Returns 0, -1 on a bad argument, -2 when memory
 * runs out.
 */
int oracle_backward(const oracle_problem* p, const uint16_t* dout, const int64_t* do_stride, double* dq, double* dk,
                    double* dv, int32_t nthreads) {
    if (!p || !dout || !do_stride || !dq || !dk || !dv) return -1;
    if (p->Hkv <= 0 || p->Hq % p->Hkv != 0 || p->D <= 0 || (p->causal && p->Nq > p->Nk)) return -1;
    pthread_once(&g_decode_once, fill_decode_tables);
    const int64_t nq = p->B * p->Hq * p->Nq, nk = p->B * p->Hkv * p->Nk;
    double* stats = (double*)malloc(sizeof(double) * 3 * (size_t)(nq > 0 ? nq : 1));
    if (!stats) return -2;
    oracle_bwd_job base;
    memset(&base, 0, sizeof base);
    base.p = p;
    base.dout = dout;
    base.do_stride[0] = do_stride[0];
    base.do_stride[1] = do_stride[1];
    base.do_stride[2] = do_stride[2];
    base.stats = stats;
    base.dq = dq;
    base.dk = dk;
    base.dv = dv;
    int rc = run_pass(bwd_query_worker, &base, nq, nthreads);
    if (rc == 0) rc = run_pass(bwd_key_worker, &base, nk, nthreads);
    free(stats);
    return rc;
}
