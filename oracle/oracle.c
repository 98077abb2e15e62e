/*
 * Plain CPU oracle for exact top-k / top-p candidate-set selection.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link,
 * load or call this file; only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg use it. It shares no code with the GPU path.
 *
 * What it computes. The Qrita summary (gist.science, "Qrita - Top-k y Top-p de
 * alto rendimiento..." / its Korean translation) states that the method
 * returns the full candidate set with the exact semantics of sort-based top-k
 * and top-p ("Declaración del Problema"; "Contribuciones Clave" 1), that the
 * pivot keeps exactly k elements at or above it ("Metodología" §2), that the
 * number of retained boundary duplicates is fixed deterministically (§2,
 * "Condición de Terminación"), and that the output matches sort-based
 * algorithms ("Resultados"). The oracle is therefore that sort-based
 * definition written out, not the pivot algorithm:
 *
 *   1. decode each logit exactly to double (bf16: bits << 16 as float;
 *      f16: IEEE binary16, sign * 2^(e-15) * (1 + f/1024), or
 *      sign * 2^-14 * f/1024 for subnormals);
 *      NaN and +inf are rejected, -inf is an ordinary value;
 *   2. order the indices by value descending, equal values by ascending
 *      index (-0.0 and +0.0 are equal values);
 *   3. top-k: K = V if k <= 0 or k >= V, else k; keep ranks 0..K-1;
 *   4. top-p (only when p < 1, p taken as the float the caller passes):
 *      p <= 0 keeps 1; otherwise with m the rank-0 value,
 *      e_r = exp(z_r - m) for r < K, S = sum e_r (sequential, rank order),
 *      cum_r = sum_{s<=r} e_s / S (sequential); keep 1 + min{r: cum_r >= p}
 *      ranks (K if no r qualifies); an all -inf row keeps 1;
 *   5. mask[i] = rank(i) < L; idx[j] = index of rank j, j < min(L, idx_cap);
 *      count = L.
 *
 * Boundary band (top-p rows): L_lo / L_hi are the cuts for p - 1e-5 and
 * p + 1e-5 (same rule, clamped to [1, K]). A row is a band row iff they
 * differ; there a GPU result must be a rank prefix with length in
 * [L_lo, L_hi]. For other rows band_lo = band_hi = L.
 *
 * Top-k before top-p, with top-p renormalised over the top-k set, is the
 * composition of the sort-based samplers Qrita replaces; the pages do not
 * spell it out.
 *
 * Sampling from the candidate set (oracle_sample; the step after the
 * selection, for which the pages motivate returning the whole candidate set,
 * "Declaración del Problema"): with the kept set of L tokens in rank order
 * and e_r = exp(z_r - m) for r < L, p_r = e_r / sum_{s<L} e_s (float64,
 * sequential sums), c_r = sum_{s<=r} p_s; for a uniform u in [0, 1) the
 * drawn token is the one of smallest rank r with c_r >= u (rank L-1 if no r
 * qualifies; rank 0 when every kept logit is -inf). Draws whose u lies
 * within 1e-6 of some c_r are band draws: the ranks for u - 1e-6 and
 * u + 1e-6 bound the answers a rounding-different computation may give.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    double v;
    int64_t i;
} oracle_item;

/* value descending, then index ascending: a total order, so the sorted
 * sequence is unique whatever sort routine produces it. */
static int cmp_desc(const void *pa, const void *pb) {
    const oracle_item *a = (const oracle_item *)pa;
    const oracle_item *b = (const oracle_item *)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->i < b->i) ? -1 : (a->i > b->i);
}

/* IEEE binary16 bits to double, from the format's definition: 1 sign bit,
 * 5 exponent bits (bias 15), 10 fraction bits; exponent 0 is subnormal,
 * exponent 31 is inf (fraction 0) or NaN. */
static double half_to_double(uint16_t h) {
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 31;
    const int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* 2^-14 * f / 2^10 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(1.0 + (double)f / 1024.0, e - 15);
    return sign ? -v : v;
}

static double decode(const void *logits, int dtype, int64_t off) {
    if (dtype == 0) {
        return (double)((const float *)logits)[off];
    }
    if (dtype == 2) {
        return half_to_double(((const uint16_t *)logits)[off]);
    }
    uint32_t u = ((uint32_t)((const uint16_t *)logits)[off]) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* smallest L in [1, K] with cum_{L-1} >= target, else K */
static int64_t prefix_cut(const double *cum, int64_t K, double target) {
    for (int64_t r = 0; r < K; ++r)
        if (cum[r] >= target) return r + 1;
    return K;
}

typedef struct {
    const void *logits;
    int64_t batch, vocab;
    int dtype;
    const int32_t *k;
    const float *p;
    uint8_t *mask;
    int32_t *idx;
    int64_t idx_cap;
    int32_t *count;
    int32_t *band_lo, *band_hi;
    int64_t row_begin, row_end;
    int status;
    int64_t bad_row, bad_col;
} oracle_job;

static void *run_rows(void *arg) {
    oracle_job *J = (oracle_job *)arg;
    const int64_t V = J->vocab;
    oracle_item *items = (oracle_item *)malloc((size_t)V * sizeof(oracle_item));
    double *cum = (double *)malloc((size_t)V * sizeof(double));
    double *e = (double *)malloc((size_t)V * sizeof(double));
    if (!items || !cum || !e) {
        J->status = 3;
        free(items); free(cum); free(e);
        return NULL;
    }
    for (int64_t b = J->row_begin; b < J->row_end; ++b) {
        /* 1. decode */
        for (int64_t i = 0; i < V; ++i) {
            double x = decode(J->logits, J->dtype, b * V + i);
            if (isnan(x) || x == INFINITY) {
                J->status = 2;
                J->bad_row = b;
                J->bad_col = i;
                goto done;
            }
            items[i].v = x;
            items[i].i = i;
        }
        /* 2. order */
        qsort(items, (size_t)V, sizeof(oracle_item), cmp_desc);
        /* 3. top-k */
        int64_t kb = J->k ? (int64_t)J->k[b] : 0;
        int64_t K = (kb <= 0 || kb >= V) ? V : kb;
        int64_t L = K, L_lo = K, L_hi = K;
        /* 4. top-p */
        double p = J->p ? (double)J->p[b] : 1.0;
        if (p < 1.0) {
            if (p <= 0.0) {
                L = L_lo = L_hi = 1;
            } else if (items[0].v == -INFINITY) {
                L = L_lo = L_hi = 1;
            } else {
                const double m = items[0].v;
                double S = 0.0;
                for (int64_t r = 0; r < K; ++r) {
                    e[r] = exp(items[r].v - m);
                    S += e[r];
                }
                double c = 0.0;
                for (int64_t r = 0; r < K; ++r) {
                    c += e[r] / S;
                    cum[r] = c;
                }
                L = prefix_cut(cum, K, p);
                L_lo = prefix_cut(cum, K, p - 1e-5);
                L_hi = prefix_cut(cum, K, p + 1e-5);
            }
        }
        /* 5. outputs */
        if (J->mask) {
            uint8_t *mrow = J->mask + b * V;
            memset(mrow, 0, (size_t)V);
            for (int64_t r = 0; r < L; ++r) mrow[items[r].i] = 1;
        }
        if (J->idx) {
            int64_t n = L < J->idx_cap ? L : J->idx_cap;
            for (int64_t r = 0; r < n; ++r) J->idx[b * J->idx_cap + r] = (int32_t)items[r].i;
        }
        if (J->count) J->count[b] = (int32_t)L;
        if (J->band_lo) J->band_lo[b] = (int32_t)L_lo;
        if (J->band_hi) J->band_hi[b] = (int32_t)L_hi;
    }
done:
    free(items);
    free(cum);
    free(e);
    return NULL;
}

int oracle_hardware_threads(void);

typedef struct {
    oracle_job base;
    const double *u;
    int32_t *token, *rank, *tok_lo, *tok_hi;
    float *prob;  /* [batch][idx_cap] or NULL */
} oracle_sample_job;

/* smallest r < L with c[r] >= x, else L - 1 */
static int64_t draw_rank(const double *c, int64_t L, double x) {
    for (int64_t r = 0; r < L; ++r)
        if (c[r] >= x) return r;
    return L - 1;
}

static void *run_sample_rows(void *arg) {
    oracle_sample_job *S = (oracle_sample_job *)arg;
    oracle_job *J = &S->base;
    const int64_t V = J->vocab;
    oracle_item *items = (oracle_item *)malloc((size_t)V * sizeof(oracle_item));
    double *e = (double *)malloc((size_t)V * sizeof(double));
    double *c = (double *)malloc((size_t)V * sizeof(double));
    if (!items || !e || !c) {
        J->status = 3;
        free(items); free(e); free(c);
        return NULL;
    }
    for (int64_t b = J->row_begin; b < J->row_end; ++b) {
        for (int64_t i = 0; i < V; ++i) {
            double x = decode(J->logits, J->dtype, b * V + i);
            if (isnan(x) || x == INFINITY) {
                J->status = 2;
                J->bad_row = b;
                J->bad_col = i;
                goto done;
            }
            items[i].v = x;
            items[i].i = i;
        }
        qsort(items, (size_t)V, sizeof(oracle_item), cmp_desc);
        /* the kept set, exactly as in run_rows */
        int64_t kb = J->k ? (int64_t)J->k[b] : 0;
        int64_t K = (kb <= 0 || kb >= V) ? V : kb;
        int64_t L = K;
        double p = J->p ? (double)J->p[b] : 1.0;
        const double m = items[0].v;
        if (p < 1.0) {
            if (p <= 0.0 || m == -INFINITY) {
                L = 1;
            } else {
                double Sk = 0.0;
                for (int64_t r = 0; r < K; ++r) {
                    e[r] = exp(items[r].v - m);
                    Sk += e[r];
                }
                double cc = 0.0;
                for (int64_t r = 0; r < K; ++r) {
                    cc += e[r] / Sk;
                    c[r] = cc;
                }
                L = prefix_cut(c, K, p);
            }
        }
        /* renormalised over the kept set */
        int64_t r0 = 0, rlo = 0, rhi = 0;
        if (m != -INFINITY) {
            double Sl = 0.0;
            for (int64_t r = 0; r < L; ++r) {
                e[r] = exp(items[r].v - m);
                Sl += e[r];
            }
            double cc = 0.0;
            for (int64_t r = 0; r < L; ++r) {
                cc += e[r] / Sl;
                c[r] = cc;
            }
            const double u = S->u[b];
            r0 = draw_rank(c, L, u);
            rlo = draw_rank(c, L, u - 1e-6);
            rhi = draw_rank(c, L, u + 1e-6);
            if (S->prob) {
                const int64_t n = L < J->idx_cap ? L : J->idx_cap;
                for (int64_t r = 0; r < n; ++r) S->prob[b * J->idx_cap + r] = (float)(e[r] / Sl);
            }
        } else if (S->prob) {
            const int64_t n = L < J->idx_cap ? L : J->idx_cap;
            for (int64_t r = 0; r < n; ++r) S->prob[b * J->idx_cap + r] = 0.0f;
        }
        S->token[b] = (int32_t)items[r0].i;
        if (S->rank) S->rank[b] = (int32_t)r0;
        if (S->tok_lo) S->tok_lo[b] = (int32_t)rlo;
        if (S->tok_hi) S->tok_hi[b] = (int32_t)rhi;
        if (J->count) J->count[b] = (int32_t)L;
        if (J->idx) {
            const int64_t n = L < J->idx_cap ? L : J->idx_cap;
            for (int64_t r = 0; r < n; ++r) J->idx[b * J->idx_cap + r] = (int32_t)items[r].i;
        }
    }
done:
    free(items);
    free(e);
    free(c);
    return NULL;
}

/*
 * Draw one token per row from the kept set (see the header comment):
 * u [batch] uniforms in [0, 1); token [batch] the drawn vocabulary index;
 * rank [batch] its rank in the kept set (may be NULL);
 * tok_lo / tok_hi [batch] the band of ranks (may be NULL); count [batch] the
 * kept count; idx [batch][idx_cap] the kept indices in rank order and prob
 * [batch][idx_cap] their renormalised probabilities (each may be NULL).
 * Returns as oracle_select.
 */
int oracle_sample(const void *logits, int64_t batch, int64_t vocab, int dtype, const int32_t *k,
                  const float *p, const double *u, int32_t *token, int32_t *rank, int32_t *tok_lo, int32_t *tok_hi,
                  int32_t *count, int32_t *idx, float *prob, int64_t idx_cap, int nthreads,
                  int64_t *bad_row, int64_t *bad_col) {
    if (!logits || !u || !token || batch < 0 || vocab <= 0 || vocab > INT32_MAX ||
        (dtype < 0 || dtype > 2) || idx_cap < 0)
        return 1;
    if (batch == 0) return 0;
    if (nthreads <= 0) nthreads = oracle_hardware_threads();
    if (nthreads > batch) nthreads = (int)batch;
    oracle_sample_job *jobs = (oracle_sample_job *)calloc((size_t)nthreads, sizeof(oracle_sample_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs); free(th);
        return 3;
    }
    for (int t = 0; t < nthreads; ++t) {
        oracle_job *J = &jobs[t].base;
        J->logits = logits; J->batch = batch; J->vocab = vocab; J->dtype = dtype;
        J->k = k; J->p = p; J->idx = idx; J->idx_cap = idx_cap; J->count = count;
        J->row_begin = batch * t / nthreads;
        J->row_end = batch * (t + 1) / nthreads;
        J->bad_row = J->bad_col = -1;
        jobs[t].u = u; jobs[t].token = token; jobs[t].rank = rank; jobs[t].tok_lo = tok_lo; jobs[t].tok_hi = tok_hi;
        jobs[t].prob = prob;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, run_sample_rows, &jobs[t]);
    run_sample_rows(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    int status = 0;
    for (int t = 0; t < nthreads && status == 0; ++t) {
        if (jobs[t].base.status) {
            status = jobs[t].base.status;
            if (bad_row) *bad_row = jobs[t].base.bad_row;
            if (bad_col) *bad_col = jobs[t].base.bad_col;
        }
    }
    free(jobs);
    free(th);
    return status;
}

int oracle_hardware_threads(void) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

/*
 * Select over `batch` rows of `vocab` logits (dtype 0 = float32, 1 = bf16 bits,
 * 2 = IEEE binary16 bits).
 * k, p: per-row controls (either may be NULL: that control is off).
 * mask [batch][vocab] uint8, idx [batch][idx_cap] int32, count [batch],
 * band_lo / band_hi [batch]: outputs, each may be NULL.
 * nthreads <= 0 uses every online core; rows are split in contiguous blocks.
 * Returns 0 on success, 1 for bad arguments, 2 if a NaN or +inf logit was
 * found (its row/column in *bad_row / *bad_col), 3 on allocation failure.
 */
int oracle_select(const void *logits, int64_t batch, int64_t vocab, int dtype,
                  const int32_t *k, const float *p, uint8_t *mask, int32_t *idx,
                  int64_t idx_cap, int32_t *count, int32_t *band_lo, int32_t *band_hi,
                  int nthreads, int64_t *bad_row, int64_t *bad_col) {
    if (!logits || batch < 0 || vocab <= 0 || vocab > INT32_MAX || (dtype < 0 || dtype > 2) ||
        idx_cap < 0)
        return 1;
    if (batch == 0) return 0;
    if (nthreads <= 0) nthreads = oracle_hardware_threads();
    if (nthreads > batch) nthreads = (int)batch;
    oracle_job *jobs = (oracle_job *)calloc((size_t)nthreads, sizeof(oracle_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs); free(th);
        return 3;
    }
    for (int t = 0; t < nthreads; ++t) {
        oracle_job *J = &jobs[t];
        J->logits = logits; J->batch = batch; J->vocab = vocab; J->dtype = dtype;
        J->k = k; J->p = p; J->mask = mask; J->idx = idx; J->idx_cap = idx_cap;
        J->count = count; J->band_lo = band_lo; J->band_hi = band_hi;
        J->row_begin = batch * t / nthreads;
        J->row_end = batch * (t + 1) / nthreads;
        J->status = 0;
        J->bad_row = J->bad_col = -1;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, run_rows, &jobs[t]);
    run_rows(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    int status = 0;
    for (int t = 0; t < nthreads && status == 0; ++t) {
        if (jobs[t].status) {
            status = jobs[t].status;
            if (bad_row) *bad_row = jobs[t].bad_row;
            if (bad_col) *bad_col = jobs[t].bad_col;
        }
    }
    free(jobs);
    free(th);
    return status;
}
