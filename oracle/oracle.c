/*
 * oracle.c -- plain fp64 CPU reference for masked attention (forward and its
 * gradients), the KV-split merge and the tile classification of a mask.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  It shares no source with the GPU
 * library (no headers, helpers or tables): every definition below is written out
 * again from the pages.
 *
 * Sources (the pages this follows):
 *   [UA]  UltraAttn blog post ("UltraAttn: hierarchical context tiling"), 3 (Full /
 *         Causal / Empty blocks), 3.1 (Q split: outputs are independent),
 *         3.2 (KV split: keep a mergeable (max, normaliser, weighted sum) summary,
 *         merge by rescaling both to the common max), 3.3 (2-D block view).
 *   [MA]  MagiAttention v1.1.0 news, "Blackwell adaptation" list (flexible masks,
 *         block-sparse mask generation, CSR mask metadata).
 *   [FT]  FlashAttention-T post, FlashAttention lineage paragraph (tiling with an
 *         incremental softmax gives the exact softmax, so the plain two-pass
 *         softmax below is the definition the tiled kernel must reproduce).
 *   [MA2] MagiAttention v1.1.0 news: the kernels cover the forward and the backward
 *         pass of the same masked attention; the backward below is the plain
 *         derivative of the forward written out (chain rule through the softmax).
 *
 * Readings taken where the pages are silent (each is listed in the design notes):
 *   - overlapping slices: the mask is the union of the slices' pair sets;
 *   - a causal slice (q0,q1,k0,k1) admits (i,j) iff j - k1 <= i - q1
 *     (bottom-right aligned; equals j <= i when k1 == q1);
 *   - a row with no admitted key: O = 0, LSE = -inf (the merge identity);
 *   - LSE is the natural log-sum-exp of the scaled scores;
 *   - GQA: query head h reads key/value head h / (Hq/Hkv).
 *
 * Every function here is pinned by tests (brute force, closed forms, split/merge,
 * mask invariance, tile counts); none is "parity unpinned".
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t q0, q1, k0, k1, type; /* type 0 = full, 1 = causal */
} oracle_slice;

/* Input element idx of an array that holds bf16 bit patterns (bf16 != 0) or doubles. */
static double bf16_to_double(uint16_t b);
static inline double ld(const void *p, size_t idx, int bf16)
{
    return bf16 ? bf16_to_double(((const uint16_t *)p)[idx]) : ((const double *)p)[idx];
}

/* bf16 -> fp64, exact: a bf16 is the top half of an IEEE binary32. */
static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ---------------------------------------------------------------------------
 * Row key set U(i) as a sorted list of disjoint half-open intervals.
 * U(i) = union over slices s with q0 <= i < q1 of
 *        { j : k0 <= j < k1 and (full or j - k1 <= i - q1) }.
 * --------------------------------------------------------------------------- */
typedef struct {
    int64_t lo, hi;
} interval;

static int cmp_interval(const void *a, const void *b)
{
    const interval *x = (const interval *)a, *y = (const interval *)b;
    if (x->lo != y->lo) return x->lo < y->lo ? -1 : 1;
    if (x->hi != y->hi) return x->hi < y->hi ? -1 : 1;
    return 0;
}

/* Writes at most n_slices intervals into out; returns how many after merging. */
static int row_key_set(const oracle_slice *s, int n_slices, int64_t i, interval *out)
{
    int m = 0;
    for (int t = 0; t < n_slices; ++t) {
        if (i < s[t].q0 || i >= s[t].q1) continue;
        int64_t lo = s[t].k0, hi = s[t].k1;
        if (s[t].type == 1) {
            int64_t last = i - (int64_t)s[t].q1 + (int64_t)s[t].k1; /* largest admitted j */
            if (hi > last + 1) hi = last + 1;
        }
        if (lo < hi) {
            out[m].lo = lo;
            out[m].hi = hi;
            ++m;
        }
    }
    if (m <= 1) return m;
    qsort(out, (size_t)m, sizeof(interval), cmp_interval);
    int w = 0;
    for (int t = 1; t < m; ++t) {
        if (out[t].lo <= out[w].hi) { /* overlapping or touching: a set union */
            if (out[t].hi > out[w].hi) out[w].hi = out[t].hi;
        } else {
            out[++w] = out[t];
        }
    }
    return w + 1;
}

/* Number of admitted (i, j) pairs summed over rows i in [0, sq). */
int64_t oracle_pair_count(const oracle_slice *s, int32_t n_slices, int32_t sq)
{
    interval *buf = (interval *)malloc(sizeof(interval) * (size_t)(n_slices > 0 ? n_slices : 1));
    int64_t total = 0;
    for (int64_t i = 0; i < sq; ++i) {
        int m = row_key_set(s, n_slices, i, buf);
        for (int t = 0; t < m; ++t) total += buf[t].hi - buf[t].lo;
    }
    free(buf);
    return total;
}

/* Row key set exported for tests: returns the interval count, fills lo/hi. */
int32_t oracle_row_key_set(const oracle_slice *s, int32_t n_slices, int64_t i,
                           int64_t *lo, int64_t *hi)
{
    interval *buf = (interval *)malloc(sizeof(interval) * (size_t)(n_slices > 0 ? n_slices : 1));
    int m = row_key_set(s, n_slices, i, buf);
    for (int t = 0; t < m; ++t) {
        lo[t] = buf[t].lo;
        hi[t] = buf[t].hi;
    }
    free(buf);
    return m;
}

/* ---------------------------------------------------------------------------
 * Tile classification ([UA] 3, [MA] CSR metadata).  The (Bq x Bk) tile at
 * (qt, kt) is Full when every in-range pair is admitted, Empty when none is,
 * Causal ("partial") otherwise.  Counts are taken row by row from U(i): a
 * different route from any geometric per-slice compiler.
 * Output: row_ptr[n_qt + 1], col[nnz] ascending per row, tag[nnz] (1 full,
 * 2 partial).  Returns 0 on success, -1 when cap is too small (nnz still set).
 * --------------------------------------------------------------------------- */
int32_t oracle_tile_csr(const oracle_slice *s, int32_t n_slices, int32_t sq, int32_t sk,
                        int32_t bq, int32_t bk, int32_t *row_ptr, int32_t *col,
                        uint8_t *tag, int64_t cap, int64_t *nnz_out)
{
    int64_t n_qt = (sq + bq - 1) / bq, n_kt = (sk + bk - 1) / bk;
    int64_t *count = (int64_t *)calloc((size_t)(n_kt > 0 ? n_kt : 1), sizeof(int64_t));
    interval *buf = (interval *)malloc(sizeof(interval) * (size_t)(n_slices > 0 ? n_slices : 1));
    int64_t nnz = 0;
    int32_t rc = 0;
    row_ptr[0] = 0;
    for (int64_t qt = 0; qt < n_qt; ++qt) {
        int64_t r0 = qt * bq, r1 = r0 + bq < sq ? r0 + bq : sq;
        memset(count, 0, sizeof(int64_t) * (size_t)n_kt);
        for (int64_t i = r0; i < r1; ++i) {
            int m = row_key_set(s, n_slices, i, buf);
            for (int t = 0; t < m; ++t) {
                int64_t lo = buf[t].lo < 0 ? 0 : buf[t].lo;
                int64_t hi = buf[t].hi > sk ? sk : buf[t].hi;
                /* add the overlap of [lo, hi) with each key tile */
                for (int64_t j = lo; j < hi;) {
                    int64_t kt = j / bk, tile_end = (kt + 1) * bk;
                    int64_t e = hi < tile_end ? hi : tile_end;
                    count[kt] += e - j;
                    j = e;
                }
            }
        }
        for (int64_t kt = 0; kt < n_kt; ++kt) {
            if (count[kt] == 0) continue;
            int64_t c0 = kt * bk, c1 = c0 + bk < sk ? c0 + bk : sk;
            int64_t area = (r1 - r0) * (c1 - c0);
            if (nnz < cap) {
                col[nnz] = (int32_t)kt;
                tag[nnz] = (uint8_t)(count[kt] == area ? 1 : 2);
            } else {
                rc = -1;
            }
            ++nnz;
        }
        row_ptr[qt + 1] = (int32_t)nnz;
    }
    free(buf);
    free(count);
    *nnz_out = nnz;
    return rc;
}

/* ---------------------------------------------------------------------------
 * Attention forward, plain fp64, two passes, no tiling.
 * Layouts (contiguous, row-major): q [sq, hq, d], k and v [sk, hkv, d] as bf16
 * bit patterns.  For each requested (h, i):
 *   s_j = scale * sum_t q[i,h,t] k[j,g,t]   for j in U(i), g = h / (hq/hkv)
 *   U(i) empty -> O = 0, LSE = -inf
 *   else M = max s_j, LSE = M + ln sum_j exp(s_j - M),
 *        O = sum_j exp(s_j - LSE) v[j,g,:].
 * Rows are given as (h, i) pairs in rows[2*r], rows[2*r+1]; when rows is NULL
 * every (h, i) is computed and o is [sq, hq, d], lse [hq, sq].  Otherwise o is
 * [n_rows, d] and lse [n_rows].
 * --------------------------------------------------------------------------- */
typedef struct {
    const void *q, *k, *v;
    int bf16;   /* inputs are bf16 bit patterns (else doubles) */
    int32_t sq, sk, hq, hkv, d;
    const oracle_slice *s;
    int32_t n_slices;
    double scale;
    const int64_t *rows;
    int64_t n_rows;
    double *o, *lse;
    int32_t n_threads, tid;
} attn_job;

static void attn_one_row(const attn_job *J, int64_t h, int64_t i, double *o_row, double *lse_out,
                         interval *ivs, double *scores)
{
    const int d = J->d;
    const int64_t g = h / (J->hq / J->hkv);
    const int m = row_key_set(J->s, J->n_slices, i, ivs);
    int64_t n_keys = 0;
    for (int t = 0; t < m; ++t) {
        int64_t lo = ivs[t].lo < 0 ? 0 : ivs[t].lo, hi = ivs[t].hi > J->sk ? J->sk : ivs[t].hi;
        if (lo < hi) n_keys += hi - lo;
    }
    for (int t = 0; t < d; ++t) o_row[t] = 0.0;
    if (n_keys == 0) {
        *lse_out = -INFINITY;
        return;
    }
    const size_t qi = ((size_t)i * J->hq + (size_t)h) * d;
    /* pass 1: scores and their maximum */
    double mx = -INFINITY;
    int64_t c = 0;
    for (int t = 0; t < m; ++t) {
        int64_t lo = ivs[t].lo < 0 ? 0 : ivs[t].lo, hi = ivs[t].hi > J->sk ? J->sk : ivs[t].hi;
        for (int64_t j = lo; j < hi; ++j) {
            const size_t kj = ((size_t)j * J->hkv + (size_t)g) * d;
            double acc = 0.0;
            for (int e = 0; e < d; ++e) acc += ld(J->q, qi + e, J->bf16) * ld(J->k, kj + e, J->bf16);
            scores[c] = J->scale * acc;
            if (scores[c] > mx) mx = scores[c];
            ++c;
        }
    }
    /* pass 2: normaliser, log-sum-exp, weighted sum of values */
    double sum = 0.0;
    for (int64_t t = 0; t < n_keys; ++t) sum += exp(scores[t] - mx);
    const double lse = mx + log(sum);
    c = 0;
    for (int t = 0; t < m; ++t) {
        int64_t lo = ivs[t].lo < 0 ? 0 : ivs[t].lo, hi = ivs[t].hi > J->sk ? J->sk : ivs[t].hi;
        for (int64_t j = lo; j < hi; ++j) {
            const double p = exp(scores[c] - lse);
            const size_t vj = ((size_t)j * J->hkv + (size_t)g) * d;
            for (int e = 0; e < d; ++e) o_row[e] += p * ld(J->v, vj + e, J->bf16);
            ++c;
        }
    }
    *lse_out = lse;
}

static void *attn_worker(void *arg)
{
    const attn_job *J = (const attn_job *)arg;
    interval *ivs = (interval *)malloc(sizeof(interval) * (size_t)(J->n_slices > 0 ? J->n_slices : 1));
    double *scores = (double *)malloc(sizeof(double) * (size_t)(J->sk > 0 ? J->sk : 1));
    const int64_t total = J->rows ? J->n_rows : (int64_t)J->hq * J->sq;
    for (int64_t r = J->tid; r < total; r += J->n_threads) {
        int64_t h, i;
        double *o_row, *lse_ptr;
        if (J->rows) {
            h = J->rows[2 * r];
            i = J->rows[2 * r + 1];
            o_row = J->o + (size_t)r * J->d;
            lse_ptr = J->lse + r;
        } else {
            h = r / J->sq;
            i = r % J->sq;
            o_row = J->o + ((size_t)i * J->hq + (size_t)h) * J->d;
            lse_ptr = J->lse + (size_t)h * J->sq + (size_t)i;
        }
        attn_one_row(J, h, i, o_row, lse_ptr, ivs, scores);
    }
    free(scores);
    free(ivs);
    return NULL;
}

static int32_t attn_fwd_any(const void *q, const void *k, const void *v, int bf16, int32_t sq, int32_t sk,
                            int32_t hq, int32_t hkv, int32_t d, const oracle_slice *slices, int32_t n_slices,
                            double scale, const int64_t *rows, int64_t n_rows, double *o, double *lse,
                            int32_t n_threads)
{
    if (hkv <= 0 || hq % hkv != 0 || d <= 0) return -1;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    pthread_t th[256];
    attn_job jobs[256];
    for (int t = 0; t < n_threads; ++t) {
        attn_job J = {q, k, v, bf16, sq, sk, hq, hkv, d, slices, n_slices, scale, rows, n_rows, o, lse,
                      n_threads, t};
        jobs[t] = J;
    }
    for (int t = 1; t < n_threads; ++t) pthread_create(&th[t], NULL, attn_worker, &jobs[t]);
    attn_worker(&jobs[0]);
    for (int t = 1; t < n_threads; ++t) pthread_join(th[t], NULL);
    return 0;
}

/* Inputs as bf16 bit patterns (the kernels' inputs, decoded exactly). */
int32_t oracle_attn_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, int32_t sq,
                        int32_t sk, int32_t hq, int32_t hkv, int32_t d, const oracle_slice *slices,
                        int32_t n_slices, double scale, const int64_t *rows, int64_t n_rows,
                        double *o, double *lse, int32_t n_threads)
{
    return attn_fwd_any(q, k, v, 1, sq, sk, hq, hkv, d, slices, n_slices, scale, rows, n_rows, o, lse,
                        n_threads);
}

/* Inputs as doubles (finite-difference checks of the backward perturb them). */
int32_t oracle_attn_fwd_f64(const double *q, const double *k, const double *v, int32_t sq, int32_t sk,
                            int32_t hq, int32_t hkv, int32_t d, const oracle_slice *slices,
                            int32_t n_slices, double scale, double *o, double *lse, int32_t n_threads)
{
    return attn_fwd_any(q, k, v, 0, sq, sk, hq, hkv, d, slices, n_slices, scale, NULL, 0, o, lse,
                        n_threads);
}

/* ---------------------------------------------------------------------------
 * Attention backward ([MA2]: gradients of the same masked attention), plain
 * fp64: the derivative of the forward above, term by term.  With
 * P_ij = exp(s_ij - LSE_i) for j in U(i) (0 elsewhere) and O_i = sum_j P_ij v_j,
 * an upstream gradient dO gives
 *   D_i   = sum_t dO_it O_it                  (= sum_j P_ij dP_ij)
 *   dP_ij = dO_i . v_j
 *   dS_ij = P_ij (dP_ij - D_i)                 (softmax Jacobian)
 *   dQ_i  = scale sum_j dS_ij k_j
 *   dK_j  = scale sum_(h in group) sum_i dS_ij q_i
 *   dV_j  = sum_(h in group) sum_i P_ij dO_i
 * where O and LSE are recomputed here in fp64 (not taken from a kernel).
 * Layouts as the forward; dq [sq, hq, d], dk and dv [sk, hkv, d] fp64, zeroed
 * here.  Threads take key/value head groups, so dk/dv rows have one writer.
 * --------------------------------------------------------------------------- */
typedef struct {
    const void *q, *k, *v, *dout;
    int bf16;
    int32_t sq, sk, hq, hkv, d;
    const oracle_slice *s;
    int32_t n_slices;
    double scale;
    double *dq, *dk, *dv;
    int32_t n_threads, tid;
} bwd_job;

/* One row (h, i): its admitted keys (keys[0 .. n)), P_ij in p[], and D_i.  Returns n;
 * 0 when U(i) is empty (then every gradient term of the row is 0). */
static int64_t bwd_row(const bwd_job *J, int64_t h, int64_t i, interval *ivs, int64_t *keys, double *p,
                       double *o_row, double *D_out)
{
    const int d = J->d;
    const int64_t g = h / (J->hq / J->hkv);
    const int m = row_key_set(J->s, J->n_slices, i, ivs);
    int64_t n_keys = 0;
    for (int t = 0; t < m; ++t) {
        int64_t lo = ivs[t].lo < 0 ? 0 : ivs[t].lo, hi = ivs[t].hi > J->sk ? J->sk : ivs[t].hi;
        for (int64_t j = lo; j < hi; ++j) keys[n_keys++] = j;
    }
    if (n_keys == 0) return 0;
    const size_t qi = ((size_t)i * J->hq + (size_t)h) * d;
    double mx = -INFINITY;
    for (int64_t c = 0; c < n_keys; ++c) {
        const size_t kj = ((size_t)keys[c] * J->hkv + (size_t)g) * d;
        double acc = 0.0;
        for (int e = 0; e < d; ++e) acc += ld(J->q, qi + e, J->bf16) * ld(J->k, kj + e, J->bf16);
        p[c] = J->scale * acc;
        if (p[c] > mx) mx = p[c];
    }
    double sum = 0.0;
    for (int64_t c = 0; c < n_keys; ++c) sum += exp(p[c] - mx);
    const double lse = mx + log(sum);
    /* P (in place of the scores), O and D */
    for (int e = 0; e < d; ++e) o_row[e] = 0.0;
    for (int64_t c = 0; c < n_keys; ++c) {
        p[c] = exp(p[c] - lse);
        const size_t vj = ((size_t)keys[c] * J->hkv + (size_t)g) * d;
        for (int e = 0; e < d; ++e) o_row[e] += p[c] * ld(J->v, vj + e, J->bf16);
    }
    double D = 0.0;
    for (int e = 0; e < d; ++e) D += ld(J->dout, qi + e, J->bf16) * o_row[e];
    *D_out = D;
    return n_keys;
}

/* dS_ij = P_ij (dO_i . v_j - D_i) for row (h, i) and key j. */
static double bwd_ds(const bwd_job *J, int64_t h, int64_t i, int64_t j, double p, double D)
{
    const int d = J->d;
    const int64_t g = h / (J->hq / J->hkv);
    const size_t qi = ((size_t)i * J->hq + (size_t)h) * d, kv = ((size_t)j * J->hkv + (size_t)g) * d;
    double dp = 0.0;
    for (int e = 0; e < d; ++e) dp += ld(J->dout, qi + e, J->bf16) * ld(J->v, kv + e, J->bf16);
    return p * (dp - D);
}

static void *bwd_worker(void *arg)
{
    const bwd_job *J = (const bwd_job *)arg;
    const int d = J->d, group = J->hq / J->hkv;
    interval *ivs = (interval *)malloc(sizeof(interval) * (size_t)(J->n_slices > 0 ? J->n_slices : 1));
    double *p = (double *)malloc(sizeof(double) * (size_t)(J->sk > 0 ? J->sk : 1));
    int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)(J->sk > 0 ? J->sk : 1));
    double *o_row = (double *)malloc(sizeof(double) * (size_t)d);
    for (int64_t g = J->tid; g < J->hkv; g += J->n_threads) {
        for (int64_t h = g * group; h < (g + 1) * group; ++h) {
            for (int64_t i = 0; i < J->sq; ++i) {
                double D = 0.0;
                const int64_t n_keys = bwd_row(J, h, i, ivs, keys, p, o_row, &D);
                const size_t qi = ((size_t)i * J->hq + (size_t)h) * d;
                for (int64_t c = 0; c < n_keys; ++c) {
                    const size_t kv = ((size_t)keys[c] * J->hkv + (size_t)g) * d;
                    const double ds = bwd_ds(J, h, i, keys[c], p[c], D);
                    for (int e = 0; e < d; ++e) {
                        J->dq[qi + e] += J->scale * ds * ld(J->k, kv + e, J->bf16);
                        J->dk[kv + e] += J->scale * ds * ld(J->q, qi + e, J->bf16);
                        J->dv[kv + e] += p[c] * ld(J->dout, qi + e, J->bf16);
                    }
                }
            }
        }
    }
    free(o_row);
    free(keys);
    free(p);
    free(ivs);
    return NULL;
}

static int32_t attn_bwd_any(const void *q, const void *k, const void *v, const void *dout, int bf16, int32_t sq,
                            int32_t sk, int32_t hq, int32_t hkv, int32_t d, const oracle_slice *slices,
                            int32_t n_slices, double scale, double *dq, double *dk, double *dv, int32_t n_threads)
{
    if (hkv <= 0 || hq % hkv != 0 || d <= 0) return -1;
    memset(dq, 0, sizeof(double) * (size_t)sq * hq * d);
    memset(dk, 0, sizeof(double) * (size_t)sk * hkv * d);
    memset(dv, 0, sizeof(double) * (size_t)sk * hkv * d);
    if (n_threads < 1) n_threads = 1;
    if (n_threads > hkv) n_threads = hkv;
    if (n_threads > 256) n_threads = 256;
    pthread_t th[256];
    bwd_job jobs[256];
    for (int t = 0; t < n_threads; ++t) {
        bwd_job J = {q, k, v, dout, bf16, sq, sk, hq, hkv, d, slices, n_slices, scale, dq, dk, dv, n_threads, t};
        jobs[t] = J;
    }
    for (int t = 1; t < n_threads; ++t) pthread_create(&th[t], NULL, bwd_worker, &jobs[t]);
    bwd_worker(&jobs[0]);
    for (int t = 1; t < n_threads; ++t) pthread_join(th[t], NULL);
    return 0;
}

int32_t oracle_attn_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                        int32_t sq, int32_t sk, int32_t hq, int32_t hkv, int32_t d, const oracle_slice *slices,
                        int32_t n_slices, double scale, double *dq, double *dk, double *dv, int32_t n_threads)
{
    return attn_bwd_any(q, k, v, dout, 1, sq, sk, hq, hkv, d, slices, n_slices, scale, dq, dk, dv, n_threads);
}

int32_t oracle_attn_bwd_f64(const double *q, const double *k, const double *v, const double *dout, int32_t sq,
                            int32_t sk, int32_t hq, int32_t hkv, int32_t d, const oracle_slice *slices,
                            int32_t n_slices, double scale, double *dq, double *dk, double *dv)
{
    return attn_bwd_any(q, k, v, dout, 0, sq, sk, hq, hkv, d, slices, n_slices, scale, dq, dk, dv, 1);
}

/* ---------------------------------------------------------------------------
 * The same gradients at sampled outputs, for problems too large for the full
 * pass: dQ rows at (h, i) pairs rows[2r], rows[2r+1] -> dq_rows [n_rows, d], and
 * dK, dV rows at (g, j) pairs keys[2t], keys[2t+1] -> dk_rows, dv_rows [n_keys, d].
 * A sampled key visits every row i of every head of its group whose key set holds
 * j, recomputing that row's P and D; the terms are summed in the full pass's order.
 * --------------------------------------------------------------------------- */
typedef struct {
    bwd_job base;
    const int64_t *rows, *keys;
    int64_t n_rows, n_keys;
    double *dq_rows, *dk_rows, *dv_rows;
} bwd_sample_job;

static void *bwd_sample_worker(void *arg)
{
    const bwd_sample_job *S = (const bwd_sample_job *)arg;
    const bwd_job *J = &S->base;
    const int d = J->d, group = J->hq / J->hkv;
    interval *ivs = (interval *)malloc(sizeof(interval) * (size_t)(J->n_slices > 0 ? J->n_slices : 1));
    double *p = (double *)malloc(sizeof(double) * (size_t)(J->sk > 0 ? J->sk : 1));
    int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)(J->sk > 0 ? J->sk : 1));
    double *o_row = (double *)malloc(sizeof(double) * (size_t)d);
    for (int64_t r = J->tid; r < S->n_rows + S->n_keys; r += J->n_threads) {
        if (r < S->n_rows) {
            const int64_t h = S->rows[2 * r], i = S->rows[2 * r + 1], g = h / group;
            double *out = S->dq_rows + (size_t)r * d;
            for (int e = 0; e < d; ++e) out[e] = 0.0;
            double D = 0.0;
            const int64_t n = bwd_row(J, h, i, ivs, keys, p, o_row, &D);
            for (int64_t c = 0; c < n; ++c) {
                const size_t kv = ((size_t)keys[c] * J->hkv + (size_t)g) * d;
                const double ds = bwd_ds(J, h, i, keys[c], p[c], D);
                for (int e = 0; e < d; ++e) out[e] += J->scale * ds * ld(J->k, kv + e, J->bf16);
            }
        } else {
            const int64_t t = r - S->n_rows, g = S->keys[2 * t], j = S->keys[2 * t + 1];
            double *ok = S->dk_rows + (size_t)t * d, *ov = S->dv_rows + (size_t)t * d;
            for (int e = 0; e < d; ++e) ok[e] = ov[e] = 0.0;
            for (int64_t h = g * group; h < (g + 1) * group; ++h)
                for (int64_t i = 0; i < J->sq; ++i) {
                    /* is j in U(i)? */
                    const int m = row_key_set(J->s, J->n_slices, i, ivs);
                    int in = 0;
                    for (int u = 0; u < m && !in; ++u) in = j >= ivs[u].lo && j < ivs[u].hi;
                    if (!in) continue;
                    double D = 0.0;
                    const int64_t n = bwd_row(J, h, i, ivs, keys, p, o_row, &D);
                    int64_t c = 0;
                    while (c < n && keys[c] != j) ++c;
                    if (c == n) continue;
                    const size_t qi = ((size_t)i * J->hq + (size_t)h) * d;
                    const double ds = bwd_ds(J, h, i, j, p[c], D);
                    for (int e = 0; e < d; ++e) {
                        ok[e] += J->scale * ds * ld(J->q, qi + e, J->bf16);
                        ov[e] += p[c] * ld(J->dout, qi + e, J->bf16);
                    }
                }
        }
    }
    free(o_row);
    free(keys);
    free(p);
    free(ivs);
    return NULL;
}

int32_t oracle_attn_bwd_sampled(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                                int32_t sq, int32_t sk, int32_t hq, int32_t hkv, int32_t d,
                                const oracle_slice *slices, int32_t n_slices, double scale, const int64_t *rows,
                                int64_t n_rows, double *dq_rows, const int64_t *keys, int64_t n_keys,
                                double *dk_rows, double *dv_rows, int32_t n_threads)
{
    if (hkv <= 0 || hq % hkv != 0 || d <= 0) return -1;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    pthread_t th[256];
    bwd_sample_job jobs[256];
    for (int t = 0; t < n_threads; ++t) {
        bwd_job J = {q, k, v, dout, 1, sq, sk, hq, hkv, d, slices, n_slices, scale, NULL, NULL, NULL, n_threads, t};
        bwd_sample_job S = {J, rows, keys, n_rows, n_keys, dq_rows, dk_rows, dv_rows};
        jobs[t] = S;
    }
    for (int t = 1; t < n_threads; ++t) pthread_create(&th[t], NULL, bwd_sample_worker, &jobs[t]);
    bwd_sample_worker(&jobs[0]);
    for (int t = 1; t < n_threads; ++t) pthread_join(th[t], NULL);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Merge of KV-split partials ([UA] 3.2).  Each partial k carries (LSE_k, O_k)
 * with O_k already normalised by its own denominator.  With M the largest
 * finite LSE_k:
 *   LSE = M + ln sum_k exp(LSE_k - M),  O = sum_k exp(LSE_k - LSE) O_k.
 * All partials at -inf -> O = 0, LSE = -inf (a partial at -inf is the identity).
 * o_parts is [n, R, d] and lse_parts [n, R] (fp64); o is [R, d], lse [R].
 * --------------------------------------------------------------------------- */
void oracle_merge(const double *o_parts, const double *lse_parts, int32_t n, int64_t n_rows,
                  int32_t d, double *o, double *lse)
{
    for (int64_t r = 0; r < n_rows; ++r) {
        double mx = -INFINITY;
        for (int32_t t = 0; t < n; ++t) {
            double x = lse_parts[(size_t)t * n_rows + r];
            if (x > mx) mx = x;
        }
        double *orow = o + (size_t)r * d;
        for (int e = 0; e < d; ++e) orow[e] = 0.0;
        if (mx == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double sum = 0.0;
        for (int32_t t = 0; t < n; ++t) sum += exp(lse_parts[(size_t)t * n_rows + r] - mx);
        const double total = mx + log(sum);
        for (int32_t t = 0; t < n; ++t) {
            const double w = exp(lse_parts[(size_t)t * n_rows + r] - total);
            const double *src = o_parts + ((size_t)t * n_rows + r) * d;
            for (int e = 0; e < d; ++e) orow[e] += w * src[e];
        }
        lse[r] = total;
    }
}
