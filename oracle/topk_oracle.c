/*
 * CPU oracle for the index-only TopK selector.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the tests, the package smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header or table
 * with the GPU library.
 *
 * Source: the web article "How to Use FlagOS's New Triton-TLE Language to
 * Build a TopK Selector Faster Than FlashInfer" (below: the TopK article).
 *
 *  - Section 01: the selector returns, per query row of indexer logits, the
 *    indices of the k largest logits; values are not returned and the output
 *    need not be sorted.
 *  - Section 02, the radix_topk pseudocode: first every element strictly above
 *    the k-th largest value T is taken, then elements equal to T are taken in
 *    scan order until k are held, i.e. ties at T go to the lowest index.
 *  - Section 5 (output flush): -1 is the value written for an output slot that
 *    holds no index.
 *
 * This oracle is the plain definition, not the radix method: for each row it
 * sorts the valid positions by (value descending, index ascending) with IEEE
 * float comparisons and keeps the first min(k, L) of them.  Readings where
 * the article is silent:
 *  - valid length L = lengths[r] clamped to [0, n] (all n when lengths is
 *    NULL); positions >= L are never returned;
 *  - when L < k the row holds all of 0..L-1 followed by k-L entries of -1;
 *  - -0.0 and +0.0 compare equal, so they tie (lowest index first);
 *    infinities and subnormals are ordinary values (build without fast-math,
 *    so subnormals are not flushed);
 *  - NaN is outside the contract: a NaN among the valid positions makes the
 *    oracle return ORACLE_ERR_NAN.
 * Each output row is written in (value desc, index asc) order; callers that
 * compare against the unsorted GPU path compare sorted index sets.
 *
 * Ordered output (oracle_topk_sorted): section 02's radix_topk has a
 * need_sorted option that sorts the collected output in descending order.
 * The order among equal values is not stated; the reading taken is the
 * same rule that decides which of them are selected: lowest index first.
 * The values returned are the logits at the selected positions, bit for bit
 * (so -0.0 stays -0.0), and -INFINITY beside each -1.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NAN 2
#define ORACLE_ERR_NOMEM 3

/* Each element carries its value and index, so the comparator needs no
 * outside state and several threads may run the oracle at once. */
typedef struct {
    float v;
    int32_t i;
} oracle_elem;

/* Total order: larger value first; equal values (including -0 vs +0) by
 * smaller index first. */
static int oracle_cmp(const void* pa, const void* pb) {
    const oracle_elem* a = (const oracle_elem*)pa;
    const oracle_elem* b = (const oracle_elem*)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    /* a->v == b->v here (NaN was rejected before sorting) */
    if (a->i < b->i) return -1;
    if (a->i > b->i) return 1;
    return 0;
}

static int oracle_row(const float* x, int32_t n, int32_t L, int32_t k, int32_t* out, oracle_elem* buf) {
    if (L < 0) L = 0;
    if (L > n) L = n;
    /* Elements enter the sort in descending index order, so the result does
     * not lean on the sort being stable: the index tie-break must come from
     * the comparator. */
    for (int32_t i = 0; i < L; ++i) {
        int32_t j = L - 1 - i;
        if (x[j] != x[j]) return ORACLE_ERR_NAN;
        buf[i].v = x[j];
        buf[i].i = j;
    }
    qsort(buf, (size_t)L, sizeof(oracle_elem), oracle_cmp);
    int32_t take = L < k ? L : k;
    for (int32_t j = 0; j < take; ++j) out[j] = buf[j].i;
    for (int32_t j = take; j < k; ++j) out[j] = -1;
    return ORACLE_OK;
}

/* logits: [rows, n] row-major float32 (host memory); lengths: [rows] or NULL;
 * out: [rows, k] int32 (host memory).  Returns ORACLE_OK or an error code. */
int oracle_topk(const float* logits, int32_t rows, int32_t n, const int32_t* lengths, int32_t k,
                int32_t* out) {
    if (rows < 0 || n < 1 || k < 1 || k > n) return ORACLE_ERR_ARG;
    if (rows == 0) return ORACLE_OK;
    if (!logits || !out) return ORACLE_ERR_ARG;
    oracle_elem* buf = (oracle_elem*)malloc(sizeof(oracle_elem) * (size_t)n);
    if (!buf) return ORACLE_ERR_NOMEM;
    int rc = ORACLE_OK;
    for (int32_t r = 0; r < rows && rc == ORACLE_OK; ++r) {
        int32_t L = lengths ? lengths[r] : n;
        rc = oracle_row(logits + (size_t)r * (size_t)n, n, L, k, out + (size_t)r * (size_t)k, buf);
    }
    free(buf);
    return rc;
}

/* The k-th largest valid value of one row (counted with multiplicity), i.e.
 * the threshold T of the article's radix_topk.  Requires 1 <= k <= L. */
int oracle_kth_largest(const float* x, int32_t n, int32_t L, int32_t k, float* kth) {
    if (L > n) L = n;
    if (n < 1 || k < 1 || L < k || !x || !kth) return ORACLE_ERR_ARG;
    oracle_elem* buf = (oracle_elem*)malloc(sizeof(oracle_elem) * (size_t)L);
    if (!buf) return ORACLE_ERR_NOMEM;
    for (int32_t i = 0; i < L; ++i) {
        int32_t j = L - 1 - i;
        if (x[j] != x[j]) {
            free(buf);
            return ORACLE_ERR_NAN;
        }
        buf[i].v = x[j];
        buf[i].i = j;
    }
    qsort(buf, (size_t)L, sizeof(oracle_elem), oracle_cmp);
    *kth = buf[k - 1].v;
    free(buf);
    return ORACLE_OK;
}

/* oracle_topk, each row in (value desc, index asc) order, plus the selected
 * values.  out_val: [rows, k] float32 (host memory); out_val[j] is the logit
 * at out_idx[j], or -INFINITY where out_idx[j] is -1. */
int oracle_topk_sorted(const float* logits, int32_t rows, int32_t n, const int32_t* lengths, int32_t k,
                       int32_t* out_idx, float* out_val) {
    if (!out_val && rows > 0) return ORACLE_ERR_ARG;
    int rc = oracle_topk(logits, rows, n, lengths, k, out_idx);
    if (rc != ORACLE_OK) return rc;
    for (int32_t r = 0; r < rows; ++r) {
        const float* x = logits + (size_t)r * (size_t)n;
        const int32_t* o = out_idx + (size_t)r * (size_t)k;
        float* v = out_val + (size_t)r * (size_t)k;
        for (int32_t j = 0; j < k; ++j) v[j] = o[j] >= 0 ? x[o[j]] : -INFINITY;
    }
    return ORACLE_OK;
}

/*
 * The indexer's logits: the TopK article, section 01, lists three DSA steps,
 * the first being logits of the current query against every historical
 * token; the article gives no formula.  Reading taken (the form the
 * selector's causal workload mirrors: a weighted sum of eight ReLU terms):
 * H indexer heads share one key per token, and
 *
 *     logits[r][t] = sum_h w[r][h] * max(0, sum_i q[r][h][i] * K[t][i])
 *
 * with q [rows, H, d], K [n, d] per row (kstride elements between the keys
 * of consecutive rows; 0 when every row uses the same keys) and w [rows, H].
 * The inputs arrive as floats (bf16 values widened exactly); the sums are
 * taken in double precision, in index order.  absterm[r][t] (optional)
 * receives sum_h |w[r][h]| * sum_i |q[r][h][i] * K[t][i]|, the scale of the
 * rounding error of any float32 evaluation of the same sums.
 */
int oracle_indexer_logits(const float* q, const float* kc, const float* w, int32_t rows, int32_t n, int32_t H,
                          int32_t d, int64_t kstride, double* logits, double* absterm) {
    if (rows < 0 || n < 0 || H < 1 || d < 1 || kstride < 0) return ORACLE_ERR_ARG;
    if (rows == 0 || n == 0) return ORACLE_OK;
    if (!q || !kc || !w || !logits) return ORACLE_ERR_ARG;
    for (int32_t r = 0; r < rows; ++r) {
        const float* K = kc + (size_t)r * (size_t)kstride;
        for (int32_t t = 0; t < n; ++t) {
            const float* kt = K + (size_t)t * (size_t)d;
            double acc = 0.0, mag = 0.0;
            for (int32_t h = 0; h < H; ++h) {
                const float* qh = q + ((size_t)r * (size_t)H + (size_t)h) * (size_t)d;
                double dot = 0.0, dmag = 0.0;
                for (int32_t i = 0; i < d; ++i) {
                    const double p = (double)qh[i] * (double)kt[i];
                    dot += p;
                    dmag += fabs(p);
                }
                const double wh = (double)w[(size_t)r * (size_t)H + (size_t)h];
                acc += wh * (dot > 0.0 ? dot : 0.0);
                mag += fabs(wh) * dmag;
            }
            logits[(size_t)r * (size_t)n + (size_t)t] = acc;
            if (absterm) absterm[(size_t)r * (size_t)n + (size_t)t] = mag;
        }
    }
    return ORACLE_OK;
}

/*
 * Attention over the selected positions: the TopK article, section 01,
 * step 3 of DSA-style decoding (attention computed only on the keys and
 * values of the k selected positions).  The article gives no formula;
 * the one taken is plain scaled dot-product attention of each query head
 * over the selected positions, keys and values shared by the heads:
 *
 *     s_j = scale * q[r][h] . K[r][idx_j],   p_j = exp(s_j) / sum_j' exp(s_j')
 *     out[r][h][:] = sum_j p_j * V[r][idx_j][:]
 *
 * over the slots j with idx_j >= 0 (a -1 slot holds no position); a row
 * with no such slot gives zeros.  q [rows, H, d]; the keys and values of
 * row r are [n, d] arrays at kc + r*kvstride and vc + r*kvstride; idx
 * [rows, k].  Double precision, softmax with its maximum subtracted.
 * mag[r][h][c] (optional) receives sum_j p_j * |V[idx_j][c]| and smax[r][h]
 * (optional) max_j scale * sum_i |q_i K[idx_j]_i|: the scales of float32
 * rounding errors.
 */
int oracle_sparse_attention(const float* q, const float* kc, const float* vc, const int32_t* idx, int32_t rows,
                            int32_t n, int32_t H, int32_t d, int64_t kvstride, int32_t k, double scale,
                            double* out, double* mag, double* smax) {
    if (rows < 0 || n < 1 || H < 1 || d < 1 || k < 1 || kvstride < 0) return ORACLE_ERR_ARG;
    if (rows == 0) return ORACLE_OK;
    if (!q || !kc || !vc || !idx || !out) return ORACLE_ERR_ARG;
    double* s = (double*)malloc(sizeof(double) * (size_t)k);
    double* sa = (double*)malloc(sizeof(double) * (size_t)k);
    if (!s || !sa) {
        free(s);
        free(sa);
        return ORACLE_ERR_NOMEM;
    }
    int rc = ORACLE_OK;
    for (int32_t r = 0; r < rows && rc == ORACLE_OK; ++r) {
        const float* K = kc + (size_t)r * (size_t)kvstride;
        const float* V = vc + (size_t)r * (size_t)kvstride;
        const int32_t* ix = idx + (size_t)r * (size_t)k;
        for (int32_t h = 0; h < H; ++h) {
            const float* qh = q + ((size_t)r * (size_t)H + (size_t)h) * (size_t)d;
            double* o = out + ((size_t)r * (size_t)H + (size_t)h) * (size_t)d;
            double* mg = mag ? mag + ((size_t)r * (size_t)H + (size_t)h) * (size_t)d : NULL;
            double best = -INFINITY, bestabs = 0.0;
            int any = 0;
            for (int32_t j = 0; j < k; ++j) {
                if (ix[j] < 0) continue;
                if (ix[j] >= n) {
                    rc = ORACLE_ERR_ARG;
                    break;
                }
                const float* kt = K + (size_t)ix[j] * (size_t)d;
                double dot = 0.0, dabs = 0.0;
                for (int32_t i = 0; i < d; ++i) {
                    dot += (double)qh[i] * (double)kt[i];
                    dabs += fabs((double)qh[i] * (double)kt[i]);
                }
                s[j] = scale * dot;
                sa[j] = fabs(scale) * dabs;
                if (s[j] > best) best = s[j];
                if (sa[j] > bestabs) bestabs = sa[j];
                any = 1;
            }
            if (rc != ORACLE_OK) break;
            for (int32_t c = 0; c < d; ++c) {
                o[c] = 0.0;
                if (mg) mg[c] = 0.0;
            }
            if (smax) smax[(size_t)r * (size_t)H + (size_t)h] = bestabs;
            if (!any) continue;
            double den = 0.0;
            for (int32_t j = 0; j < k; ++j)
                if (ix[j] >= 0) den += exp(s[j] - best);
            for (int32_t j = 0; j < k; ++j) {
                if (ix[j] < 0) continue;
                const double p = exp(s[j] - best) / den;
                const float* vt = V + (size_t)ix[j] * (size_t)d;
                for (int32_t c = 0; c < d; ++c) {
                    o[c] += p * (double)vt[c];
                    if (mg) mg[c] += p * fabs((double)vt[c]);
                }
            }
        }
    }
    free(s);
    free(sa);
    return rc;
}
