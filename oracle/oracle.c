/*
 * oracle.c -- plain, slow CPU oracle for the DSA lightning indexer and the
 * ADIndex group token bank.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU path; it reads the same input bytes.
 *
 * Everything is computed in fp64 from the dequantised inputs and follows the
 * definitions of "ADIndex: Layer-Adaptive Sparse Attention Indexing via
 * Group-Level Distillation" (Qi et al.):
 *
 *   score   I_{t,s} = sum_{j=1..H} w_{t,j} * ReLU(q_{t,j} . k_s),  s <= t
 *           (Section 3, Eq. (1); Appendix C.3 states that the ReLU acts on each
 *           query-key dot product before the weighted sum over heads)
 *   select  T_t = TopK_{s<=t}(I_{t,s}, K)                 (Section 3, Eq. (2))
 *   bank    P_t = TopK_{s<=t}(Ibar_{t,s}, P) with the group indexer of Eq. (8),
 *           built only when the anchor-visible prefix t+1 exceeds P
 *                                                          (Section 4.3, Eq. (13))
 *   refine  C_i = P_t U {t+1..i},  T_i = TopK_{s in C_i}(I_{i,s}, K)
 *                                                          (Section 4.3, Eq. (14))
 *   grouping: consecutive, non-overlapping groups of G; incomplete groups use
 *           the original indexer                          (Section 4.3, prefill)
 *   MTP:    windows of m queries; the window reuses banks only when its first
 *           query sees more than P keys, then every group scans its anchor's
 *           visible prefix (Section 4.3, MTP; Appendix A.2, Eq. (20)-(21))
 *   pooled: the training-free group query is the mean of the group's own
 *           queries and gates (Section 5 Abl. 2; Appendix B.3, B.4)
 *
 * Readings where the pages are silent (each one also listed in the design
 * notes): no extra scale factor in Eq. (1); s = t is visible; ties rank the
 * lower index first; -0 is ranked as +0; a row's selected indices are written
 * in ascending order and padded with -1 (scores with -inf); the bank is the
 * whole prefix when it is built for a prefix not longer than P (forced mode);
 * query i = t sees only the bank (the literal candidate set of Eq. (14));
 * the mean pooling averages the final indexer queries and gates head by head
 * (the fp64 mean, rounded once: the query to bf16, the gates to fp32); query r
 * of an MTP window whose first query sees N keys sits at position N - 1 + r.
 *
 * Precision: inputs are widened to double (bf16 and E4M3 widen exactly; an
 * E4M3 value times its fp32 scale is exact in double), every sum is a double
 * sum in index order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#include "oracle.h"

/* ---------------------------------------------------------------- inputs */

/* OCP 8-bit floating point specification, E4M3 ("fn"): 1 sign bit, 4 exponent
 * bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
 * m/8 * 2^-6; S.1111.111 is NaN; there are no infinities (max 448). */
double oracle_e4m3_to_double(uint8_t c)
{
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9); /* (m/8) * 2^(1-7) */
    else
        v = ldexp(8.0 + m, e - 10); /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_elem(const void *p, int dtype, int64_t i)
{
    switch (dtype) {
    case ORACLE_F32: return (double)((const float *)p)[i];
    case ORACLE_BF16: return oracle_bf16_to_double(((const uint16_t *)p)[i]);
    case ORACLE_E4M3: return oracle_e4m3_to_double(((const uint8_t *)p)[i]);
    }
    return NAN;
}

/* Row r (n values) of a tensor, widened to double and multiplied by the row's
 * scale when one is given (per-token fp32 scale of the E4M3 inputs). */
static void load_row(const void *p, const float *scale, int dtype, int64_t r, int n, double *out)
{
    double sc = scale ? (double)scale[r] : 1.0;
    for (int c = 0; c < n; ++c)
        out[c] = load_elem(p, dtype, r * (int64_t)n + c) * sc;
}

/* ----------------------------------------------------------- score, Eq. 1 */

/* I = sum_j w_j * ReLU(q_j . k): qrow is [H*d], wrow is [H], krow is [d]. */
static double indexer_score(const double *qrow, const double *wrow, const double *krow, int H, int d)
{
    double total = 0.0;
    for (int j = 0; j < H; ++j) {
        double dot = 0.0;
        for (int c = 0; c < d; ++c)
            dot += qrow[(int64_t)j * d + c] * krow[c];
        double relu = dot > 0.0 ? dot : 0.0;
        total += wrow[j] * relu;
    }
    if (total == 0.0)
        total = 0.0; /* rank -0 as +0 */
    return total;
}

/* ------------------------------------------------------- top-K, Eq. 2/13/14 */

typedef struct {
    double s;
    int64_t idx;
} cand_t;

/* Ranking order: higher score first, then lower index. */
static int by_rank(const void *a, const void *b)
{
    const cand_t *x = a, *y = b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->idx > y->idx) - (x->idx < y->idx);
}

static int by_index(const void *a, const void *b)
{
    const cand_t *x = a, *y = b;
    return (x->idx > y->idx) - (x->idx < y->idx);
}

/* Keep the first min(K, n) candidates of the ranking order; write their
 * indices in ascending order, then -1 padding (scores: -inf padding). */
static void select_topk(cand_t *c, int64_t n, int K, int32_t *out_idx, double *out_score)
{
    qsort(c, (size_t)n, sizeof *c, by_rank);
    int64_t m = n < K ? n : K;
    qsort(c, (size_t)m, sizeof *c, by_index);
    for (int64_t r = 0; r < K; ++r) {
        if (r < m) {
            if (out_idx) out_idx[r] = (int32_t)c[r].idx;
            if (out_score) out_score[r] = c[r].s;
        } else {
            if (out_idx) out_idx[r] = -1;
            if (out_score) out_score[r] = -INFINITY;
        }
    }
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Dequantised copy of every key row: [Tk, d] doubles. */
static double *load_keys(const void *k, const float *k_scale, int dtype, int64_t Tk, int d)
{
    double *K = malloc(sizeof(double) * (size_t)(Tk > 0 ? Tk : 1) * (size_t)d);
    if (!K) return NULL;
    for (int64_t s = 0; s < Tk; ++s)
        load_row(k, k_scale, dtype, s, d, K + s * d);
    return K;
}

/* ------------------------------------------------- single scores, Eq. 1 */

int oracle_score_pairs(const void *q, const float *q_scale, int q_dtype, const void *k,
                       const float *k_scale, int k_dtype, const float *w, int H, int d,
                       const int64_t *rows, const int64_t *keys, int64_t n, double *out,
                       int nthreads)
{
    if (H <= 0 || d <= 0 || n < 0)
        return -1;
    set_threads(nthreads);
    int err = 0;
#pragma omp parallel
    {
        double *qrow = malloc(sizeof(double) * (size_t)H * d);
        double *wrow = malloc(sizeof(double) * (size_t)H);
        double *krow = malloc(sizeof(double) * (size_t)d);
        if (!qrow || !wrow || !krow)
            err = -2;
#pragma omp for schedule(static)
        for (int64_t p = 0; p < n; ++p) {
            if (!qrow || !wrow || !krow) continue;
            load_row(q, q_scale, q_dtype, rows[p], H * d, qrow);
            for (int j = 0; j < H; ++j) wrow[j] = (double)w[rows[p] * H + j];
            load_row(k, k_scale, k_dtype, keys[p], d, krow);
            out[p] = indexer_score(qrow, wrow, krow, H, d);
        }
        free(qrow); free(wrow); free(krow);
    }
    return err;
}

/* The absolute condition of Eq. (1) for one pair: sum_j |w_j| sum_c |q_jc| |k_c|.
 * Any evaluation of the score in binary32 arithmetic (a sum of about d + H
 * rounded products and partial sums) errs by at most a small multiple of the
 * unit roundoff times this sum of magnitudes: the standard forward error bound
 * of a floating-point sum, |fl(sum x_i) - sum x_i| <= gamma_n sum |x_i|. */
static double indexer_cond(const double *qrow, const double *wrow, const double *krow, int H, int d)
{
    double total = 0.0;
    for (int j = 0; j < H; ++j) {
        double dot = 0.0;
        for (int c = 0; c < d; ++c)
            dot += fabs(qrow[(int64_t)j * d + c]) * fabs(krow[c]);
        total += fabs(wrow[j]) * dot;
    }
    return total;
}

int oracle_score_pairs_cond(const void *q, const float *q_scale, int q_dtype, const void *k,
                            const float *k_scale, int k_dtype, const float *w, int H, int d,
                            const int64_t *rows, const int64_t *keys, int64_t n, double *out,
                            int nthreads)
{
    if (H <= 0 || d <= 0 || n < 0)
        return -1;
    set_threads(nthreads);
    int err = 0;
#pragma omp parallel
    {
        double *qrow = malloc(sizeof(double) * (size_t)H * d);
        double *wrow = malloc(sizeof(double) * (size_t)H);
        double *krow = malloc(sizeof(double) * (size_t)d);
        if (!qrow || !wrow || !krow)
            err = -2;
#pragma omp for schedule(static)
        for (int64_t p = 0; p < n; ++p) {
            if (!qrow || !wrow || !krow) continue;
            load_row(q, q_scale, q_dtype, rows[p], H * d, qrow);
            for (int j = 0; j < H; ++j) wrow[j] = (double)w[rows[p] * H + j];
            load_row(k, k_scale, k_dtype, keys[p], d, krow);
            out[p] = indexer_cond(qrow, wrow, krow, H, d);
        }
        free(qrow); free(wrow); free(krow);
    }
    return err;
}

/* ------------------------------------------------------ dense prefill */

int oracle_prefill(const void *q, const float *q_scale, const void *k, const float *k_scale,
                   const float *w, int dtype, int64_t Tq, int64_t Tk, int H, int d, int64_t q_pos0,
                   int topk, const int64_t *rows, int64_t nrows, int32_t *out_idx,
                   double *out_score, int nthreads)
{
    if (q_pos0 < 0 || q_pos0 + Tq > Tk || topk <= 0 || H <= 0 || d <= 0)
        return -1;
    set_threads(nthreads);
    double *K = load_keys(k, k_scale, dtype, Tk, d);
    if (!K) return -2;
    int64_t n_out = rows ? nrows : Tq;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_out; ++r) {
        int64_t i = rows ? rows[r] : r;
        if (i < 0 || i >= Tq) { err = -1; continue; }
        int64_t t = q_pos0 + i; /* the query's position; it sees keys 0..t */
        double *qrow = malloc(sizeof(double) * (size_t)H * d);
        double *wrow = malloc(sizeof(double) * (size_t)H);
        cand_t *c = malloc(sizeof(cand_t) * (size_t)(t + 1));
        if (!qrow || !wrow || !c) { err = -2; free(qrow); free(wrow); free(c); continue; }
        load_row(q, q_scale, dtype, i, H * d, qrow);
        for (int j = 0; j < H; ++j) wrow[j] = (double)w[i * H + j];
        for (int64_t s = 0; s <= t; ++s) {
            c[s].s = indexer_score(qrow, wrow, K + s * d, H, d);
            c[s].idx = s;
        }
        select_topk(c, t + 1, topk, out_idx ? out_idx + r * topk : NULL,
                    out_score ? out_score + r * topk : NULL);
        free(qrow); free(wrow); free(c);
    }
    free(K);
    return err;
}

/* ------------------------------------------------------------- decode */

int oracle_decode(const void *q, const uint8_t *k_cache, const float *k_scale, const float *w,
                  const int32_t *seq_lens, int B, int64_t Nmax, int H, int d, int topk,
                  const int64_t *rows, int64_t nrows, int32_t *out_idx, double *out_score,
                  int nthreads)
{
    if (B < 0 || topk <= 0 || H <= 0 || d <= 0)
        return -1;
    set_threads(nthreads);
    int64_t n_out = rows ? nrows : B;
    for (int64_t r = 0; r < n_out; ++r) {
        int64_t b = rows ? rows[r] : r;
        if (b < 0 || b >= B) return -1;
        int64_t n = seq_lens[b]; /* one new query sees the whole cache 0..n-1 */
        if (n < 0 || n > Nmax) return -1;
        double *qrow = malloc(sizeof(double) * (size_t)H * d);
        double *wrow = malloc(sizeof(double) * (size_t)H);
        cand_t *c = malloc(sizeof(cand_t) * (size_t)(n > 0 ? n : 1));
        if (!qrow || !wrow || !c) { free(qrow); free(wrow); free(c); return -2; }
        load_row(q, NULL, ORACLE_BF16, b, H * d, qrow);
        for (int j = 0; j < H; ++j) wrow[j] = (double)w[b * H + j];
#pragma omp parallel
        {
            double *krow = malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(static)
            for (int64_t s = 0; s < n; ++s) {
                load_row(k_cache, k_scale, ORACLE_E4M3, b * Nmax + s, d, krow);
                c[s].s = indexer_score(qrow, wrow, krow, H, d);
                c[s].idx = s;
            }
            free(krow);
        }
        select_topk(c, n, topk, out_idx ? out_idx + r * topk : NULL,
                    out_score ? out_score + r * topk : NULL);
        free(qrow); free(wrow); free(c);
    }
    return 0;
}

/* ---------------------------------------------------------- group bank */

/* Is group g (queries gG .. gG+G-1 of the call) served by a shared bank?
 * Complete groups whose anchor t = q_pos0 + gG sees more than P keys build a
 * bank; the forced mode builds one for every complete group. */
static int group_uses_bank(int64_t g, int64_t Tq, int64_t q_pos0, int G, int P, unsigned flags)
{
    if ((g + 1) * G > Tq)
        return 0; /* incomplete group: original indexer */
    int64_t anchor = q_pos0 + g * G;
    if (flags & ORACLE_NO_BANK)
        return 0;
    if (flags & ORACLE_FORCE_BANK)
        return 1;
    if (flags & ORACLE_WINDOW)
        anchor = q_pos0; /* MTP: decided once, on the window's first query */
    return anchor + 1 > P;
}

int64_t oracle_group_bank_pairs(int64_t Tq, int64_t q_pos0, int G, int P, unsigned flags)
{
    int64_t pairs = 0;
    for (int64_t i = 0; i < Tq; ++i) {
        int64_t g = i / G, t = q_pos0 + i;
        if (!group_uses_bank(g, Tq, q_pos0, G, P, flags)) {
            pairs += t + 1;
            continue;
        }
        int64_t anchor = q_pos0 + g * G;
        int64_t nb = anchor + 1 < P ? anchor + 1 : P;
        if (i == g * G)
            pairs += anchor + 1; /* the group indexer's one prefix scan */
        pairs += nb + (t - anchor); /* bank plus post-anchor tokens */
    }
    return pairs;
}

/* The bank of group g: the P best prefix positions by the group score, in
 * ascending order; returns its size min(P, anchor+1). */
static int64_t build_bank(const double *K, const void *qbar, const float *qbar_scale,
                          const float *wbar, int dtype, int Hs, int d, int64_t g, int64_t anchor,
                          int P, int64_t *bank)
{
    double *qrow = malloc(sizeof(double) * (size_t)Hs * d);
    double *wrow = malloc(sizeof(double) * (size_t)Hs);
    cand_t *c = malloc(sizeof(cand_t) * (size_t)(anchor + 1));
    int32_t *sel = malloc(sizeof(int32_t) * (size_t)P);
    if (!qrow || !wrow || !c || !sel) { free(qrow); free(wrow); free(c); free(sel); return -1; }
    load_row(qbar, qbar_scale, dtype, g, Hs * d, qrow);
    for (int j = 0; j < Hs; ++j) wrow[j] = (double)wbar[g * Hs + j];
    for (int64_t s = 0; s <= anchor; ++s) {
        c[s].s = indexer_score(qrow, wrow, K + s * d, Hs, d);
        c[s].idx = s;
    }
    select_topk(c, anchor + 1, P, sel, NULL);
    int64_t nb = anchor + 1 < P ? anchor + 1 : P;
    for (int64_t r = 0; r < nb; ++r) bank[r] = sel[r];
    free(qrow); free(wrow); free(c); free(sel);
    return nb;
}

/* Eq. (13)-(14) over keys already widened to fp64 (K [>= q_pos0+Tq, d]);
 * q, qbar in `dtype` codes.  Rows and outputs as in oracle_group_bank. */
static int group_bank_core(const double *K, const void *q, const float *q_scale, const float *w,
                           int dtype, int64_t Tq, int H, int d, int64_t q_pos0, const void *qbar,
                           const float *qbar_scale, const float *wbar, int Hs, int G, int P,
                           int topk, unsigned flags, const int64_t *rows, int64_t nrows,
                           int32_t *out_idx, double *out_score, int32_t *out_bank)
{
    int64_t NG = (Tq + G - 1) / G;
    int64_t n_out = rows ? nrows : Tq;

    /* which groups' banks are needed: those of the requested rows (every row
     * when `rows` is NULL); out_bank rows of other groups are written as -1 */
    char *need = calloc((size_t)(NG > 0 ? NG : 1), 1);
    int64_t **banks = calloc((size_t)(NG > 0 ? NG : 1), sizeof(int64_t *));
    int64_t *nbank = calloc((size_t)(NG > 0 ? NG : 1), sizeof(int64_t));
    if (!need || !banks || !nbank) { free(need); free(banks); free(nbank); return -2; }
    for (int64_t r = 0; r < n_out; ++r) {
        int64_t i = rows ? rows[r] : r;
        if (i < 0 || i >= Tq) { free(need); free(banks); free(nbank); return -1; }
        need[i / G] = 1;
    }

    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t g = 0; g < NG; ++g) {
        if (!need[g] || !group_uses_bank(g, Tq, q_pos0, G, P, flags)) continue;
        int64_t anchor = q_pos0 + g * G;
        banks[g] = malloc(sizeof(int64_t) * (size_t)P);
        if (!banks[g]) { err = -2; continue; }
        nbank[g] = build_bank(K, qbar, qbar_scale, wbar, dtype, Hs, d, g, anchor, P, banks[g]);
        if (nbank[g] < 0) err = -2;
    }
    if (out_bank)
        for (int64_t g = 0; g < NG; ++g)
            for (int64_t r = 0; r < P; ++r)
                out_bank[g * P + r] = (banks[g] && r < nbank[g]) ? (int32_t)banks[g][r] : -1;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_out; ++r) {
        int64_t i = rows ? rows[r] : r;
        int64_t g = i / G, t = q_pos0 + i;
        double *qrow = malloc(sizeof(double) * (size_t)H * d);
        double *wrow = malloc(sizeof(double) * (size_t)H);
        cand_t *c = malloc(sizeof(cand_t) * (size_t)(t + 1 + P));
        if (!qrow || !wrow || !c) { err = -2; free(qrow); free(wrow); free(c); continue; }
        load_row(q, q_scale, dtype, i, H * d, qrow);
        for (int j = 0; j < H; ++j) wrow[j] = (double)w[i * H + j];
        int64_t n = 0;
        if (banks[g]) {
            /* candidate set of Eq. (14): the bank, then anchor+1 .. t */
            int64_t anchor = q_pos0 + g * G;
            for (int64_t b = 0; b < nbank[g]; ++b) c[n++].idx = banks[g][b];
            for (int64_t s = anchor + 1; s <= t; ++s) c[n++].idx = s;
        } else {
            for (int64_t s = 0; s <= t; ++s) c[n++].idx = s;
        }
        for (int64_t m = 0; m < n; ++m)
            c[m].s = indexer_score(qrow, wrow, K + c[m].idx * d, H, d);
        select_topk(c, n, topk, out_idx ? out_idx + r * topk : NULL,
                    out_score ? out_score + r * topk : NULL);
        free(qrow); free(wrow); free(c);
    }
    for (int64_t g = 0; g < NG; ++g) free(banks[g]);
    free(banks); free(nbank); free(need);
    return err;
}

int oracle_group_bank(const void *q, const float *q_scale, const void *k, const float *k_scale,
                      const float *w, int dtype, int64_t Tq, int64_t Tk, int H, int d,
                      int64_t q_pos0, const void *qbar, const float *qbar_scale, const float *wbar,
                      int Hs, int G, int P, int topk, unsigned flags, const int64_t *rows,
                      int64_t nrows, int32_t *out_idx, double *out_score, int32_t *out_bank,
                      int64_t *pairs, int nthreads)
{
    if (q_pos0 < 0 || q_pos0 + Tq > Tk || topk <= 0 || H <= 0 || Hs <= 0 || d <= 0 || G <= 0 ||
        P <= 0)
        return -1;
    set_threads(nthreads);
    double *K = load_keys(k, k_scale, dtype, Tk, d);
    if (!K) return -2;
    int err = group_bank_core(K, q, q_scale, w, dtype, Tq, H, d, q_pos0, qbar, qbar_scale, wbar, Hs,
                              G, P, topk, flags, rows, nrows, out_idx, out_score, out_bank);
    if (pairs)
        *pairs = oracle_group_bank_pairs(Tq, q_pos0, G, P, flags);
    free(K);
    return err;
}

/* ------------------------------------------------ MTP target verification
 * Section 4.3 (application to MTP) and Appendix A.2, Eq. (20)-(22).  Each of
 * B sequences verifies a window of m query tokens: query r of sequence b sits
 * at position N_b - 1 + r, so it sees N_b + r keys of that sequence's cache.
 * Whether the window reuses banks is decided once, on N_b: N_b <= P sends all
 * m queries to the original indexer; otherwise the window splits into m/G
 * groups, the anchor of group g (query gG) builds a bank of the P best of its
 * N_b + gG visible keys with the group query, and every member refines over
 * the bank plus the keys after the anchor (Eq. 14).  Queries are bf16; the
 * cache is E4M3 codes with one fp32 scale per token, as in decode.  With
 * ORACLE_NO_BANK every window uses the original indexer (the baseline). */
int64_t oracle_mtp_pairs(const int32_t *prefix_lens, int B, int m, int G, int P, unsigned flags)
{
    int64_t pairs = 0;
    for (int b = 0; b < B; ++b)
        pairs += oracle_group_bank_pairs(m, (int64_t)prefix_lens[b] - 1, G, P,
                                         ORACLE_WINDOW | (flags & ORACLE_NO_BANK));
    return pairs;
}

int oracle_mtp(const void *q, const uint8_t *k_cache, const float *k_scale, const float *w,
               const void *qbar, const float *wbar, const int32_t *prefix_lens, int B,
               int64_t Nmax, int m, int H, int Hs, int d, int G, int P, int topk, unsigned flags,
               const int64_t *rows, int64_t nrows, int32_t *out_idx, double *out_score,
               int32_t *out_bank, int64_t *pairs, int nthreads)
{
    if (B < 0 || m <= 0 || G <= 0 || m % G || topk <= 0 || H <= 0 || Hs <= 0 || d <= 0 || P <= 0)
        return -1;
    for (int b = 0; b < B; ++b)
        if (prefix_lens[b] < 1 || prefix_lens[b] + m - 1 > Nmax) return -1;
    for (int64_t r = 1; rows && r < nrows; ++r)
        if (rows[r] <= rows[r - 1]) return -1; /* rows ascending */
    set_threads(nthreads);
    const int NGs = m / G;
    int err = 0;
    int64_t r0 = 0; /* first entry of `rows` in sequence b */
    for (int b = 0; b < B && !err; ++b) {
        int64_t r1 = r0;
        if (rows)
            while (r1 < nrows && rows[r1] < (int64_t)(b + 1) * m) ++r1;
        if (rows && r1 == r0 && !out_bank) continue; /* nothing requested here */
        int64_t *lrows = NULL;
        if (rows) {
            lrows = malloc(sizeof(int64_t) * (size_t)(r1 > r0 ? r1 - r0 : 1));
            if (!lrows) return -2;
            for (int64_t r = r0; r < r1; ++r) lrows[r - r0] = rows[r] - (int64_t)b * m;
        }
        const int64_t Tk = prefix_lens[b] + m - 1; /* keys the window's last query sees */
        double *K = malloc(sizeof(double) * (size_t)Tk * (size_t)d);
        if (!K) { free(lrows); return -2; }
        for (int64_t s = 0; s < Tk; ++s)
            load_row(k_cache, k_scale, ORACLE_E4M3, (int64_t)b * Nmax + s, d, K + s * d);
        const int64_t o = rows ? r0 : (int64_t)b * m; /* output row of this call's first row */
        err = group_bank_core(K, (const uint16_t *)q + (size_t)b * m * H * d, NULL,
                              w + (size_t)b * m * H, ORACLE_BF16, m, H, d,
                              (int64_t)prefix_lens[b] - 1,
                              qbar ? (const uint16_t *)qbar + (size_t)b * NGs * Hs * d : NULL,
                              NULL, wbar ? wbar + (size_t)b * NGs * Hs : NULL, Hs, G, P, topk,
                              ORACLE_WINDOW | (flags & ORACLE_NO_BANK), lrows, rows ? r1 - r0 : 0,
                              out_idx ? out_idx + o * topk : NULL,
                              out_score ? out_score + o * topk : NULL,
                              out_bank ? out_bank + (size_t)b * NGs * P : NULL);
        free(K); free(lrows);
        r0 = r1;
    }
    if (pairs)
        *pairs = oracle_mtp_pairs(prefix_lens, B, m, G, P, flags);
    return err;
}

/* ------------------------------------------- training-free group query
 * The "w/o training" variant of Section 5 (Abl. 2, Table 3) and the mean
 * pooling of Appendix B.3 (Table 8) and B.4: the frozen DSA indexer builds the
 * bank with a group query that is the mean of the group's own indexer
 * queries, head by head, and head weights that are the mean of theirs.
 * The pooled query is stored in bf16 and the weights in fp32, so each is the
 * mean rounded once to the nearest value of its format (ties to even).  The
 * mean is taken in fp64: the sum of G <= 16 bf16 values (8 significant bits
 * each) is exact in fp64 unless their magnitudes span more than 2^40, and the
 * sum of G fp32 gates unless theirs span more than 2^25; 1/G is a power of
 * two.  Complete groups only; the rows of an incomplete last group (which
 * never builds a bank) are zero.  bf16 queries only. */
static double bf16_bits_to_f64(uint16_t b)
{
    const uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, 4);
    return (double)x;
}

/* x rounded to the nearest bf16 value, ties to the even significand: bf16
 * values with exponent e (2^e <= |v| < 2^(e+1), e >= -126) are the multiples
 * of 2^(e-7); below 2^-126 (subnormal) the multiples of 2^-133.  The scaled
 * value is rounded to an integer with nearbyint (round to nearest even in the
 * default mode); scaling by a power of two is exact.  |x| stays below the
 * largest bf16 here (a mean of bf16 values). */
static uint16_t f64_to_bf16_nearest(double x)
{
    if (x == 0.0) return signbit(x) ? 0x8000u : 0u;
    int e;
    frexp(x, &e);           /* |x| = f * 2^e, f in [0.5, 1): exponent e - 1 */
    int ex = e - 1;
    if (ex < -126) ex = -126;
    const double v = ldexp(nearbyint(ldexp(x, 7 - ex)), ex - 7);
    const float f = (float)v; /* exact: v has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

int oracle_pool_mean_bf16(const uint16_t *q, const float *w, int64_t Tq, int H, int d, int G,
                          uint16_t *qbar, float *wbar)
{
    if (Tq < 0 || H <= 0 || d <= 0 || (G != 4 && G != 8 && G != 16)) return -1;
    const int64_t NG = (Tq + G - 1) / G, nfull = Tq / G;
    for (int64_t g = 0; g < NG; ++g) {
        for (int64_t e = 0; e < (int64_t)H * d; ++e) {
            double s = 0.0;
            if (g < nfull)
                for (int i = 0; i < G; ++i) s += bf16_bits_to_f64(q[(g * G + i) * (int64_t)H * d + e]);
            qbar[g * (int64_t)H * d + e] = f64_to_bf16_nearest(s / G);
        }
        for (int j = 0; j < H; ++j) {
            double s = 0.0;
            if (g < nfull)
                for (int i = 0; i < G; ++i) s += (double)w[(g * G + i) * (int64_t)H + j];
            wbar[g * (int64_t)H + j] = (float)(s / G);
        }
    }
    return 0;
}

/* --------------------------------------------- scoring-count cost model
 * Appendix A of the same paper: one query-key score is one unit of cost. */

/* Eq. (15): the original indexer over a prefill of L tokens, L^2/2. */
double oracle_cost_prefill_base(double L) { return L * L / 2.0; }

/* Eq. (19): bank sharing over a prefill of L tokens (continuous form); the
 * original indexer below P, then per group N + GP + G(G-1)/2 amortised. */
double oracle_cost_prefill_reuse(double L, double G, double P)
{
    if (L <= P)
        return L * L / 2.0;
    return P * P / 2.0 + (L * L - P * P) / (2.0 * G) + (P + (G - 1.0) / 2.0) * (L - P);
}

/* Eq. (16), one round: m queries seeing N, N+1, ..., N+m-1 keys. */
double oracle_cost_mtp_base_round(double N, int m) { return m * N + m * (m - 1) / 2.0; }

/* Eq. (20)-(21), one round: the whole window falls back when N <= P;
 * otherwise m/G groups, group b scanning N + bG keys, then G*P bank scores
 * and G(G-1)/2 post-anchor scores. */
double oracle_cost_mtp_reuse_round(double N, int G, double P, int m)
{
    if (N <= P)
        return oracle_cost_mtp_base_round(N, m);
    double c = 0.0;
    for (int b = 0; b < m / G; ++b)
        c += N + (double)b * G + G * P + G * (G - 1) / 2.0;
    return c;
}

/* Eq. (24) with the workload of Eq. (28): R rounds, round j sees
 * N_j = L + (j-1) a keys at its first query. */
double oracle_speedup_joint(double L, int G, double P, int R, int m, double a)
{
    double base = oracle_cost_prefill_base(L), reuse = oracle_cost_prefill_reuse(L, G, P);
    for (int j = 1; j <= R; ++j) {
        double N = L + (j - 1) * a;
        base += oracle_cost_mtp_base_round(N, m);
        reuse += oracle_cost_mtp_reuse_round(N, G, P, m);
    }
    return base / reuse;
}
