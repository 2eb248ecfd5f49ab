/*
 * oracle.h -- interface of the CPU oracle (test infrastructure only; see
 * oracle.c).  This header belongs to the oracle alone: the GPU library has its
 * own header and the two share nothing.
 *
 * All pointers are host memory.  Tensors are row-major with the last dimension
 * fastest: q [Tq,H,d], k [Tk,d], w [Tq,H], qbar [ceil(Tq/G),Hs,d],
 * wbar [ceil(Tq/G),Hs]; per-token fp32 scales q_scale [Tq], k_scale [Tk],
 * qbar_scale [ceil(Tq/G)] are given for E4M3 inputs and NULL otherwise.
 * Query i of a call sits at position q_pos0 + i.
 *
 * `rows` (optional) selects which query rows to compute; output row r then
 * holds query rows[r].  Outputs: out_idx [n,topk] int32 (ascending indices,
 * then -1), out_score [n,topk] double (-inf at padding).  Return 0 on success,
 * -1 on bad arguments, -2 when out of memory.
 */
#ifndef DSA_ORACLE_H
#define DSA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_E4M3 = 2 };
enum {
    ORACLE_FORCE_BANK = 1u,
    ORACLE_WINDOW = 4u,  /* MTP: one eligibility test per window */
    ORACLE_NO_BANK = 8u  /* every group uses the original indexer */
};

double oracle_e4m3_to_double(uint8_t c);
double oracle_bf16_to_double(uint16_t b);
int oracle_max_threads(void);

/* Eq. (1) for n given (query row, key row) pairs: q rows of [*, H, d] in
 * q_dtype, k rows of [*, d] in k_dtype, w rows of [*, H]. */
int oracle_score_pairs(const void *q, const float *q_scale, int q_dtype, const void *k,
                       const float *k_scale, int k_dtype, const float *w, int H, int d,
                       const int64_t *rows, const int64_t *keys, int64_t n, double *out,
                       int nthreads);

/* The absolute condition of Eq. (1) for the same pairs: sum_j |w_j| sum_c
 * |q_jc| |k_c| (dequantised), the scale of any binary32 evaluation's error. */
int oracle_score_pairs_cond(const void *q, const float *q_scale, int q_dtype, const void *k,
                            const float *k_scale, int k_dtype, const float *w, int H, int d,
                            const int64_t *rows, const int64_t *keys, int64_t n, double *out,
                            int nthreads);

int oracle_prefill(const void *q, const float *q_scale, const void *k, const float *k_scale,
                   const float *w, int dtype, int64_t Tq, int64_t Tk, int H, int d, int64_t q_pos0,
                   int topk, const int64_t *rows, int64_t nrows, int32_t *out_idx,
                   double *out_score, int nthreads);

/* q [B,H,d] bf16; k_cache [B,Nmax,d] E4M3; k_scale [B,Nmax]; the query of
 * sequence b sees keys 0 .. seq_lens[b]-1. */
int oracle_decode(const void *q, const uint8_t *k_cache, const float *k_scale, const float *w,
                  const int32_t *seq_lens, int B, int64_t Nmax, int H, int d, int topk,
                  const int64_t *rows, int64_t nrows, int32_t *out_idx, double *out_score,
                  int nthreads);

/* The training-free group query: qbar [ceil(Tq/G), H, d] bf16 bits and wbar
 * [ceil(Tq/G), H] are the means of each complete group's q [Tq, H, d] bf16 and
 * w [Tq, H] (fp32 sums in query order, times 1/G, q rounded to bf16). */
int oracle_pool_mean_bf16(const uint16_t *q, const float *w, int64_t Tq, int H, int d, int G,
                          uint16_t *qbar, float *wbar);

/* out_bank [ceil(Tq/G), P] (ascending bank positions, -1 padding, all -1 for
 * groups that use the original indexer) or NULL; with `rows`, only the banks
 * of the requested rows' groups are computed (other rows all -1).  *pairs
 * receives the number of query-key scores the method evaluates over the
 * whole call. */
int oracle_group_bank(const void *q, const float *q_scale, const void *k, const float *k_scale,
                      const float *w, int dtype, int64_t Tq, int64_t Tk, int H, int d,
                      int64_t q_pos0, const void *qbar, const float *qbar_scale, const float *wbar,
                      int Hs, int G, int P, int topk, unsigned flags, const int64_t *rows,
                      int64_t nrows, int32_t *out_idx, double *out_score, int32_t *out_bank,
                      int64_t *pairs, int nthreads);

int64_t oracle_group_bank_pairs(int64_t Tq, int64_t q_pos0, int G, int P, unsigned flags);

/* MTP target verification windows: q [B,m,H,d] bf16, k_cache [B,Nmax,d] E4M3
 * with k_scale [B,Nmax], w [B,m,H]; qbar [B,m/G,Hs,d] bf16 and wbar [B,m/G,Hs]
 * the group indexer's query; prefix_lens [B]: N_b, the keys the window's first
 * query sees (1 <= N_b, N_b + m - 1 <= Nmax).  Rows index [B*m] and must be
 * ascending; out_bank [B,m/G,P] (-1 rows for windows that fall back).
 * flags: ORACLE_NO_BANK (every window falls back) or 0. */
int oracle_mtp(const void *q, const uint8_t *k_cache, const float *k_scale, const float *w,
               const void *qbar, const float *wbar, const int32_t *prefix_lens, int B,
               int64_t Nmax, int m, int H, int Hs, int d, int G, int P, int topk, unsigned flags,
               const int64_t *rows, int64_t nrows, int32_t *out_idx, double *out_score,
               int32_t *out_bank, int64_t *pairs, int nthreads);
int64_t oracle_mtp_pairs(const int32_t *prefix_lens, int B, int m, int G, int P, unsigned flags);

double oracle_cost_prefill_base(double L);
double oracle_cost_prefill_reuse(double L, double G, double P);
double oracle_cost_mtp_base_round(double N, int m);
double oracle_cost_mtp_reuse_round(double N, int G, double P, int m);
double oracle_speedup_joint(double L, int G, double P, int R, int m, double a);

#ifdef __cplusplus
}
#endif
#endif
