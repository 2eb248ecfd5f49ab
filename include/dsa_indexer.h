/*
 * dsa_indexer.h -- C ABI of the MI355X (gfx950) DSA lightning-indexer library
 * (libdsaidx.so).
 *
 * The operations are those of "ADIndex: Layer-Adaptive Sparse Attention
 * Indexing via Group-Level Distillation" (Qi et al.):
 *
 *   Section 3, Eq. (1):  I_{t,s} = sum_{j<H} w_{t,j} * ReLU(q_{t,j} . k_s), s <= t
 *                        (no further scale factor; per-token fp8 scales are part
 *                        of the dequantised q and k)
 *   Section 3, Eq. (2):  T_t = TopK_{s<=t}(I_{t,s}, K)
 *   Section 4.3, Eq. (13)-(14) with Eq. (8): the group token bank P_t = TopK of
 *                        the group score over s <= t (size P), built for
 *                        complete groups whose anchor t sees t+1 > P keys, and
 *                        T_i = TopK over C_i = P_t U {t+1..i} with the original
 *                        indexer; other groups use Eq. (2).
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is DEVICE memory owned by the caller, contiguous,
 *    row-major (last dimension fastest) and 16-byte aligned.  The library never
 *    allocates or frees device memory: scratch comes from the caller's
 *    workspace `ws` of `ws_bytes` bytes (16-byte aligned), sized by the
 *    matching *_workspace_size() call.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously; nothing synchronises the host.
 *  - Ranking: higher score first, ties to the lower key index; -0 ranks as +0.
 *    Each output row holds the selected key indices in ascending order, then -1
 *    up to `topk`; the optional score row holds fp32 scores, -inf at padding.
 *    Exactly min(topk, number of candidates) entries are valid.  Outputs are
 *    deterministic run to run.
 *  - Inputs must be finite; they are not checked on the device.
 *  - Return value: DSAIDX_OK, or a negative dsaidx_status.  Argument errors are
 *    detected on the host before anything is enqueued and leave the outputs
 *    untouched; a failed launch returns DSAIDX_ERR_HIP; device faults surface at
 *    the caller's next synchronisation.  indexer_last_error() then returns a
 *    message for the calling thread.  No C++ exception crosses this interface.
 *  - Supported sizes: 1 <= H <= 64 (heads are padded to 32 or 64 on the
 *    device); d in {32, 64, 128} for bf16 and {64, 128} for fp8;
 *    1 <= topk <= 2048; group size G in {4, 8, 16}; topk <= P <= 16384.
 */
#ifndef DSA_INDEXER_H
#define DSA_INDEXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSAIDX_OK = 0,
    DSAIDX_ERR_INVALID_ARG = -1, /* null pointer, bad size, bad alignment */
    DSAIDX_ERR_UNSUPPORTED = -2, /* valid but outside the supported sizes */
    DSAIDX_ERR_WORKSPACE = -3,   /* ws_bytes below the *_workspace_size() value */
    DSAIDX_ERR_HIP = -4          /* a HIP launch or runtime call failed */
} dsaidx_status;

typedef enum {
    DSAIDX_BF16 = 1,     /* bfloat16 q and k, no scales */
    DSAIDX_FP8_E4M3 = 2  /* OCP FP8 E4M3 ("fn") codes, one fp32 scale per token */
} dsaidx_dtype;

enum {
    DSAIDX_FORCE_BANK = 1u, /* group bank: also build banks when t+1 <= P */
    DSAIDX_POOL_MEAN = 2u,  /* group bank, MTP: training-free group query (mean pooling) */
    DSAIDX_NO_BANK = 8u     /* MTP: every window uses the original indexer (no reuse) */
};

/*
 * Dense causal indexer, Eq. (1)-(2).  Query i of the call sits at position
 * q_pos0 + i and sees keys 0 .. q_pos0 + i; a chunked prefill passes each
 * query chunk with its q_pos0 and Tk >= q_pos0 + Tq.
 *   q        [Tq, H, d]   dtype codes
 *   q_scale  [Tq] fp32    per-query-token scale (fp8 only, else NULL)
 *   k        [Tk, d]      dtype codes
 *   k_scale  [Tk] fp32    per-key-token scale (fp8 only, else NULL)
 *   w        [Tq, H] fp32 per-query head weights
 *   out_idx  [Tq, topk] int32;  out_score [Tq, topk] fp32 or NULL
 * The Tq x Tk score matrix is never stored: each query keeps a candidate
 * buffer of cap = 2 topk + 2048 entries (rounded up to a multiple of 64) in
 * `ws`, 8 bytes per entry, for the queries of one launch (at most 16384), so
 * the workspace does not depend on Tk.  A query that sees at most cap keys
 * stores its whole (short) score row there and selects once at the end; a
 * longer one streams: only scores above a running threshold enter the
 * buffer, and a radix selection compacts it to the best topk when it fills.
 */
int indexer_prefill(const void *q, const float *q_scale, const void *k, const float *k_scale,
                    const float *w, int dtype, int64_t Tq, int64_t Tk, int H, int d,
                    int64_t q_pos0, int topk, int32_t *out_idx, float *out_score, void *ws,
                    size_t ws_bytes, void *stream);
size_t indexer_prefill_workspace_size(int64_t Tq, int64_t Tk, int H, int d, int topk, int dtype);

/*
 * Decode indexer, Eq. (1)-(2) for one new query per sequence, scanning its
 * whole cache (Section 3: O(L) per decoding query).
 *   q        [B, H, d] bf16
 *   k_cache  [B, Nmax, d] E4M3 codes;  k_scale [B, Nmax] fp32
 *   w        [B, H] fp32
 *   seq_lens [B] int32 (device): sequence b's query sees keys 0 .. seq_lens[b]-1,
 *            0 <= seq_lens[b] <= Nmax (checked on the device: out-of-range
 *            lengths are clamped to [0, Nmax])
 *   out_idx  [B, topk] int32;  out_score [B, topk] fp32 or NULL
 */
int indexer_decode(const void *q, const uint8_t *k_cache, const float *k_scale, const float *w,
                   const int32_t *seq_lens, int B, int64_t Nmax, int H, int d, int topk,
                   int32_t *out_idx, float *out_score, void *ws, size_t ws_bytes, void *stream);
size_t indexer_decode_workspace_size(int B, int64_t Nmax, int H, int d, int topk);

/*
 * indexer_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops, harnesses that forbid hipMalloc): the same
 * arguments and kernels, with the workspace taken from a fixed device array
 * inside the library instead of `ws`.  Each GPU the library runs on holds its
 * own array of indexer_decode_noalloc_max_bytes() bytes (96 MiB: enough for
 * 32 sequences of 262144 keys) from the library's load until the process
 * ends.  Sizes whose workspace would exceed it are refused on the host
 * (DSAIDX_ERR_UNSUPPORTED).  The call allocates nothing; it clears what must
 * start at zero on `stream` itself.  Calls that overlap on one GPU share the
 * array and race: issue them on one stream, or wait between them.  `stream`
 * must belong to the current device.
 */
int indexer_decode_noalloc(const void *q, const uint8_t *k_cache, const float *k_scale, const float *w,
                           const int32_t *seq_lens, int B, int64_t Nmax, int H, int d, int topk,
                           int32_t *out_idx, float *out_score, void *stream);
size_t indexer_decode_noalloc_max_bytes(void);

/*
 * ADIndex group token bank, Section 4.3 Eq. (13)-(14) with the group score of
 * Eq. (8).  Queries are as in indexer_prefill; the call's queries form
 * consecutive groups of G starting at query 0 (q_pos0 must be a multiple of
 * G).  Group g's anchor sits at t = q_pos0 + gG.
 *   qbar       [ceil(Tq/G), Hs, d] dtype codes: the group indexer's query
 *   qbar_scale [ceil(Tq/G)] fp32 (fp8 only, else NULL)
 *   wbar       [ceil(Tq/G), Hs] fp32: the group indexer's head weights
 *   flags      DSAIDX_FORCE_BANK and/or DSAIDX_POOL_MEAN, or 0
 *   out_idx    [Tq, topk] int32; out_score [Tq, topk] fp32 or NULL
 *   out_bank   [ceil(Tq/G), P] int32 or NULL: each bank in ascending order
 *              (min(P, t+1) entries, then -1); rows of groups that use the
 *              original indexer are all -1
 * DSAIDX_POOL_MEAN is the training-free variant of Section 5 (ablation 2,
 * Table 3) and Appendix B.3-B.4: no group indexer; each bank group's query
 * and gates are the mean of its G members' q and w (fp32 sums in query
 * order, times 1/G, the query rounded to the nearest bf16), over all H heads.
 * It takes bf16 inputs, qbar = wbar = qbar_scale = NULL and Hs == H; the
 * pooled values live in `ws` (no extra allocation).
 */
int indexer_group_bank(const void *q, const float *q_scale, const void *k, const float *k_scale,
                       const float *w, int dtype, int64_t Tq, int64_t Tk, int H, int d,
                       int64_t q_pos0, const void *qbar, const float *qbar_scale,
                       const float *wbar, int Hs, int G, int P, int topk, unsigned flags,
                       int32_t *out_idx, int32_t *out_bank, float *out_score, void *ws,
                       size_t ws_bytes, void *stream);
/* Workspace bytes for any q_pos0 and bank layout; `flags` as in the call (only
 * DSAIDX_POOL_MEAN changes the size: it adds the pooled queries and gates). */
size_t indexer_group_bank_workspace_size(int64_t Tq, int64_t Tk, int H, int Hs, int d, int G,
                                         int P, int topk, int dtype, unsigned flags);

/*
 * Layer-wise reuse, Section 4.1 (Eq. (5): each layer keeps its own calibrated
 * group size and bank budget), Section 4.3 and Appendix C.4 (Tables 9-14 list
 * the per-layer (G, P) of two models): one call runs the indexer of nlayers
 * layers that share the shapes (Tq, Tk, H, d, q_pos0, topk, dtype), each with
 * its own tensors and setting.  A layer with G = 0 runs the original indexer
 * (indexer_prefill; its qbar, qbar_scale, wbar, out_bank must be NULL and
 * flags 0); any other layer runs indexer_group_bank with its G, P, Hs and
 * flags.  Every layer is checked before anything is enqueued (an error names
 * the layer and leaves every output untouched); the layers then run in
 * order on `stream`, one after another, sharing one workspace of
 * indexer_layers_workspace_size() bytes (the largest layer's need).
 */
typedef struct {
    const void *q;          /* [Tq, H, d] dtype codes */
    const float *q_scale;   /* [Tq] (fp8) or NULL */
    const void *k;          /* [Tk, d] dtype codes */
    const float *k_scale;   /* [Tk] (fp8) or NULL */
    const float *w;         /* [Tq, H] */
    const void *qbar;       /* G > 0: [ceil(Tq/G), Hs, d] (NULL with DSAIDX_POOL_MEAN) */
    const float *qbar_scale;/* G > 0, fp8: [ceil(Tq/G)] */
    const float *wbar;      /* G > 0: [ceil(Tq/G), Hs] (NULL with DSAIDX_POOL_MEAN) */
    int Hs;                 /* G > 0: group-indexer heads */
    int G, P;               /* G = 0: the original indexer (P ignored) */
    unsigned flags;         /* G > 0: DSAIDX_FORCE_BANK, DSAIDX_POOL_MEAN or 0 */
    int32_t *out_idx;       /* [Tq, topk] */
    float *out_score;       /* [Tq, topk] or NULL */
    int32_t *out_bank;      /* G > 0: [ceil(Tq/G), P] or NULL */
} dsaidx_layer;

int indexer_layers(const dsaidx_layer *layers, int nlayers, int dtype, int64_t Tq, int64_t Tk, int H,
                   int d, int64_t q_pos0, int topk, void *ws, size_t ws_bytes, void *stream);
/* Workspace bytes of indexer_layers for any q_pos0 (0 on bad arguments). */
size_t indexer_layers_workspace_size(const dsaidx_layer *layers, int nlayers, int64_t Tq, int64_t Tk,
                                     int H, int d, int topk, int dtype);

/* Number of query-key scores indexer_group_bank evaluates for these sizes
 * (the unit of the cost model of Appendix A.1): fallback queries score t+1
 * keys, a bank group scores its anchor prefix once and each member i scores
 * |P_t| + (i - t) candidates.  Host only; -1 on bad arguments. */
int64_t indexer_group_bank_pairs(int64_t Tq, int64_t q_pos0, int G, int P, unsigned flags);

/*
 * MTP target verification with bank sharing: Section 4.3 ("Application to
 * Prefill and MTP") and Appendix A.2, Eq. (20)-(22).  Each of B sequences
 * verifies a window of m draft queries.  Query r of sequence b sits at
 * position N_b - 1 + r, so it sees keys 0 .. N_b - 1 + r of its cache, where
 * N_b = prefix_lens[b].  A window reuses banks only when N_b > P (decided once
 * per window): it splits into m/G groups; group g's anchor (query gG) ranks its
 * N_b + gG visible keys with the group indexer and keeps the best P (the
 * bank, Eq. (8), (13)); member i ranks the bank plus the i keys after the
 * anchor with its own query (Eq. (14)).  A window with N_b <= P uses the
 * original indexer for all m queries.  The arithmetic is that of
 * indexer_decode (bf16 queries against the E4M3 cache).
 *   q           [B, m, H, d] bf16;  w [B, m, H] fp32
 *   k_cache     [B, Nmax, d] E4M3 codes;  k_scale [B, Nmax] fp32
 *   qbar, wbar  [B, m/G, Hs, d] bf16 and [B, m/G, Hs] fp32: the group
 *               indexer's query and gates; NULL with DSAIDX_POOL_MEAN (then
 *               each group's mean query and gates are used, Hs == H)
 *   prefix_lens [B] int32, device: N_b, clamped on the device to [1, Nmax-m+1]
 *               (the cache must hold the window's own keys)
 *   flags       DSAIDX_POOL_MEAN, DSAIDX_NO_BANK (the original indexer for
 *               every window, as for a layer configured without reuse; qbar
 *               and wbar are then not read) or 0
 *   out_idx     [B, m, topk] int32 (ascending token indices, then -1);
 *   out_score   [B, m, topk] fp32 or NULL
 *   out_bank    [B, m/G, P] int32 or NULL: the banks (ascending; rows of
 *               windows that fall back are all -1)
 * G in {4, 8, 16}, m a multiple of G and at most 64, B*m <= 65535,
 * topk <= P <= 16384, d in {64, 128}, H and Hs <= 64.
 */
int indexer_mtp(const void *q, const uint8_t *k_cache, const float *k_scale, const float *w,
                const void *qbar, const float *wbar, const int32_t *prefix_lens, int B,
                int64_t Nmax, int m, int H, int Hs, int d, int G, int P, int topk, unsigned flags,
                int32_t *out_idx, int32_t *out_bank, float *out_score, void *ws, size_t ws_bytes,
                void *stream);
/* Workspace bytes for any prefix lengths (sized for the longest rows). */
size_t indexer_mtp_workspace_size(int B, int64_t Nmax, int m, int H, int Hs, int d, int G, int P,
                                  int topk, unsigned flags);
/* Query-key scores indexer_mtp evaluates for these (host) prefix lengths and
 * flags: Eq. (21) summed over the windows.  -1 on bad arguments. */
int64_t indexer_mtp_pairs(const int32_t *prefix_lens, int B, int64_t Nmax, int m, int G, int P,
                          unsigned flags);

/*
 * The group indexer's query and gates: Section 4.2, Eq. (6)-(7) and Appendix
 * C.3.  For each complete group of G consecutive query rows (anchor position
 * t = q_pos0 + gG):
 *   cbar = W_pool [max c; min c; mean c] (element-wise over the group's rows),
 *   hbar = mean h,  qbar_j = RoPE_t([W_Q cbar]_j),  wbar_j = sigmoid([W_G hbar]_j).
 *   c       [Tq, dc] bf16: the (normalized) query latents
 *   h       [Tq, dh] bf16: the (normalized) hidden states
 *   w_pool  [dc, 3*dc] bf16;  w_q [Hs*d, dc] bf16;  w_g [Hs, dh] bf16
 *   qbar    [ceil(Tq/G), Hs, d] bf16 out;  wbar [ceil(Tq/G), Hs] fp32 out
 *           (the row of an incomplete last group is zero)
 * The rotary embedding turns the pairs (i, i + rope_dim/2), i < rope_dim/2, of
 * each head by t * rope_base^(-2i/rope_dim) (rope_dim even, <= d; 0: none).
 * Pooled values and cbar are bf16 (the products' operands; fp32 sums and
 * accumulation).  G in {4, 8, 16}; dc, dh, d multiples of 16; Hs <= 64.
 * These feed indexer_group_bank / indexer_mtp as qbar, wbar.
 */
int indexer_group_query(const void *c, const void *h, const void *w_pool, const void *w_q,
                        const void *w_g, int64_t Tq, int dc, int dh, int Hs, int d, int G,
                        int64_t q_pos0, int rope_dim, float rope_base, void *qbar, float *wbar,
                        void *ws, size_t ws_bytes, void *stream);
size_t indexer_group_query_workspace_size(int64_t Tq, int dc, int dh, int Hs, int d, int G);

/*
 * Calibration statistics for layer-wise reuse: Section 4.1, Eq. (4)-(5);
 * Appendix B.2 (capacity statistics), B.4 (coverage); Appendix A, Eq. (15)-(28)
 * (scoring counts).  Index sets are the indexer's output rows: ascending
 * token indices, then -1.
 *
 * indexer_union_sizes: out_union [T/G] int32 (device) gets, for each complete
 * group of G consecutive rows of topk_idx [T, K] (device), the size of the
 * union of their index sets (the inner term of Eq. (4)).  G <= 64, K <= 16384
 * and a multiple of 4, topk_idx 16-byte aligned.
 * indexer_topk_overlap: out_count [n] int32 (device) gets |A_i ∩ B_i| for the
 * rows of a [n, K] and b [n, K] (device); coverage is out_count / K.  K a
 * multiple of 4 and at most 16384; a 16-byte aligned.
 */
int indexer_union_sizes(const int32_t *topk_idx, int64_t T, int K, int G, int32_t *out_union,
                        void *stream);
int indexer_topk_overlap(const int32_t *a, const int32_t *b, int64_t n, int K, int32_t *out_count,
                         void *stream);
/* Host: the capacity statistic of n union sizes (host memory): stat 0 = max,
 * 1 = mean, 2 = nearest-rank 90th percentile.  -1 on bad arguments. */
double indexer_union_stat(const int32_t *sizes, int64_t n, int stat);
/* Host: the joint scoring speedup of prefill of L tokens plus R verification
 * rounds of m queries whose first query sees L + (j-1) a keys (Eq. (24),
 * (28), with Eq. (15)-(16), (19)-(21)).  -1 on bad arguments. */
double indexer_speedup_joint(double L, int G, int P, int R, int m, double a);
/* Host: Eq. (5).  stat_by_G [3] holds the union statistic for G = 4, 8, 16;
 * writes the (G, P), P in {4096, 8192, 16384}, with the largest joint speedup
 * among those with P >= the statistic of their G (the first such on equal
 * speedups), or G = P = 0 when none is feasible.  m a multiple of 16. */
int indexer_select_setting(const double *stat_by_G, double L, int R, int m, double a, int *out_G,
                           int *out_P);
/* Host: Eq. (26)-(27), joint: the speedup of a per-layer assignment (G[i],
 * P[i]; G[i] = 0 is the original indexer), from scoring counts summed over
 * the layers.  -1 on bad arguments. */
double indexer_layerwise_speedup(const int *G, const int *P, int nlayers, double L, int R, int m,
                                 double a);

/*
 * Measurement aid (not an operation of the pages): read `bytes` bytes of
 * device memory at p (16-byte aligned) once with coalesced 16-byte loads,
 * spread over nblocks workgroups (1..65535), and write one XOR checksum word
 * per workgroup to out [nblocks] (device).  Its rate is the plain HBM read
 * stream that the memory-bound kernels (the decode scan above all) are
 * compared with.
 */
int indexer_read_probe(const void *p, int64_t bytes, uint32_t *out, int nblocks, void *stream);

/*
 * Measurement aid (not an operation of the pages): the matrix-core stream.
 * nblocks workgroups (1..65535; one per CU when nblocks is at most the CU
 * count, as each holds 96 KiB of LDS) of waves_per_simd (1, 2 or 4) waves per
 * SIMD each run `iters` (>= 1) rounds of four independent MFMAs on register
 * operands, with no memory traffic in the loop: 32x32x64 E4M3 MFMAs for
 * dtype DSAIDX_FP8_E4M3 (2 * 32 * 32 * 64 * 4 * iters flops per wave) or
 * 32x32x16 bf16 MFMAs for DSAIDX_BF16 (2 * 32 * 32 * 16 * 4 * iters).  The
 * operand words are a 32-bit mix of their index (h = i * 0x9E3779B1;
 * h ^= h >> 15; h *= 0x85EBCA77; h ^= h >> 13) ANDed with operand_mask,
 * which must keep every operand a number: each byte must clear one of its
 * low seven bits (E4M3), each 16-bit half one of its exponent bits (bf16).
 * E4M3 0x37373737 gives magnitudes below 1, 0xFEFEFEFE the whole E4M3 range
 * with random signs; bf16 0xBFFFBFFF random signs and mantissas below 2 in
 * magnitude.  The sustained rate depends on the data through the chip's
 * power limit.  out [nblocks * 256 * waves_per_simd] (device) receives each
 * lane's sum of its accumulators; clocks [2 * waves] (device, waves =
 * nblocks * 4 * waves_per_simd) each wave's shader-clock count (s_memtime)
 * and 100 MHz constant-clock count (s_memrealtime) around its loop.  Its rate
 * is the sustained matrix-core ceiling the prefill kernels are compared with.
 */
int indexer_mfma_probe(int dtype, int iters, int waves_per_simd, int nblocks, uint32_t operand_mask, float *out,
                       uint64_t *clocks, void *stream);

/* Message describing the calling thread's last non-OK return ("" if none). */
const char *indexer_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_INDEXER_H */
