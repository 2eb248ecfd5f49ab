"""Comparison of a GPU indexer result with the CPU oracle's.

Integer-valued inputs: every fp32 partial sum is exact, so indices and scores
must be bit-identical.  Random inputs: a selected index may differ from the
oracle's only where both scores are within rtol * |s_K| of the oracle's K-th
score s_K, and every GPU score must be within rtol * max(|s_ref|, |s_K|) of the
oracle's score of the same key (rtol = 1e-2).  Both bounds also allow the
rounding any binary32 evaluation of Eq. (1) makes: 2^-16 times the pair's
absolute condition C = sum_j |w_j| sum_c |q_jc k_c| (the forward error bound
of a floating-point sum of about d + H terms, gamma_n <= n u with u = 2^-24,
n <= 256).  That term matters only where a row's K-th score lies near zero
compared with its terms' magnitudes, where 1e-2 * |s_K| falls below what
fp32 can resolve; it is evaluated (by the oracle) only for the keys that
fail the relative bound alone.
"""
import numpy as np

ATOL_COND = 2.0 ** -16


def _valid(row):
    return row[row >= 0]


def compare(gpu_idx, gpu_score, ref_idx, ref_score, exact, ref_score_of=None, rtol=1e-2, label="",
            ref_cond_of=None):
    """Raise AssertionError with the first mismatches.

    gpu_idx/gpu_score: [n, K] arrays of the GPU rows; ref_idx/ref_score: the
    oracle's rows (same order).  ref_score_of(r, keys) -> oracle scores of the
    given keys for local row r (needed only for tolerance checks);
    ref_cond_of(r, keys) -> their absolute conditions (optional: without it
    the bounds are purely relative).
    """
    gpu_idx = np.asarray(gpu_idx)
    ref_idx = np.asarray(ref_idx)
    assert gpu_idx.shape == ref_idx.shape, (gpu_idx.shape, ref_idx.shape)
    errs = []
    for r in range(ref_idx.shape[0]):
        gi, ri = gpu_idx[r], ref_idx[r]
        if exact:
            if not np.array_equal(gi, ri):
                bad = np.nonzero(gi != ri)[0]
                errs.append(f"{label} row {r}: idx differ at {bad[:5]} gpu {gi[bad[:5]]} ref {ri[bad[:5]]}")
            elif gpu_score is not None:
                gs = np.asarray(gpu_score[r], np.float64)
                rs = np.asarray(ref_score[r], np.float64)
                if not np.array_equal(gs, rs):
                    bad = np.nonzero(gs != rs)[0]
                    errs.append(f"{label} row {r}: scores differ at {bad[:5]} gpu {gs[bad[:5]]} ref {rs[bad[:5]]}")
        else:
            gv, rv = _valid(gi), _valid(ri)
            if len(gv) != len(rv):
                errs.append(f"{label} row {r}: {len(gv)} valid entries, oracle {len(rv)}")
                continue
            if len(rv) == 0:
                continue
            if not (np.all(np.diff(gv) > 0) and np.all(gi[len(gv):] == -1)):
                errs.append(f"{label} row {r}: indices not ascending / padding wrong")
                continue
            rs = np.asarray(ref_score[r][:len(rv)], np.float64)
            sK = rs.min()
            kth = rv[np.argmin(rs)]
            tol = rtol * abs(sK) + 1e-30

            def cond(keys, r=r):
                if ref_cond_of is None or len(keys) == 0:
                    return np.zeros(len(keys))
                return np.asarray(ref_cond_of(r, np.asarray(keys)), np.float64)
            extra = np.setdiff1d(gv, rv)
            missing = np.setdiff1d(rv, gv)
            if len(extra):
                se = ref_score_of(r, extra)
                bad = se < sK - tol
                if bad.any():
                    c = cond(extra[bad]) + cond([kth])[0]
                    bad[bad] = se[bad] < sK - tol - ATOL_COND * c
                if bad.any():
                    errs.append(f"{label} row {r}: selected {extra[bad][:5]} with oracle scores "
                                f"{se[bad][:5]} below K-th {sK} - tol")
            if len(missing):
                sm = rs[np.searchsorted(rv, missing)]
                bad = sm > sK + tol
                if bad.any():
                    c = cond(missing[bad]) + cond([kth])[0]
                    bad[bad] = sm[bad] > sK + tol + ATOL_COND * c
                if bad.any():
                    errs.append(f"{label} row {r}: dropped {missing[bad][:5]} with oracle scores "
                                f"{sm[bad][:5]} above K-th {sK} + tol")
            if gpu_score is not None:
                gs = np.asarray(gpu_score[r][:len(gv)], np.float64)
                ref_g = ref_score_of(r, gv) if len(extra) else rs
                lim = rtol * np.maximum(np.abs(ref_g), abs(sK)) + 1e-30
                bad = np.abs(gs - ref_g) > lim
                if bad.any():
                    bad[bad] = np.abs(gs - ref_g)[bad] > lim[bad] + ATOL_COND * cond(gv[bad])
                if bad.any():
                    b = np.nonzero(bad)[0][:5]
                    errs.append(f"{label} row {r}: scores off at keys {gv[b]}: gpu {gs[b]} ref {ref_g[b]}")
        if len(errs) > 8:
            break
    assert not errs, "\n".join(errs)


def pair_refs(q, k, w, rows, q_dtype, k_dtype, q_scale=None, k_scale=None, key_of=None):
    """(score_of, cond_of) for compare(): the oracle's Eq. (1) scores and
    absolute conditions of the pairs (query row rows[r], key) for local row r.
    key_of(r, keys) maps a row's key indices to rows of k (a flattened decode
    cache); by default they are rows of k as they are."""
    import oracle

    def args(r, keys):
        keys = np.asarray(keys, np.int64)
        kk = keys if key_of is None else key_of(r, keys)
        return (q, k, w, np.full(len(keys), rows[r]), kk, q_dtype, k_dtype, q_scale, k_scale)

    def score_of(r, keys):
        return oracle.score_pairs(*args(r, keys))

    def cond_of(r, keys):
        return oracle.score_pairs_cond(*args(r, keys))
    return score_of, cond_of


def refine_over_bank(h, bank, rows, G, K, dt="bf16"):
    """Eq. (14) for the given query rows over the given banks (one row of
    `bank` per group of G): the candidates are the row's group bank and the
    keys after the anchor up to the row, scored one pair at a time by the
    oracle and ranked by a full lexsort.  h holds host q, k, w (and E4M3
    scales).  Returns (idx [n, K], score [n, K])."""
    import oracle
    from tests.bruteforce import lexsort_topk
    out_i = np.empty((len(rows), K), np.int32)
    out_s = np.empty((len(rows), K))
    for n, r in enumerate(rows):
        g = r // G
        cand = np.concatenate([bank[g][bank[g] >= 0], np.arange(g * G + 1, r + 1)])
        sc = oracle.score_pairs(h["q"], h["k"], h["w"], np.full(len(cand), r), cand, dt, dt, h.get("q_scale"),
                                h.get("k_scale"))
        full = np.full((1, r + 1), -np.inf)
        full[0, cand] = sc
        valid = np.zeros((1, r + 1), bool)
        valid[0, cand] = True
        i, s_ = lexsort_topk(full, valid, K)
        out_i[n], out_s[n] = i[0], s_[0]
    return out_i, out_s
