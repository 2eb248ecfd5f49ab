"""Comparison of a GPU indexer result with the CPU oracle's.

Integer-valued inputs: every fp32 partial sum is exact, so indices and scores
must be bit-identical.  Random inputs: a selected index may differ from the
oracle's only where both scores are within rtol * |s_K| of the oracle's K-th
score s_K, and every GPU score must be within rtol * max(|s_ref|, |s_K|) of the
oracle's score of the same key.
"""
import numpy as np


def _valid(row):
    return row[row >= 0]


def compare(gpu_idx, gpu_score, ref_idx, ref_score, exact, ref_score_of=None, rtol=1e-2, label=""):
    """Raise AssertionError with the first mismatches.

    gpu_idx/gpu_score: [n, K] arrays of the GPU rows; ref_idx/ref_score: the
    oracle's rows (same order).  ref_score_of(r, keys) -> oracle scores of the
    given keys for local row r (needed only for tolerance checks).
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
            tol = rtol * abs(sK) + 1e-30
            extra = np.setdiff1d(gv, rv)
            missing = np.setdiff1d(rv, gv)
            if len(extra):
                se = ref_score_of(r, extra)
                if np.any(se < sK - tol):
                    errs.append(f"{label} row {r}: selected {extra[se < sK - tol][:5]} with oracle scores "
                                f"{se[se < sK - tol][:5]} below K-th {sK} - tol")
            if len(missing):
                sm = rs[np.searchsorted(rv, missing)]
                if np.any(sm > sK + tol):
                    errs.append(f"{label} row {r}: dropped {missing[sm > sK + tol][:5]} with oracle scores "
                                f"{sm[sm > sK + tol][:5]} above K-th {sK} + tol")
            if gpu_score is not None:
                gs = np.asarray(gpu_score[r][:len(gv)], np.float64)
                ref_g = ref_score_of(r, gv) if len(extra) else rs
                lim = rtol * np.maximum(np.abs(ref_g), abs(sK)) + 1e-30
                if np.any(np.abs(gs - ref_g) > lim):
                    b = np.nonzero(np.abs(gs - ref_g) > lim)[0][:5]
                    errs.append(f"{label} row {r}: scores off at keys {gv[b]}: gpu {gs[b]} ref {ref_g[b]}")
        if len(errs) > 8:
            break
    assert not errs, "\n".join(errs)
