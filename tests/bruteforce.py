"""Brute-force checker for tiny inputs (numpy): the full causal score matrix,
then a full lexicographic sort of every row.  Used only by the tests."""
import numpy as np


def lexsort_topk(scores: np.ndarray, valid: np.ndarray, K: int):
    """Per row: rank valid entries by (score desc, index asc), keep min(K, #valid),
    return (idx [n,K] ascending then -1, score [n,K] with -inf padding)."""
    n, m = scores.shape
    out_i = np.full((n, K), -1, np.int32)
    out_s = np.full((n, K), -np.inf)
    cols = np.arange(m)
    for r in range(n):
        c = cols[valid[r]]
        s = scores[r, valid[r]]
        order = np.lexsort((c, -s))[:K]
        keep = np.sort(c[order])
        out_i[r, :len(keep)] = keep
        out_s[r, :len(keep)] = scores[r, keep]
    return out_i, out_s
