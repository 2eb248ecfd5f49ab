"""Oracle for the calibration statistics of layer-wise reuse (TEST
INFRASTRUCTURE ONLY: only tests, the smoke check and the benchmark's CPU leg
use it).  Plain numpy over the same index sets the GPU path reads.

"ADIndex: Layer-Adaptive Sparse Attention Indexing via Group-Level
Distillation" (Qi et al.):

- Section 4.1, Eq. (4): the union size |U_{r<G} T_{t+r}| of the reference
  top-K index sets of each group of G consecutive queries (anchor t), and its
  maximum over the valid anchors; Appendix B.2 also uses the mean and the 90th
  percentile of these sizes.
- Section 4.1, Eq. (5): among G in {4, 8, 16}, P in {4K, 8K, 16K}, pick the
  setting with the largest joint scoring speedup at L = 128K whose P is at
  least the statistic for its G.
- Appendix A.5, Eq. (26)-(27): the speedup of a per-layer assignment of
  settings, from scoring counts summed over layers.
- Coverage (Appendix B.4, Figure 4): the fraction of a query's reference
  top-K that a reuse result keeps.

Readings where the pages are silent: an empty index slot is -1 and counts for
nothing; anchors are the starts of complete groups of the given rows; the 90th
percentile is the nearest-rank one (the smallest size that at least 90% of the
anchors do not exceed); equal speedups keep the first setting in (G, P)
order; with no feasible setting the layer gets none (the original indexer).
"""
from __future__ import annotations

import math

import numpy as np

from . import cost_mtp_base_round, cost_mtp_reuse_round, cost_prefill_base, cost_prefill_reuse

SETTINGS = [(G, P) for G in (4, 8, 16) for P in (4096, 8192, 16384)]


def union_sizes(idx, G):
    """Eq. (4), inner term, for every complete group of G consecutive rows."""
    idx = np.asarray(idx)
    out = np.empty(idx.shape[0] // G, np.int64)
    for g in range(len(out)):
        s = idx[g * G:(g + 1) * G].ravel()
        out[g] = len(np.unique(s[s >= 0]))
    return out


def union_stat(sizes, stat="max"):
    """The capacity statistic of Appendix B.2: 'max', 'mean' or 'p90'."""
    s = np.sort(np.asarray(sizes, np.int64))
    if stat == "max":
        return float(s[-1])
    if stat == "mean":
        return float(s.mean())
    if stat == "p90":
        return float(s[math.ceil(0.9 * len(s)) - 1])
    raise ValueError(stat)


def overlap_counts(a, b):
    """|A_i intersect B_i| per row of two index-set arrays (-1 slots ignored)."""
    a, b = np.asarray(a), np.asarray(b)
    return np.array([len(np.intersect1d(x[x >= 0], y[y >= 0])) for x, y in zip(a, b)], np.int64)


def _cost_joint(L, G, P, R, m, a):
    """Reuse and baseline scoring counts of prefill plus R MTP rounds (Eq. (24), (28))."""
    base = cost_prefill_base(L) + sum(cost_mtp_base_round(L + j * a, m) for j in range(R))
    if G is None:
        return base, base
    reuse = cost_prefill_reuse(L, G, P) + sum(cost_mtp_reuse_round(L + j * a, G, P, m) for j in range(R))
    return base, reuse


def select_setting(stat_by_G, L=131072, R=32, m=16, a=8):
    """Eq. (5): the feasible (G, P) with the largest joint speedup, or None."""
    best, best_s = None, -1.0
    for G, P in SETTINGS:
        if stat_by_G[G] > P:
            continue
        base, reuse = _cost_joint(L, G, P, R, m, a)
        if base / reuse > best_s:
            best, best_s = (G, P), base / reuse
    return best


def layerwise_speedup(settings, L, R=32, m=16, a=8):
    """Eq. (27), x = joint: |layers| * C_base / sum over layers of C_reuse
    (a layer whose setting is None runs the original indexer)."""
    tot_base = tot_reuse = 0.0
    for s in settings:
        base, reuse = _cost_joint(L, *(s if s is not None else (None, None)), R, m, a)
        tot_base += base
        tot_reuse += reuse
    return tot_base / tot_reuse
