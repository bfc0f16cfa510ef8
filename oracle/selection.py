"""Selection rules shared by every method's view producer (oracle side).

[tokendh] section "把边界划在'生命周期'上" and [aifeeds] section 方法/关键模块:
each method's cache manager hands attention a view that exposes the chosen
positions.  The pages do not say how ties are broken or in what order the
positions are listed; the reading taken here is: larger score first, equal
scores go to the lower index, and the chosen indices are listed in ascending
order.  Scores are compared as float32 (numerically equal values, including
+0.0 and -0.0, tie).
"""
import numpy as np


def top_k_ascending(score, k, valid=None):
    """Indices of the k largest scores (ties -> lower index), ascending.

    score: 1-D array; valid: optional bool mask of candidates.  Returns an int64
    array of min(k, #candidates) indices."""
    s = np.asarray(score, dtype=np.float32).astype(np.float64)
    idx = np.arange(s.shape[0])
    if valid is not None:
        idx = idx[np.asarray(valid, bool)]
        s = s[idx]
    order = np.lexsort((idx, -s))          # primary: -score, secondary: index
    return np.sort(idx[order[:max(0, int(k))]])


def argmin_lower(score, key_for_ties, valid):
    """Index of the smallest float32 score among `valid`; ties go to the lower
    `key_for_ties` (H2O: the lower token position).  -1 when no candidate."""
    s = np.asarray(score, dtype=np.float32).astype(np.float64)
    cand = np.nonzero(np.asarray(valid, bool))[0]
    if cand.size == 0:
        return -1
    order = np.lexsort((np.asarray(key_for_ties)[cand], s[cand]))
    return int(cand[order[0]])


def boundary_gap(score, k, valid=None):
    """Relative distance, at the top-k boundary, between the k-th best score and the
    nearest different score across the boundary (inf when every candidate or none is
    kept).  When equal scores straddle the boundary, the distance to the nearest
    different score on either side.  Used to keep generated inputs clear of
    near-ties that float32 rounding could reorder."""
    s = np.asarray(score, dtype=np.float64)
    if valid is not None:
        s = s[np.asarray(valid, bool)]
    n = s.shape[0]
    if k <= 0 or k >= n:
        return np.inf
    srt = np.sort(s)[::-1]
    kth, nxt = srt[k - 1], srt[k]
    if kth != nxt:
        return float((kth - nxt) / abs(kth))
    gap = np.inf
    above, below = srt[srt > kth], srt[srt < kth]
    if above.size:
        gap = min(gap, float((above.min() - kth) / abs(kth)))
    if below.size:
        gap = min(gap, float((kth - below.max()) / abs(kth)))
    return gap


def argmin_gap(score, valid):
    """Relative distance between the smallest candidate score and the next different one."""
    s = np.sort(np.asarray(score, dtype=np.float64)[np.asarray(valid, bool)])
    if s.size < 2:
        return np.inf
    d = s[s > s[0]]
    return float((d[0] - s[0]) / abs(s[0])) if d.size else np.inf
