"""StreamingLLM and PyramidKV kept-set rules (oracle side).

[netics] "SparseEngine 统一接入十五种稀疏注意力", section "哪些情况下加速幅度会缩小":
on AIME 2024 the paper compares StreamingLLM and PyramidKV against SnapKV and
reports their accuracy and speed-up; the pages state nothing else about them.
The readings below are the plainest forms of the two methods that fit the
pages' cache contract (a method chooses which positions it keeps and hands an
AttentionView to attention).

StreamingLLM, reading taken:
  * a unit keeps the first `sink` positions and the last `recent` positions of
    its history and attends over those only; with sink + recent >= length it
    keeps everything;
  * the kept positions are listed in ascending order (a token view).

PyramidKV, reading taken:
  * layers keep a budget that shrinks with depth along an arithmetic sequence:
    layer l of n gets b_min + (b_max - b_min) * (n - 1 - l) / (n - 1) with
    b_max = 2 * avg - b_min, so the layers' mean is the average budget `avg`;
  * budgets are whole tokens and sum to exactly n * avg: each layer takes the
    floor of its value and the remaining tokens go one each to the layers with
    the largest fractional parts (the lower layer first on equal parts);
  * inside a layer the kept set is the SnapKV rule (window plus the best pooled
    votes) with that layer's budget.
"""
from fractions import Fraction

import numpy as np


def streaming_kept(length, sink, recent):
    """Ascending positions a StreamingLLM unit of `length` tokens attends over."""
    length = int(length)
    head = list(range(min(sink, length)))
    tail = list(range(max(len(head), length - recent), length))
    return np.array(head + tail, dtype=np.int64)


def streaming_view(seq_len, n_kv_heads, sink, recent, view_cap):
    """Token view of every unit: view [B][Hkv][view_cap] int32 (-1 padded), view_len [B][Hkv]."""
    B = len(seq_len)
    view = np.full((B, n_kv_heads, view_cap), -1, np.int32)
    vlen = np.zeros((B, n_kv_heads), np.int32)
    for b in range(B):
        kept = streaming_kept(seq_len[b], sink, recent)[:view_cap]
        view[b, :, : len(kept)] = kept
        vlen[b, :] = len(kept)
    return view, vlen


def pyramid_budgets(n_layers, avg_budget, min_budget):
    """Per-layer budgets (list of ints, layer 0 first), exact rational arithmetic."""
    n, avg, bmin = int(n_layers), int(avg_budget), int(min_budget)
    assert n >= 1 and 0 <= bmin <= avg
    if n == 1:
        return [avg]
    bmax = 2 * avg - bmin
    exact = [bmin + Fraction((bmax - bmin) * (n - 1 - l), n - 1) for l in range(n)]
    base = [int(x) for x in exact]                     # floor: every value is >= 0
    left = n * avg - sum(base)
    order = sorted(range(n), key=lambda l: (-(exact[l] - base[l]), l))
    for l in order[:left]:
        base[l] += 1
    return base
