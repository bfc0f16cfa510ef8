"""Quest-style query-aware page selection (oracle side).

[tokendh] section "历史太长,会撑爆什么": dynamic-sparse methods keep the whole
history plus a summary index, and Quest picks KV pages per query.  [netics]
section "SparseEngine 围绕 KV cache 构建了什么" says the same: page-selection
methods choose KV pages for each query.

Readings taken where the pages are silent:
  * the per-page summary index is the elementwise min and max of the page's
    keys over its valid tokens;
  * a page's score for one query head is the upper bound
    sum_d max(q_d * min_d, q_d * max_d) of q . k over the page's keys, unscaled;
  * the score of a page for a KV head is the max of that bound over the query
    heads that read the KV head (so one view serves the whole group);
  * pages holding no valid token are not candidates; no page is forced in;
  * the view lists the top_pages best pages in ascending page order.
"""
import numpy as np

from .selection import top_k_ascending


def n_pages(length, page_size):
    return (int(length) + page_size - 1) // page_size


def page_meta(K, seq_len, page_size):
    """Per (batch, KV head, page): elementwise min and max of K over the page's valid tokens.

    K: [B][Hkv][cap][D]; seq_len: [B].  Returns (kmin, kmax) float64
    [B][Hkv][ceil(cap/P)][D]; pages with no valid token hold NaN."""
    K = np.asarray(K, dtype=np.float64)
    B, H, cap, D = K.shape
    NP = n_pages(cap, page_size)
    kmin = np.full((B, H, NP, D), np.nan)
    kmax = np.full((B, H, NP, D), np.nan)
    for b in range(B):
        L = int(seq_len[b])
        for p in range(n_pages(L, page_size)):
            rows = K[b, :, p * page_size:min((p + 1) * page_size, L), :]   # [H][t][D]
            kmin[b, :, p] = rows.min(axis=1)
            kmax[b, :, p] = rows.max(axis=1)
    return kmin, kmax


def quest_bounds(q, kmin, kmax, seq_len, page_size):
    """U [B][Hq][NP]: per query head h and page p, sum_d max(q_hd * min_pd, q_hd * max_pd);
    S [B][Hkv][NP]: max of U over the heads of the group.  Invalid pages: -inf."""
    q = np.asarray(q, dtype=np.float64)
    kmin = np.asarray(kmin, dtype=np.float64)
    kmax = np.asarray(kmax, dtype=np.float64)
    B, Hq, D = q.shape
    _, H, NP, _ = kmin.shape
    G = Hq // H
    U = np.full((B, Hq, NP), -np.inf)
    S = np.full((B, H, NP), -np.inf)
    for b in range(B):
        npv = n_pages(int(seq_len[b]), page_size)
        for h in range(Hq):
            lo = q[b, h][None, :] * kmin[b, h // G, :npv]     # [npv][D]
            hi = q[b, h][None, :] * kmax[b, h // G, :npv]
            U[b, h, :npv] = np.maximum(lo, hi).sum(axis=1)
        for kv in range(H):
            S[b, kv, :npv] = U[b, kv * G:(kv + 1) * G, :npv].max(axis=0)
    return U, S


def quest_select(q, kmin, kmax, seq_len, page_size, top_pages):
    """The Quest view: (view_idx [B][Hkv][top_pages] int32 ascending page ids, -1 padded;
    view_len [B][Hkv]; S [B][Hkv][NP] float64)."""
    _, S = quest_bounds(q, kmin, kmax, seq_len, page_size)
    B, H, NP = S.shape
    view = np.full((B, H, top_pages), -1, np.int32)
    vlen = np.zeros((B, H), np.int32)
    for b in range(B):
        npv = n_pages(int(seq_len[b]), page_size)
        for kv in range(H):
            sel = top_k_ascending(S[b, kv, :npv], top_pages)
            view[b, kv, :sel.size] = sel
            vlen[b, kv] = sel.size
    return view, vlen, S
