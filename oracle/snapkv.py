"""SnapKV-style prefill-end eviction (oracle side).

[tokendh] section "把边界划在'生命周期'上": at its hook SnapKV looks at how the
last few prompt tokens attend over the history, keeps the important part and
physically deletes the rest.  [tokendh] section "聊天记录也能'续命':Chain
Cache" adds that what it drops can differ from layer to layer.

Readings taken where the pages are silent:
  * the observation window is the last W prompt positions; window row (h, i)
    sits at position L - W + i and its softmax runs over every key up to and
    including its own position (causal);
  * a history position's vote is the sum of those softmax weights over the
    window rows of all query heads of the KV head;
  * votes are smoothed by a max-pool of odd width k, stride 1, positions outside
    the history ignored;
  * the window is always kept and counts in the budget: the budget - W best
    pooled votes are kept with it, ties to the lower position, and the kept
    positions are listed in ascending order;
  * with budget >= L every position is kept.
"""
import numpy as np

from .selection import top_k_ascending


def unit_votes(qg_obs, Kt, L, W, scale):
    """qg_obs [G][W][D], Kt [>=L][D] -> votes [L - W] (float64)."""
    G, W_, D = qg_obs.shape
    assert W_ == W
    Q = np.asarray(qg_obs, np.float64).reshape(G * W, D)
    Kt = np.asarray(Kt[:L], np.float64)
    logits = scale * (Q @ Kt.T)                                  # [G*W][L]
    row_pos = np.tile(np.arange(L - W, L), G)                    # position of each window row
    allowed = np.arange(L)[None, :] <= row_pos[:, None]
    logits = np.where(allowed, logits, -np.inf)
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    w /= w.sum(axis=1, keepdims=True)
    return w[:, :L - W].sum(axis=0)


def snapkv_votes(q_obs, K, L, W, scale):
    """q_obs [B][Hq][W][D], K [B][Hkv][cap][D] -> votes [B][Hkv][L - W]."""
    B, Hq = q_obs.shape[:2]
    H = K.shape[1]
    G = Hq // H
    votes = np.zeros((B, H, L - W))
    for b in range(B):
        for kv in range(H):
            votes[b, kv] = unit_votes(q_obs[b, kv * G:(kv + 1) * G], K[b, kv], L, W, scale)
    return votes


def snapkv_pool(votes, kernel):
    """pooled[j] = max(votes[j'] for |j' - j| <= kernel // 2, 0 <= j' < n), along the last axis."""
    v = np.asarray(votes, np.float64)
    n = v.shape[-1]
    r = kernel // 2
    out = np.full(v.shape, -np.inf)
    for d in range(-r, r + 1):
        lo, hi = max(0, -d), min(n, n - d)          # j in [lo, hi) has neighbour j + d in range
        if lo < hi:
            out[..., lo:hi] = np.maximum(out[..., lo:hi], v[..., lo + d:hi + d])
    return out


def snapkv_keep(pooled_row, L, W, budget):
    """Kept positions of one unit, ascending: best budget - W history positions + the window."""
    if budget >= L:
        return np.arange(L)
    top = top_k_ascending(pooled_row, budget - W)
    return np.concatenate([top, np.arange(L - W, L)])


def snapkv_compact(rows, kept):
    """Physical compaction: out[i] = rows[kept[i]] (a copy of each kept row)."""
    return np.asarray(rows)[np.asarray(kept)]


def snapkv(q_obs, K, V, L, W, kernel, budget, scale):
    """Whole eviction: (kept [B][Hkv][min(budget, L)], votes, K', V')."""
    votes = snapkv_votes(q_obs, K, L, W, scale)
    pooled = snapkv_pool(votes, kernel)
    B, H = votes.shape[:2]
    n = min(budget, L)
    kept = np.zeros((B, H, n), np.int64)
    Ko = np.zeros((B, H, n, K.shape[3]), np.asarray(K).dtype)
    Vo = np.zeros((B, H, n, V.shape[3]), np.asarray(V).dtype)
    for b in range(B):
        for kv in range(H):
            kept[b, kv] = snapkv_keep(pooled[b, kv], L, W, budget)
            Ko[b, kv] = snapkv_compact(K[b, kv], kept[b, kv])
            Vo[b, kv] = snapkv_compact(V[b, kv], kept[b, kv])
    return kept, votes, Ko, Vo
