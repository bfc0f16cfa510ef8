"""Decode attention over an AttentionView (oracle side).

[tokendh] section "把边界划在'生命周期'上" and [aifeeds] section 方法/关键模块:
whatever a method keeps, attention reads it through one view format that
exposes the chosen positions, so one attention routine serves every method.

The view used here: a list of entries per (batch, KV head); each entry names
`granularity` consecutive cache slots (a page id when granularity is the page
size, a slot id when it is 1); slots at or past seq_len[b] are skipped.  No
view means every slot below seq_len[b].  Attention itself is the plain
definition: softmax(scale * q . k) over the view's slots, weights times V.
Query head h reads KV head h // G.  An empty view gives out = 0, lse = -inf.
"""
import numpy as np


def view_tokens(seq_len_b, view_row=None, view_len=None, granularity=1):
    """(slots, tokens) of one unit's view: slot = position in view order
    (entry * granularity + offset), token = cache slot it reads.  Only valid ones."""
    L = int(seq_len_b)
    if view_row is None:
        t = np.arange(L)
        return t, t
    slots, toks = [], []
    for e in range(int(view_len)):
        base = int(view_row[e]) * granularity
        for o in range(granularity):
            if 0 <= base + o < L:
                slots.append(e * granularity + o)
                toks.append(base + o)
    return np.asarray(slots, np.int64), np.asarray(toks, np.int64)


def unit_attention(qg, Kt, Vt, scale):
    """qg [G][D], Kt [n][D], Vt [n][Dv] -> (out [G][Dv], lse [G], logits [G][n]) in float64."""
    qg = np.asarray(qg, np.float64)
    Kt = np.asarray(Kt, np.float64)
    Vt = np.asarray(Vt, np.float64)
    G = qg.shape[0]
    if Kt.shape[0] == 0:
        return np.zeros((G, Vt.shape[1])), np.full(G, -np.inf), np.zeros((G, 0))
    logits = scale * (qg @ Kt.T)                            # [G][n]
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    den = w.sum(axis=1, keepdims=True)
    out = (w / den) @ Vt
    lse = (m + np.log(den))[:, 0]
    return out, lse, logits


def decode_attention(q, K, V, seq_len, scale, view_idx=None, view_len=None, granularity=1,
                     latent_dv=None, logit_cap=0):
    """q [B][Hq][Dk]; K [B][Hkv][cap][Dk]; V [B][Hkv][cap][Dv] (or None with
    latent_dv: V = K[..., :latent_dv]).  Returns out [B][Hq][Dv], lse [B][Hq] and,
    if logit_cap > 0, logits [B][Hq][logit_cap] indexed by view slot (-inf where
    the slot holds no valid token)."""
    q = np.asarray(q, np.float64)
    B, Hq, _ = q.shape
    H = K.shape[1]
    G = Hq // H
    Dv = latent_dv if V is None else V.shape[3]
    out = np.zeros((B, Hq, Dv))
    lse = np.full((B, Hq), -np.inf)
    logits = np.full((B, Hq, logit_cap), -np.inf) if logit_cap else None
    for b in range(B):
        for kv in range(H):
            if view_idx is None:
                slots, toks = view_tokens(seq_len[b])
            else:
                slots, toks = view_tokens(seq_len[b], view_idx[b][kv], view_len[b][kv], granularity)
            Kt = np.asarray(K[b, kv], np.float64)[toks]
            Vt = Kt[:, :latent_dv] if V is None else np.asarray(V[b, kv], np.float64)[toks]
            o, l, lg = unit_attention(q[b, kv * G:(kv + 1) * G], Kt, Vt, scale)
            out[b, kv * G:(kv + 1) * G] = o
            lse[b, kv * G:(kv + 1) * G] = l
            if logits is not None:
                keep = slots < logit_cap
                logits[b, kv * G:(kv + 1) * G][:, slots[keep]] = lg[:, keep]
    return out, lse, logits
