"""H2O-style running-score eviction (oracle side).

[tokendh] section "历史太长,会撑爆什么": H2O keeps a continuously accumulated
table of attention scores and physically deletes entries from memory.
[tokendh] section "把边界划在'生命周期'上": at every decode step it first
updates the accumulated scores and then decides what to delete.

Readings taken where the pages are silent:
  * one table per (batch, KV head): a slot's score grows by the softmax weight
    every query head of the group gives it at this step;
  * step order: the new token is written into the free slot, attention runs
    over every occupied slot (the new one included), the scores are
    accumulated (the new token starts from 0), and then, if more than
    heavy + recent slots are occupied, exactly one is evicted;
  * the recent window protects the newest `recent` positions
    (position > cur_pos - recent); among the rest the lowest score goes,
    ties to the lower position;
  * the evicted slot is freed (position -1, score 0) and receives the next token.
"""
import numpy as np

from .attention import unit_attention
from .selection import argmin_gap, argmin_lower


def h2o_accumulate_evict(logits, lse, slot_pos, acc, n_slots, cur_pos, new_slot, heavy, recent, gap_out=None):
    """One unit.  logits [G][>=n_slots] and lse [G] from attention over slots [0, n_slots);
    slot_pos [cap] int (-1 free), acc [cap] float64; new_slot = slot holding cur_pos.
    Returns (slot_pos', acc', evicted slot or -1).  If gap_out is a list, the relative
    gap of the eviction decision (argmin_gap) is appended to it."""
    slot_pos = np.array(slot_pos, np.int64)
    acc = np.array(acc, np.float64)
    slot_pos[new_slot] = cur_pos
    acc[new_slot] = 0.0
    n = int(n_slots)
    occupied = slot_pos[:n] >= 0
    p = np.exp(np.asarray(logits, np.float64)[:, :n] - np.asarray(lse, np.float64)[:, None])   # [G][n]
    acc[:n] += np.where(occupied, p.sum(axis=0), 0.0)
    if int((slot_pos >= 0).sum()) <= heavy + recent:
        return slot_pos, acc, -1
    cand = np.zeros(slot_pos.shape[0], bool)
    cand[:n] = occupied & (slot_pos[:n] <= cur_pos - recent)
    ev = argmin_lower(acc, slot_pos, cand)
    if gap_out is not None:
        gap_out.append(argmin_gap(acc, cand))
    if ev >= 0:
        slot_pos[ev] = -1
        acc[ev] = 0.0
    return slot_pos, acc, ev


def h2o_step(Kslots, Vslots, slot_pos, acc, n_slots, free_slot, qg, k_new, v_new, cur_pos,
             heavy, recent, scale, gap_out=None):
    """One decode step of one unit.  Kslots [cap][D], Vslots [cap][Dv] are updated in place.
    free_slot: slot to write the new token into (-1: append at n_slots).
    Returns (out [G][Dv], lse [G], slot_pos', acc', n_slots', evicted)."""
    slot = free_slot if free_slot >= 0 else n_slots
    if free_slot < 0:
        n_slots += 1
    Kslots[slot] = k_new
    Vslots[slot] = v_new
    out, lse, logits = unit_attention(qg, Kslots[:n_slots], Vslots[:n_slots], scale)
    slot_pos, acc, ev = h2o_accumulate_evict(logits, lse, slot_pos, acc, n_slots, cur_pos, slot, heavy, recent,
                                             gap_out)
    return out, lse, slot_pos, acc, n_slots, ev


def prefill_scores(qg, Kt, L, scale):
    """H2O scores after a prefill of L tokens, one unit: qg [G][L][D] (every prompt
    query of the group's heads), Kt [>=L][D].  acc0[j] = sum over heads and over the
    queries i >= j of the causal softmax weight of key j (float64, [L]).

    [tokendh] sections "历史太长,会撑爆什么" / "把边界划在'生命周期'上": H2O's table
    accumulates the attention every token receives; at the end of the prefill that
    is the attention of every prompt query (reading: causal, summed over the
    group's heads, all prompt queries included)."""
    qg = np.asarray(qg, np.float64)
    Kt = np.asarray(Kt, np.float64)[:L]
    acc = np.zeros(L)
    for h in range(qg.shape[0]):
        S = scale * (qg[h, :L] @ Kt.T)                     # [L queries][L keys]
        S[np.triu_indices(L, 1)] = -np.inf                 # causal: key <= query
        m = S.max(axis=1, keepdims=True)
        P = np.exp(S - m)
        P /= P.sum(axis=1, keepdims=True)
        acc += P.sum(axis=0)
    return acc


def prefill_scores_tail(qg, Kt, L, scale, j0):
    """acc0[j] of prefill_scores for the keys j0 <= j < L only, one unit (float64,
    [L - j0]): the same definition restricted to them.  Key j receives weight only
    from the queries i >= j, so only the rows i >= j0 are formed, each softmax
    still running over all of its keys 0..i."""
    qg = np.asarray(qg, np.float64)
    Kt = np.asarray(Kt, np.float64)[:L]
    acc = np.zeros(L - j0)
    for h in range(qg.shape[0]):
        for i in range(j0, L):
            s = scale * (Kt[:i + 1] @ qg[h, i])            # keys 0..i of query i
            p = np.exp(s - s.max())
            p /= p.sum()
            acc[:i + 1 - j0] += p[j0:]
    return acc


def prefill_state(acc0, L, heavy, recent, cap):
    """Slot state after the prefill (reading: the SnapKV-style keep rule on the scores,
    no pooling): the `heavy` best positions below L - recent (ties to the lower
    position) and the recent window, ascending, in slots 0..; slot_pos -1 and score 0
    for the remaining slots.  Returns (kept positions, slot_pos [cap], acc [cap])."""
    from .snapkv import snapkv_keep
    kept = snapkv_keep(np.asarray(acc0[:L - recent], np.float64), L, recent, heavy + recent)
    slot_pos = np.full(cap, -1, np.int64)
    acc = np.zeros(cap)
    slot_pos[:len(kept)] = kept
    acc[:len(kept)] = np.asarray(acc0, np.float64)[kept]
    return kept, slot_pos, acc

