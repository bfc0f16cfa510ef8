"""Pins of the H2O prefill-end oracle (no GPU): every prompt query's weights sum
to one, the closed form for equal keys (harmonic sums), the last key, agreement
with the separately pinned SnapKV votes on the last W queries, a torch softmax
cross-check, and the kept-set layout of the slot state."""
import numpy as np
import torch

from oracle import h2o as oh2o
from oracle import snapkv as osnap


def rand(L, G=3, D=16, seed=0):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(G, L, D)), rng.normal(size=(L + 3, D))


def test_scores_sum_to_rows_and_last_key():
    q, K = rand(40)
    acc = oh2o.prefill_scores(q, K, 40, 0.3)
    assert abs(acc.sum() - 3 * 40) < 1e-9                     # each (head, query) row sums to one
    s = 0.3 * (q[:, 39] @ K[:40].T)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    assert abs(acc[39] - (p[:, 39] / p.sum(axis=1)).sum()) < 1e-12    # only the last query sees the last key


def test_equal_keys_closed_form():
    L, G = 25, 2
    q, _ = rand(L, G)
    K = np.tile(np.random.default_rng(1).normal(size=(1, 16)), (L, 1))
    acc = oh2o.prefill_scores(q, K, L, 0.5)
    ref = G * np.array([sum(1.0 / (i + 1) for i in range(j, L)) for j in range(L)])
    np.testing.assert_allclose(acc, ref, rtol=1e-12)


def test_last_window_part_equals_snapkv_votes():
    """Scores of the full prompt minus those of its first L - W queries are the SnapKV
    votes of the last W queries (the same causal rows), for every history key."""
    L, W, G = 48, 8, 2
    q, K = rand(L, G, seed=2)
    full = oh2o.prefill_scores(q, K, L, 0.25)
    head = oh2o.prefill_scores(q[:, :L - W], K, L - W, 0.25)
    votes = osnap.unit_votes(q[:, L - W:], K, L, W, 0.25)
    np.testing.assert_allclose(full[:L - W] - head, votes, rtol=1e-9, atol=1e-12)


def test_torch_causal_softmax_cross_check():
    L = 30
    q, K = rand(L, seed=3)
    S = torch.from_numpy(0.2 * np.einsum("gld,kd->glk", q, K[:L]))
    S = S.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
    ref = torch.softmax(S, dim=-1).sum(dim=(0, 1)).numpy()
    np.testing.assert_allclose(oh2o.prefill_scores(q, K, L, 0.2), ref, rtol=1e-12)


def test_prefill_state_layout():
    rng = np.random.default_rng(4)
    L, heavy, recent, cap = 60, 10, 8, 19
    acc0 = rng.random(L)
    kept, slot_pos, acc = oh2o.prefill_state(acc0, L, heavy, recent, cap)
    best = np.sort(np.argsort(-acc0[:L - recent], kind="stable")[:heavy])
    np.testing.assert_array_equal(kept, np.concatenate([best, np.arange(L - recent, L)]))
    np.testing.assert_array_equal(slot_pos[:heavy + recent], kept)
    assert slot_pos[-1] == -1 and acc[-1] == 0.0
    np.testing.assert_array_equal(acc[:heavy + recent], acc0[kept])
    # a prompt that fits keeps every position
    kept, slot_pos, _ = oh2o.prefill_state(acc0[:12], 12, heavy, recent, cap)
    np.testing.assert_array_equal(kept, np.arange(12))
    assert np.all(slot_pos[12:] == -1)


def test_tail_scores_equal_the_full_scores_past_j0():
    """prefill_scores_tail (the keys j0.. only, for full-size parity samples) against
    the pinned full scores, and against the harmonic closed form for equal keys."""
    L = 37
    q, K = rand(L, G=3, D=16, seed=5)
    full = oh2o.prefill_scores(q, K, L, 0.35)
    for j0 in (0, 1, 20, L - 1):
        np.testing.assert_allclose(oh2o.prefill_scores_tail(q, K, L, 0.35, j0), full[j0:], rtol=1e-12, atol=1e-15)
    G = 2
    qe, _ = rand(L, G, seed=6)
    Ke = np.tile(np.random.default_rng(7).normal(size=(1, 16)), (L, 1))
    harmonic = np.array([G * sum(1.0 / (i + 1) for i in range(j, L)) for j in range(L)])
    np.testing.assert_allclose(oh2o.prefill_scores_tail(qe, Ke, L, 0.5, 30), harmonic[30:], rtol=1e-12)
