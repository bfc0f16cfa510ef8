"""Pins of the CPU oracle to things other than itself: library routines,
closed forms, invariants and brute force on tiny inputs.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from oracle import h2o as oh2o
from oracle import omnikv as oomni
from oracle import quest as oquest
from oracle import snapkv as osnap
from workloads import generator as gen


def grid(rng, *shape):
    return np.clip(np.rint(rng.standard_normal(shape) * 32), -255, 255) / 32


# ------------------------------------------------------------------ selection rule

def test_top_k_matches_python_sort_and_ties_go_low():
    rng = np.random.default_rng(0)
    for trial in range(50):
        n = rng.integers(1, 40)
        s = rng.integers(-3, 4, size=n).astype(np.float64)      # many exact ties
        k = int(rng.integers(0, n + 3))
        got = oracle.top_k_ascending(s, k)
        brute = sorted(sorted(range(n), key=lambda i: (-s[i], i))[:k])
        assert list(got) == brute


def test_top_k_signed_zero_ties_and_mask():
    s = np.array([0.0, -0.0, 1.0, -0.0, 0.0])
    assert list(oracle.top_k_ascending(s, 3)) == [0, 1, 2]
    valid = np.array([False, True, True, True, False])
    assert list(oracle.top_k_ascending(s, 2, valid)) == [1, 2]


def test_argmin_lower_ties_by_key():
    acc = np.array([3.0, 1.0, 1.0, 0.5, 2.0])
    pos = np.array([10, 7, 3, 99, 1])
    assert oracle.argmin_lower(acc, pos, [True, True, True, False, True]) == 2
    assert oracle.argmin_lower(acc, pos, [False] * 5) == -1


# ------------------------------------------------------------------ O1 page metadata

def test_page_meta_brute_force_with_partial_pages():
    rng = np.random.default_rng(1)
    B, H, cap, D, P = 2, 3, 37, 5, 8
    K = grid(rng, B, H, cap, D)
    seq = np.array([37, 19])
    kmin, kmax = oquest.page_meta(K, seq, P)
    for b in range(B):
        for h in range(H):
            for p in range(kmin.shape[2]):
                toks = [t for t in range(p * P, (p + 1) * P) if t < seq[b]]
                for d in range(D):
                    if toks:
                        assert kmin[b, h, p, d] == min(K[b, h, t, d] for t in toks)
                        assert kmax[b, h, p, d] == max(K[b, h, t, d] for t in toks)
                    else:
                        assert math.isnan(kmin[b, h, p, d]) and math.isnan(kmax[b, h, p, d])


# ------------------------------------------------------------------ O2 Quest bound and selection

def test_quest_bound_is_an_upper_bound_and_group_max():
    rng = np.random.default_rng(2)
    B, Hq, H, D, P, L = 2, 6, 2, 16, 4, 30
    K = grid(rng, B, H, L, D)
    q = grid(rng, B, Hq, D)
    seq = np.array([30, 23])
    kmin, kmax = oquest.page_meta(K, seq, P)
    U, S = oquest.quest_bounds(q, kmin, kmax, seq, P)
    G = Hq // H
    for b in range(B):
        for h in range(Hq):
            for p in range(oquest.n_pages(seq[b], P)):
                toks = range(p * P, min((p + 1) * P, seq[b]))
                true_max = max(float(q[b, h] @ K[b, h // G, t]) for t in toks)
                assert U[b, h, p] >= true_max             # exact on grid values
        for kv in range(H):
            np.testing.assert_array_equal(S[b, kv], U[b, kv * G:(kv + 1) * G].max(axis=0))
        assert np.all(np.isneginf(S[b, :, oquest.n_pages(seq[b], P):]))


def test_quest_bound_tight_for_single_token_pages_and_constant_pages():
    rng = np.random.default_rng(3)
    B, H, D, L = 1, 1, 12, 9
    K = grid(rng, B, H, L, D)
    q = grid(rng, B, 1, D)
    U, _ = oquest.quest_bounds(q, *oquest.page_meta(K, [L], 1), [L], 1)
    np.testing.assert_array_equal(U[0, 0], K[0, 0] @ q[0, 0])          # page of one token: bound = q.k
    Kc = np.repeat(K[:, :, :1], 8, axis=2)                             # every key of a page equal
    U2, _ = oquest.quest_bounds(q, *oquest.page_meta(Kc, [8], 4), [8], 4)
    np.testing.assert_array_equal(U2[0, 0], [K[0, 0, 0] @ q[0, 0]] * 2)


def test_quest_bound_attained_by_extreme_token():
    # A page where one token holds the max in dims with q > 0 and the min in dims with q < 0:
    # the bound equals that token's dot product exactly.
    D = 10
    rng = np.random.default_rng(4)
    q = grid(rng, D)
    other = grid(rng, 3, D)
    star = np.where(q >= 0, other.max(axis=0) + 1, other.min(axis=0) - 1)
    K = np.concatenate([other, star[None]], 0)[None, None]
    U, _ = oquest.quest_bounds(q[None, None], *oquest.page_meta(K, [4], 4), [4], 4)
    assert U[0, 0, 0] == star @ q


def test_quest_select_page1_equals_exact_topk_of_group_max():
    rng = np.random.default_rng(5)
    B, Hq, H, D, L, k = 2, 4, 2, 8, 40, 7
    K = grid(rng, B, H, L, D)
    q = grid(rng, B, Hq, D)
    seq = np.array([40, 33])
    view, vlen, _ = oquest.quest_select(q, *oquest.page_meta(K, seq, 1), seq, 1, k)
    for b in range(B):
        for kv in range(H):
            s = [max(float(q[b, h] @ K[b, kv, t]) for h in range(kv * 2, kv * 2 + 2)) for t in range(seq[b])]
            brute = sorted(sorted(range(seq[b]), key=lambda t: (-s[t], t))[:k])
            assert vlen[b, kv] == k and list(view[b, kv, :k]) == brute


def test_quest_select_all_pages_when_k_exceeds():
    rng = np.random.default_rng(6)
    K = grid(rng, 1, 1, 50, 4)
    q = grid(rng, 1, 2, 4)
    view, vlen, _ = oquest.quest_select(q, *oquest.page_meta(K, [50], 16), [50], 16, 10)
    assert vlen[0, 0] == 4 and list(view[0, 0]) == [0, 1, 2, 3] + [-1] * 6


# ------------------------------------------------------------------ O3 attention

def _sdpa(q, K, V, scale):
    """torch's fp64 scaled_dot_product_attention on CPU, KV heads repeated per group."""
    B, Hq, D = q.shape
    G = Hq // K.shape[1]
    qt = torch.from_numpy(np.asarray(q, np.float64))[:, :, None, :]
    Kt = torch.from_numpy(np.asarray(K, np.float64)).repeat_interleave(G, dim=1)
    Vt = torch.from_numpy(np.asarray(V, np.float64)).repeat_interleave(G, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)[:, :, 0].numpy()


def test_attention_dense_matches_torch_sdpa():
    rng = np.random.default_rng(7)
    B, Hq, H, D, Dv, L = 2, 8, 2, 16, 12, 45
    q, K, V = grid(rng, B, Hq, D), grid(rng, B, H, L, D), grid(rng, B, H, L, Dv)
    out, lse, logits = oatt.decode_attention(q, K, V, [L, L], 0.3, logit_cap=L)
    np.testing.assert_allclose(out, _sdpa(q, K, V, 0.3), rtol=0, atol=1e-12)
    ref_lse = np.log(np.exp(logits).sum(-1))
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13)


def test_attention_page_view_of_all_pages_equals_dense_and_order_free():
    rng = np.random.default_rng(8)
    B, Hq, H, D, L, P = 1, 4, 1, 8, 37, 8
    q, K, V = grid(rng, B, Hq, D), grid(rng, B, H, 40, D), grid(rng, B, H, 40, D)
    dense, dl, _ = oatt.decode_attention(q, K, V, [L], 0.25)
    view = np.array([[[0, 1, 2, 3, 4]]])
    sp, sl, _ = oatt.decode_attention(q, K, V, [L], 0.25, view, [[5]], P)
    np.testing.assert_allclose(sp, dense, atol=1e-13)
    perm = np.array([[[3, 0, 4, 2, 1]]])
    sp2, _, _ = oatt.decode_attention(q, K, V, [L], 0.25, perm, [[5]], P)
    np.testing.assert_allclose(sp2, dense, atol=1e-13)
    # a subset view equals sdpa restricted to the subset's tokens
    sub = np.array([[[1, 3]]])
    o3, _, _ = oatt.decode_attention(q, K, V, [L], 0.25, sub, [[2]], P)
    toks = list(range(8, 16)) + list(range(24, 32))
    np.testing.assert_allclose(o3, _sdpa(q, K[:, :, toks], V[:, :, toks], 0.25), atol=1e-12)


def test_attention_degenerate_views():
    rng = np.random.default_rng(9)
    q, K, V = grid(rng, 1, 2, 4), grid(rng, 1, 1, 10, 4), grid(rng, 1, 1, 10, 3)
    out, lse, _ = oatt.decode_attention(q, K, V, [10], 1.0, np.array([[[0]]]), [[0]], 1)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    out, lse, _ = oatt.decode_attention(q, K, V, [10], 1.0, np.array([[[6]]]), [[1]], 1)
    np.testing.assert_array_equal(out[0], np.repeat(V[0, 0, 6][None], 2, 0))
    np.testing.assert_allclose(lse[0], q[0] @ K[0, 0, 6], rtol=1e-15)
    # pages past seq_len are skipped
    out, lse, _ = oatt.decode_attention(q, K, V, [3], 1.0, np.array([[[0, 1]]]), [[2]], 2)
    ref, _, _ = oatt.decode_attention(q, K, V, [3], 1.0)
    np.testing.assert_allclose(out, ref, atol=1e-14)
    # equal keys: output is the mean of the values
    Ke = np.repeat(K[:, :, :1], 10, axis=2)
    out, _, _ = oatt.decode_attention(q, Ke, V, [10], 1.0)
    np.testing.assert_allclose(out[0], np.repeat(V[0, 0].mean(0)[None], 2, 0), atol=1e-14)


def test_attention_latent_alias_equals_explicit_values():
    rng = np.random.default_rng(10)
    q, C = grid(rng, 2, 4, 9), grid(rng, 2, 1, 20, 9)
    a, la, _ = oatt.decode_attention(q, C, None, [20, 17], 0.5, latent_dv=6)
    b, lb, _ = oatt.decode_attention(q, C, C[..., :6].copy(), [20, 17], 0.5)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


# ------------------------------------------------------------------ O4 SnapKV

def test_snapkv_pool_matches_torch_max_pool1d():
    rng = np.random.default_rng(11)
    v = rng.random((3, 2, 50))
    ref = torch.nn.functional.max_pool1d(torch.from_numpy(v), 7, stride=1, padding=3).numpy()
    np.testing.assert_array_equal(osnap.snapkv_pool(v, 7), ref)
    np.testing.assert_array_equal(osnap.snapkv_pool(v, 1), v)


def test_snapkv_votes_brute_force_tiny():
    rng = np.random.default_rng(12)
    G, W, L, D, s = 2, 3, 9, 4, 0.7
    qo, K = grid(rng, G, W, D), grid(rng, L, D)
    votes = osnap.unit_votes(qo, K, L, W, s)
    brute = [0.0] * (L - W)
    for h in range(G):
        for i in range(W):
            pos = L - W + i
            lg = [s * sum(qo[h, i, d] * K[j, d] for d in range(D)) for j in range(pos + 1)]
            z = sum(math.exp(x) for x in lg)
            for j in range(L - W):
                brute[j] += math.exp(lg[j]) / z
    np.testing.assert_allclose(votes, brute, rtol=1e-12)


def test_snapkv_votes_closed_form_equal_keys():
    # With all keys equal each causal row is uniform over its pos + 1 keys.
    G, W, L, D = 3, 4, 20, 5
    K = np.ones((L, D)) * 0.5
    qo = grid(np.random.default_rng(13), G, W, D)
    votes = osnap.unit_votes(qo, K, L, W, 1.0)
    expect = G * sum(1.0 / (L - W + i + 1) for i in range(W))
    np.testing.assert_allclose(votes, np.full(L - W, expect), rtol=1e-13)


def test_snapkv_votes_are_causal():
    rng = np.random.default_rng(14)
    G, W, L, D = 1, 2, 10, 4
    qo, K = grid(rng, G, W, D), grid(rng, L, D)
    K2 = K.copy()
    K2[L - 1] += 3.0          # only the last window row sees the last key
    v1 = osnap.unit_votes(qo[:, :1], K, L - 1, 1, 1.0)
    v2 = osnap.unit_votes(qo[:, :1], K2, L - 1, 1, 1.0)
    np.testing.assert_array_equal(v1, v2)
    assert not np.allclose(osnap.unit_votes(qo, K, L, W, 1.0), osnap.unit_votes(qo, K2, L, W, 1.0))


def test_snapkv_keep_invariants_and_identity():
    rng = np.random.default_rng(15)
    L, W, budget = 60, 6, 20
    pooled = osnap.snapkv_pool(rng.random(L - W), 7)
    kept = osnap.snapkv_keep(pooled, L, W, budget)
    assert kept.size == budget and np.all(np.diff(kept) > 0)
    assert set(range(L - W, L)) <= set(kept.tolist())
    hist = kept[kept < L - W]
    brute = sorted(sorted(range(L - W), key=lambda j: (-np.float32(pooled[j]), j))[:budget - W])
    assert hist.tolist() == brute
    np.testing.assert_array_equal(osnap.snapkv_keep(pooled, L, W, L), np.arange(L))
    np.testing.assert_array_equal(osnap.snapkv_keep(pooled, L, W, L + 5), np.arange(L))


def test_snapkv_compaction_copies_rows():
    rng = np.random.default_rng(16)
    B, Hq, H, W, L, D = 1, 2, 1, 4, 30, 6
    K, V, qo = grid(rng, B, H, L, D), grid(rng, B, H, L, D), grid(rng, B, Hq, W, D)
    kept, votes, Ko, Vo = osnap.snapkv(qo, K, V, L, W, 3, 12, 0.5)
    assert votes.shape == (1, 1, L - W)
    np.testing.assert_array_equal(Ko[0, 0], K[0, 0, kept[0, 0]])
    np.testing.assert_array_equal(Vo[0, 0], V[0, 0, kept[0, 0]])


# ------------------------------------------------------------------ O5 H2O

def _h2o_run(steps, G=2, D=4, L=24, heavy=6, recent=4, seed=17, equal_keys=False):
    rng = np.random.default_rng(seed)
    cap = heavy + recent + 1
    Ks, Vs = grid(rng, cap, D), grid(rng, cap, D)
    if equal_keys:
        Ks[:] = 0.25
    pos = np.full(cap, -1)
    pos[:heavy + recent] = np.sort(rng.choice(L, heavy + recent, replace=False))
    pos[heavy:heavy + recent] = np.arange(L - recent, L)
    pos[:heavy] = np.sort(rng.choice(L - recent, heavy, replace=False))
    acc = rng.random(cap) * G
    acc[cap - 1] = 0
    n, free, log = cap - 1, -1, []
    for t in range(steps):
        qg, kn, vn = grid(rng, G, D), grid(rng, D), grid(rng, D)
        if equal_keys:
            kn[:] = 0.25
        before = acc.copy()
        out, lse, pos, acc, n, ev = oh2o.h2o_step(Ks, Vs, pos, acc, n, free, qg, kn, vn, L + t,
                                                  heavy, recent, 0.5)
        log.append((before, acc.copy(), pos.copy(), ev, n, L + t))
        free = ev
    return log


def test_h2o_invariants():
    heavy, recent = 6, 4
    for before, after, pos, ev, n, t in _h2o_run(30, heavy=heavy, recent=recent):
        assert (pos >= 0).sum() == heavy + recent
        assert ev >= 0
        assert set(range(t - recent + 1, t + 1)) <= set(pos.tolist())      # newest positions kept
        # the evicted slot had the lowest score among the candidates
        assert pos[ev] == -1 and after[ev] == 0


def test_h2o_increment_sums_to_group_size():
    rng = np.random.default_rng(18)
    G, n = 3, 7
    logits = grid(rng, G, n)
    lse = np.log(np.exp(logits).sum(1))
    pos = np.arange(n)
    acc = np.zeros(n)
    pos2, acc2, ev = oh2o.h2o_accumulate_evict(logits, lse, pos, acc, n, n - 1, n - 1, 10, 5)
    assert ev == -1                         # 7 <= 15 occupied: nothing evicted
    np.testing.assert_allclose(acc2.sum(), G, rtol=1e-14)


def test_h2o_equal_keys_closed_form():
    # Equal keys: every occupied slot gets G / n per step; the oldest candidate with the
    # lowest score is evicted.
    log = _h2o_run(3, equal_keys=True)
    before, after, pos, ev, n, t = log[0]
    G = 2
    inc = after + (pos < 0) * 0
    occupied = pos >= 0
    changed = [s for s in range(n) if occupied[s] and s != np.argmax(pos)]
    np.testing.assert_allclose(after[changed] - before[changed], G / n, rtol=1e-13)


def test_h2o_brute_force_tiny():
    rng = np.random.default_rng(19)
    G, D, heavy, recent, L = 2, 3, 3, 2, 10
    cap = heavy + recent + 1
    Ks, Vs = grid(rng, cap, D), grid(rng, cap, D)
    pos = np.array([1, 4, 6, 8, 9, -1])
    acc = np.array([0.5, 1.5, 0.25, 1.0, 1.0, 0.0])
    # brute force: dict position -> (k, v, score)
    mem = {int(p): [Ks[s].copy(), Vs[s].copy(), float(acc[s])] for s, p in enumerate(pos) if p >= 0}
    n, free = cap - 1, -1
    for t in range(L, L + 6):
        qg, kn, vn = grid(rng, G, D), grid(rng, D), grid(rng, D)
        out, lse, pos, acc, n, ev = oh2o.h2o_step(Ks, Vs, pos, acc, n, free, qg, kn, vn, t, heavy, recent, 1.0)
        free = ev
        mem[t] = [kn, vn, 0.0]
        keys = sorted(mem)
        for h in range(G):
            lg = {p: float(qg[h] @ mem[p][0]) for p in keys}
            z = sum(math.exp(x) for x in lg.values())
            for p in keys:
                mem[p][2] += math.exp(lg[p]) / z
        if len(mem) > heavy + recent:
            cands = [p for p in keys if p <= t - recent]
            victim = min(cands, key=lambda p: (np.float32(mem[p][2]), p))
            del mem[victim]
        assert sorted(mem) == sorted(int(p) for p in pos if p >= 0)
        for s, p in enumerate(pos):
            if p >= 0:
                assert abs(acc[s] - mem[int(p)][2]) < 1e-12


# ------------------------------------------------------------------ O6 OmniKV

def test_omnikv_plan():
    plan = oomni.omnikv_layer_views(6, (1, 3))
    assert plan == [("dense", None), ("filter", None), ("sparse", 1), ("filter", None), ("sparse", 3), ("sparse", 3)]
    plan48 = oomni.omnikv_layer_views(48, (2, 8, 16))
    assert sum(m != "sparse" for m, _ in plan48) == 5 and plan48[47] == ("sparse", 16)


def _omni_unit(seed, n_layers=6, G=2, D=4, n=30):
    rng = np.random.default_rng(seed)
    return ([grid(rng, G, D) for _ in range(n_layers)], [grid(rng, n, D) for _ in range(n_layers)],
            [grid(rng, n, D) for _ in range(n_layers)])


def test_omnikv_full_budget_equals_dense_and_filter_is_dense():
    qs, Ks, Vs = _omni_unit(20)
    outs, views = oomni.unit_sweep(qs, Ks, Vs, 30, (1, 3), 30, 0.5)
    outs_small, _ = oomni.unit_sweep(qs, Ks, Vs, 30, (1, 3), 5, 0.5)
    for layer in range(6):
        dense, _, _ = oatt.unit_attention(qs[layer], Ks[layer], Vs[layer], 0.5)
        np.testing.assert_allclose(outs[layer], dense, atol=1e-13)
        if layer in (0, 1, 3):
            np.testing.assert_allclose(outs_small[layer], dense, atol=1e-13)
    assert list(views[1]) == list(range(30))


def test_omnikv_brute_force_views():
    qs, Ks, Vs = _omni_unit(21)
    outs, views = oomni.unit_sweep(qs, Ks, Vs, 30, (1, 3), 7, 0.5)
    for f in (1, 3):
        sc = [0.0] * 30
        for h in range(2):
            lg = [0.5 * float(qs[f][h] @ Ks[f][j]) for j in range(30)]
            z = sum(math.exp(x) for x in lg)
            for j in range(30):
                sc[j] += math.exp(lg[j]) / z
        assert abs(sum(sc) - 2.0) < 1e-12
        brute = sorted(sorted(range(30), key=lambda j: (-np.float32(sc[j]), j))[:7])
        assert list(views[f]) == brute
    # layer 4 attends only over the filter-3 view
    toks = views[3]
    ref, _, _ = oatt.unit_attention(qs[4], Ks[4][toks], Vs[4][toks], 0.5)
    np.testing.assert_allclose(outs[4], ref, atol=1e-14)


# ------------------------------------------------------------------ generator preconditions

def test_generator_values_are_grid_and_bf16_exact():
    from workloads import get_config
    cfg = get_config(1)
    k, v = gen.unit_kv(cfg, 0, 3, length=4096)
    for x in (k, v, gen.unit_query(cfg, 0, 0, 3)):
        assert np.all(np.abs(x) <= 255 / 32)
        np.testing.assert_array_equal(x * 32, np.rint(x * 32))
        np.testing.assert_array_equal(torch.from_numpy(x).to(torch.bfloat16).float().numpy(), x)
    k2, _ = gen.unit_kv(cfg, 0, 3, length=4096)
    np.testing.assert_array_equal(k, k2)
    # planted pages are present in the first 2048 pages
    pages = gen.planted_pages(cfg, 0, 3)
    assert pages.size == 8 and pages.max() < 2048


def test_grid_dot_products_are_exact_in_fp32():
    # the exactness precondition: sum of |q_d k_d| stays below 2^14 for the workloads' shapes
    from workloads import get_config
    for cfg_id in (1, 4):
        cfg = get_config(cfg_id)
        q = gen.unit_query(cfg, 0, 0, 0)
        k, _ = gen.unit_kv(cfg, 0, 0, length=256)
        bound = np.abs(q).sum(1).max() * np.abs(k).max()
        assert bound < 2 ** 14
        exact = q.astype(np.float64) @ k.astype(np.float64).T
        np.testing.assert_array_equal((q @ k.T).astype(np.float64), exact)
