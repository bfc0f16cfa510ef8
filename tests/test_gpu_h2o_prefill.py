"""GPU parity of se_h2o_prefill_init (H2O scores at the end of a prefill, the
heavy + recent kept slots and their rows) against the CPU oracle, through the
C ABI."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import boundary_gap
from oracle import h2o as oh2o
from tests.gpu_util import TOL, banner, dev, host, zeros
from tests.h2o_omni_cases import (PREFILL_CASES, PREFILL_DECODE_CFG, PREFILL_DECODE_LAYER, PREFILL_KV_LAYER,
                                  prefill_queries)
from workloads import generator as gen

pytestmark = pytest.mark.gpu

ATTEMPTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "attempts.json")))
GAP = ATTEMPTS["gap"]


def prefill_attempts(name):
    """unit -> attempt of the prompt queries of one prefill case."""
    return {int(k): v for k, v in ATTEMPTS.get("h2o_prefill", {}).get(name, {}).items()}


@pytest.mark.parametrize("name", list(PREFILL_CASES))
def test_h2o_prefill_init_matches_oracle(se, name):
    """Scores within fp32 tolerance, and for every unit the kept set, its scores and
    its rows equal to the oracle's (the prompt queries are drawn so that no unit's
    heavy-hitter boundary is within the near-tie gap)."""
    cfg, L, heavy, recent = PREFILL_CASES[name]
    banner(f"h2o prefill {name}")
    B, H, Hq, D, G = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.group
    cap = L + 7
    scale = 1.0 / np.sqrt(D)
    K, V = gen.cache_kv(cfg, PREFILL_KV_LAYER, cap, length=cap)
    q = prefill_queries(cfg, list(PREFILL_CASES).index(name), L, prefill_attempts(name))
    c = se.cache(B, Hq, H, D, D, cap, "bf16")
    scap = heavy + recent + 1
    sl = se.cache(B, Hq, H, D, D, scap, "bf16")
    k_slots = torch.zeros((B, H, scap, D), dtype=torch.bfloat16, device="cuda")
    v_slots = torch.zeros_like(k_slots)
    slot_pos = torch.full((B, H, scap), -9, dtype=torch.int32, device="cuda")
    acc = torch.full((B, H, scap), -9.0, device="cuda")
    scores = torch.zeros((B, H, L), device="cuda")
    ws = se.workspace(se.SE_OP_H2O_PREFILL, c, L, recent)
    kd, vd, qd = dev(K, torch.bfloat16), dev(V, torch.bfloat16), dev(q, torch.bfloat16)
    for rep in range(2):   # the second call checks that the workspace counters came back to zero
        se.se_h2o_prefill_init(c, qd, kd, vd, L, heavy, recent, scale, sl, k_slots, v_slots, slot_pos, acc, scores, ws)
        torch.cuda.synchronize()
    g_sc, g_pos, g_acc = host(scores), host(slot_pos), host(acc)
    g_k, g_v = host(k_slots), host(v_slots)
    for b in range(B):
        for h in range(H):
            where = f"{name} b={b} h={h}"
            ref = oh2o.prefill_scores(q[b, h * G:(h + 1) * G], K[b, h], L, scale)
            np.testing.assert_allclose(g_sc[b, h], ref, rtol=2e-4, atol=1e-6, err_msg=f"scores {where}")
            if heavy + recent < L:
                assert boundary_gap(ref[:L - recent], heavy) >= GAP, f"{where}: generated input has a near-tie"
            rk, rpos, racc = oh2o.prefill_state(ref, L, heavy, recent, scap)
            n = len(rk)
            np.testing.assert_array_equal(g_pos[b, h], rpos, err_msg=f"slot positions {where}")
            np.testing.assert_allclose(g_acc[b, h], racc, rtol=2e-4, atol=1e-6, err_msg=f"slot scores {where}")
            assert np.all(g_acc[b, h, n:] == 0.0)
            np.testing.assert_array_equal(g_k[b, h, :n], K[b, h][rk])           # bit copies of the rows
            np.testing.assert_array_equal(g_v[b, h, :n], V[b, h][rk])


def test_h2o_decode_continues_from_prefill_state(se):
    """The prefill-end state feeds se_h2o_accumulate_evict directly: six decode steps
    from it match the oracle's H2O steps started from the oracle's own prefill-end state
    (its kept rows, positions and float64 scores)."""
    cfg = PREFILL_DECODE_CFG
    banner("h2o decode from the prefill state")
    B, H, Hq, D, G = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.group
    L, heavy, recent = cfg.context, cfg.h2o_heavy, cfg.h2o_recent
    cap = heavy + recent + 1
    scale = cfg.softmax_scale
    att = ATTEMPTS.get("h2o_prefill_decode", {})
    prompt_att = {int(k): v for k, v in att.get("prompt", {}).items()}
    step_att = {tuple(int(x) for x in k.split(",")): v for k, v in att.get("steps", {}).items()}
    K, V = gen.cache_kv(cfg, PREFILL_DECODE_LAYER, L, length=L)
    q_prompt = prefill_queries(cfg, 99, L, prompt_att)
    c = se.cache(B, Hq, H, D, D, L, "bf16")
    sl = se.cache(B, Hq, H, D, D, cap, "bf16")
    k = torch.zeros((B, H, cap, D), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    slot_pos = torch.zeros((B, H, cap), dtype=torch.int32, device="cuda")
    acc = torch.zeros((B, H, cap), device="cuda")
    se.se_h2o_prefill_init(c, dev(q_prompt, torch.bfloat16), dev(K, torch.bfloat16), dev(V, torch.bfloat16), L, heavy,
                           recent, scale, sl, k, v, slot_pos, acc, None, se.workspace(se.SE_OP_H2O_PREFILL, c, L, recent))
    torch.cuda.synchronize()
    st = {}
    for u in range(B * H):
        b, h = divmod(u, H)
        acc0 = oh2o.prefill_scores(q_prompt[b, h * G:(h + 1) * G], K[b, h], L, scale)
        assert boundary_gap(acc0[:L - recent], heavy) >= GAP, f"unit {u}: prompt near-tie"
        kept, pos, acc_o = oh2o.prefill_state(acc0, L, heavy, recent, cap)
        rows_k = np.zeros((cap, D))
        rows_v = np.zeros((cap, D))
        rows_k[:len(kept)] = K[b, h][kept]
        rows_v[:len(kept)] = V[b, h][kept]
        np.testing.assert_array_equal(host(slot_pos)[b, h], pos, err_msg=f"unit {u}: prefill-end slots")
        st[u] = dict(k=rows_k, v=rows_v, pos=pos, acc=acc_o, n=cap, free=cap - 1)
    seq = torch.full((B,), cap, dtype=torch.int32, device="cuda")
    evict = torch.full((B, H), cap - 1, dtype=torch.int32, device="cuda")
    out, lse, logits = zeros((B, Hq, D)), zeros((B, Hq)), zeros((B, Hq, cap))
    ws = se.workspace(se.SE_OP_ATTN, sl, cap, 0)
    for t in range(cfg.decode_steps):
        qd = gen.decode_query(cfg, PREFILL_DECODE_LAYER, t, {(PREFILL_DECODE_LAYER, t, u): a
                                                              for (tt, u), a in step_att.items() if tt == t})
        kn, vn = gen.decode_kv_new(cfg, PREFILL_DECODE_LAYER, t)
        se.se_kv_append(sl, k, v, dev(kn, torch.bfloat16), dev(vn, torch.bfloat16), evict, seq)
        se.se_sparse_decode_attn(sl, dev(qd, torch.bfloat16), k, v, seq, None, None, 0, 1, scale, out, lse, logits, cap,
                                 0, ws)
        se.se_h2o_accumulate_evict(sl, logits, lse, cap, seq, slot_pos, acc, L + t, heavy, recent, evict)
        torch.cuda.synchronize()
        for u in range(B * H):
            b, h = divmod(u, H)
            s = st[u]
            gaps = []
            o, _, s["pos"], s["acc"], s["n"], s["free"] = oh2o.h2o_step(
                s["k"], s["v"], s["pos"], s["acc"], s["n"], s["free"], qd[b, h * G:(h + 1) * G], kn[b, h], vn[b, h],
                L + t, heavy, recent, scale, gaps)
            assert all(g >= GAP for g in gaps), f"step {t} unit {u}: eviction near-tie"
            assert host(evict)[b, h] == s["free"], f"step {t} unit {u}"
            np.testing.assert_array_equal(host(slot_pos)[b, h], s["pos"])
            np.testing.assert_allclose(host(acc)[b, h], s["acc"], rtol=2e-4, atol=1e-5)
            np.testing.assert_allclose(host(out)[b, h * G:(h + 1) * G], o, rtol=0, atol=TOL["bf16"])


def test_h2o_prefill_init_full_size(se):
    """The bench's prefill-end shape (64 rows x 4 KV heads x 8 query heads, 16K-token
    prompt, 1024 heavy + 256 recent slots).  Every unit: its scores sum to G * L (each
    query row's weights sum to one), and its kept set is the recent window plus the
    1024 best scores below it (ties to the lower position), ascending, with those
    scores.  Units (0, 0), (31, 2) and (63, 3): the scores of the last 48 keys against
    the oracle's (those keys get weight only from the last 48 query rows), and the
    kept rows as bit copies."""
    from workloads import get_config
    cfg = get_config(3)
    B, H, Hq, D, G, L = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.group, cfg.context
    heavy, recent = cfg.h2o_heavy, cfg.h2o_recent
    banner(f"h2o prefill full size B={B} Hkv={H} G={G} L={L}")
    scale = 1.0 / np.sqrt(D)
    gcuda = torch.Generator(device="cuda")
    gcuda.manual_seed(20261)
    q = torch.randn((B, Hq, L, D), generator=gcuda, device="cuda").to(torch.bfloat16)
    k = torch.randn((B, H, L, D), generator=gcuda, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, H, L, D), generator=gcuda, device="cuda").to(torch.bfloat16)
    c = se.cache(B, Hq, H, D, D, L, "bf16")
    scap = heavy + recent + 1
    sl = se.cache(B, Hq, H, D, D, scap, "bf16")
    k_slots = torch.zeros((B, H, scap, D), dtype=torch.bfloat16, device="cuda")
    v_slots = torch.zeros_like(k_slots)
    slot_pos = torch.full((B, H, scap), -9, dtype=torch.int32, device="cuda")
    acc = torch.full((B, H, scap), -9.0, device="cuda")
    scores = torch.zeros((B, H, L), device="cuda")
    ws = se.workspace(se.SE_OP_H2O_PREFILL, c, L, recent)
    se.se_h2o_prefill_init(c, q, k, v, L, heavy, recent, scale, sl, k_slots, v_slots, slot_pos, acc, scores, ws)
    torch.cuda.synchronize()
    g_sc, g_pos, g_acc = host(scores), host(slot_pos), host(acc)
    np.testing.assert_allclose(g_sc.astype(np.float64).sum(axis=-1), G * L, rtol=1e-4)
    n = heavy + recent
    for b in range(B):
        for h in range(H):
            where = f"b={b} h={h}"
            cand = g_sc[b, h, :L - recent]
            order = np.lexsort((np.arange(L - recent), -cand))   # best first, ties to the lower position
            kept = np.concatenate([np.sort(order[:heavy]), np.arange(L - recent, L)])
            np.testing.assert_array_equal(g_pos[b, h, :n], kept, err_msg=f"kept positions {where}")
            assert np.all(g_pos[b, h, n:] == -1) and np.all(g_acc[b, h, n:] == 0.0), where
            np.testing.assert_array_equal(g_acc[b, h, :n], g_sc[b, h, kept], err_msg=f"kept scores {where}")
    j0 = L - 48
    for b, h in ((0, 0), (31, 2), (63, 3)):
        qg = q[b, h * G:(h + 1) * G].float().cpu().numpy()
        kh = k[b, h].float().cpu().numpy()
        ref = oh2o.prefill_scores_tail(qg, kh, L, scale, j0)
        np.testing.assert_allclose(g_sc[b, h, j0:], ref, rtol=2e-4, atol=1e-6, err_msg=f"tail scores b={b} h={h}")
        kept = g_pos[b, h, :n]
        np.testing.assert_array_equal(host(k_slots[b, h, :n]), host(k[b, h][torch.from_numpy(kept).long().cuda()]))
        np.testing.assert_array_equal(host(v_slots[b, h, :n]), host(v[b, h][torch.from_numpy(kept).long().cuda()]))
