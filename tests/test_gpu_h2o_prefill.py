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
from tests.gpu_util import banner, dev, host
from workloads import generator as gen
from workloads import get_config

pytestmark = pytest.mark.gpu

GAP = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "attempts.json")))["gap"]

CASES = {
    "d128_g8": (get_config(0, dtype="bf16", batch=2, n_q_heads=16, n_kv_heads=2, d_k=128, d_v=128), 700, 64, 32),
    "d128_g16_ragged": (get_config(0, dtype="bf16", batch=1, n_q_heads=32, n_kv_heads=2, d_k=128, d_v=128), 1033, 100,
                        50),
    "d64_g4": (get_config(0, dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2), 333, 40, 16),
    # G = 6: the (position, head) query rows straddle the 16-row MFMA column blocks
    "d128_g6_ragged": (get_config(0, dtype="bf16", batch=2, n_q_heads=12, n_kv_heads=2, d_k=128, d_v=128), 1111, 90,
                       33),
    "keep_all": (get_config(0, dtype="bf16", batch=1, n_q_heads=8, n_kv_heads=2), 90, 64, 32),
}


@pytest.mark.parametrize("name", list(CASES))
def test_h2o_prefill_init_matches_oracle(se, name):
    cfg, L, heavy, recent = CASES[name]
    banner(f"h2o prefill {name}")
    B, H, Hq, D, G = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.group
    cap = L + 7
    scale = 1.0 / np.sqrt(D)
    rng = np.random.default_rng(L)
    K, V = gen.cache_kv(cfg, 41, cap, length=cap)
    q = np.round(rng.normal(size=(B, Hq, L, D)) * 32).clip(-255, 255) / 32      # grid values, bf16-exact
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
    exact = 0
    for b in range(B):
        for h in range(H):
            ref = oh2o.prefill_scores(q[b, h * G:(h + 1) * G], K[b, h], L, scale)
            np.testing.assert_allclose(g_sc[b, h], ref, rtol=2e-4, atol=1e-6, err_msg=f"scores b={b} h={h}")
            n = min(heavy + recent, L)
            pos = g_pos[b, h]
            assert np.all(pos[n:] == -1) and np.all(g_acc[b, h, n:] == 0.0)
            kept = pos[:n]
            assert np.all(np.diff(kept) > 0) and np.all(kept >= 0) and np.all(kept < L)
            assert set(range(L - recent, L)) <= set(kept.tolist())
            np.testing.assert_array_equal(g_acc[b, h, :n], g_sc[b, h][kept])       # the kernel's own scores
            np.testing.assert_array_equal(g_k[b, h, :n], K[b, h][kept])           # bit copies of the rows
            np.testing.assert_array_equal(g_v[b, h, :n], V[b, h][kept])
            if heavy + recent >= L or boundary_gap(ref[:L - recent], heavy) >= GAP:
                rk, _, _ = oh2o.prefill_state(ref, L, heavy, recent, scap)
                np.testing.assert_array_equal(kept, rk, err_msg=f"kept b={b} h={h}")
                exact += 1
    assert exact >= (B * H + 1) // 2, f"only {exact} units had a clear heavy-hitter boundary"


def test_h2o_decode_continues_from_prefill_state(se):
    """The prefill-end state feeds se_h2o_accumulate_evict directly: six decode steps from
    it match the oracle's H2O steps started from the same slots."""
    from oracle import h2o as oh2o_mod
    from tests.gpu_util import TOL, zeros
    cfg = get_config(3, batch=2, n_q_heads=8, n_kv_heads=2, context=200, h2o_heavy=24, h2o_recent=12)
    banner("h2o decode from the prefill state")
    B, H, Hq, D, G = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.group
    L, heavy, recent = cfg.context, cfg.h2o_heavy, cfg.h2o_recent
    cap = heavy + recent + 1
    scale = cfg.softmax_scale
    K, V = gen.cache_kv(cfg, 43, L, length=L)
    q_prompt = np.round(np.random.default_rng(43).normal(size=(B, Hq, L, D)) * 32).clip(-255, 255) / 32
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
        pos = host(slot_pos)[b, h].astype(np.int64)
        rows_k = np.zeros((cap, D))
        rows_v = np.zeros((cap, D))
        rows_k[pos >= 0] = K[b, h][pos[pos >= 0]]
        rows_v[pos >= 0] = V[b, h][pos[pos >= 0]]
        st[u] = dict(k=rows_k, v=rows_v, pos=pos, acc=host(acc)[b, h].astype(np.float64), n=cap, free=cap - 1)
    seq = torch.full((B,), cap, dtype=torch.int32, device="cuda")
    evict = torch.full((B, H), cap - 1, dtype=torch.int32, device="cuda")
    out, lse, logits = zeros((B, Hq, D)), zeros((B, Hq)), zeros((B, Hq, cap))
    ws = se.workspace(se.SE_OP_ATTN, sl, cap, 0)
    for t in range(6):
        qd = gen.decode_query(cfg, 43, t)
        kn, vn = gen.decode_kv_new(cfg, 43, t)
        se.se_kv_append(sl, k, v, dev(kn, torch.bfloat16), dev(vn, torch.bfloat16), evict, seq)
        se.se_sparse_decode_attn(sl, dev(qd, torch.bfloat16), k, v, seq, None, None, 0, 1, scale, out, lse, logits, cap,
                                 0, ws)
        se.se_h2o_accumulate_evict(sl, logits, lse, cap, seq, slot_pos, acc, L + t, heavy, recent, evict)
        torch.cuda.synchronize()
        for u in range(B * H):
            b, h = divmod(u, H)
            s = st[u]
            o, _, s["pos"], s["acc"], s["n"], s["free"] = oh2o_mod.h2o_step(
                s["k"], s["v"], s["pos"], s["acc"], s["n"], s["free"], qd[b, h * G:(h + 1) * G], kn[b, h], vn[b, h],
                L + t, heavy, recent, scale)
            assert host(evict)[b, h] == s["free"], f"step {t} unit {u}"
            np.testing.assert_array_equal(host(slot_pos)[b, h], s["pos"])
            np.testing.assert_allclose(host(acc)[b, h], s["acc"], rtol=1e-4, atol=1e-5)
            np.testing.assert_allclose(host(out)[b, h * G:(h + 1) * G], o, rtol=0, atol=TOL["bf16"])
