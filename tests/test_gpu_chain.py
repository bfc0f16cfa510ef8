"""GPU parity of the Chain Cache bookkeeping (se_chain_remap,
se_chain_append_positions) over a two-turn conversation: SnapKV compaction at the
end of turn 1, turn 2 appended to the compacted cache without re-prefill, decode
attention over it, and a second compaction at the end of turn 2.  Every physical
row must be the row of the logical position its map names (bit copies), the maps
must equal the oracle's, and attention over the chained cache must equal the
oracle's attention over those logical rows."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import boundary_gap
from oracle import chain as och
from oracle import snapkv as osnap
from tests.gpu_util import TOL, banner, dev, host, zeros
from tests.h2o_omni_cases import CHAIN_BUDGET2, CHAIN_CASES, CHAIN_TAGS, CHAIN_TURN2
from workloads import generator as gen

pytestmark = pytest.mark.gpu


ATTEMPTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "attempts.json")))
GAP = ATTEMPTS["gap"]


def oracle_kept(cfg, qo, rows, n, budget, where):
    """The oracle's SnapKV kept set of one unit (its boundary clear of near-ties)."""
    W = cfg.snap_window
    pooled = osnap.snapkv_pool(osnap.unit_votes(qo, rows, n, W, cfg.softmax_scale), cfg.snap_pool)
    assert boundary_gap(pooled, budget - W) >= GAP, f"{where}: generated input has a near-tie"
    return osnap.snapkv_keep(pooled, n, W, budget)


@pytest.mark.parametrize("dtype", list(CHAIN_CASES))
def test_two_turn_chain(se, dtype):
    cfg = CHAIN_CASES[dtype]
    banner(f"chain cache two turns {dtype}")
    att = {tuple(int(x) for x in k.split(",")): v for k, v in ATTEMPTS["chain"][dtype].items()}
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    B, H, Hq, D, G = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.group
    L1, W, pool, budget, n2 = cfg.context, cfg.snap_window, cfg.snap_pool, cfg.snap_budget, CHAIN_TURN2
    # the logical history: turn 1's prompt and turn 2's new tokens, rows by logical position
    Klog, Vlog = gen.cache_kv(cfg, CHAIN_TAGS[0], L1 + n2, length=L1 + n2)
    Klog = torch.from_numpy(Klog).to(dt).float().numpy()
    Vlog = torch.from_numpy(Vlog).to(dt).float().numpy()
    c1 = se.cache(B, Hq, H, D, D, L1, dtype)
    cap = budget + n2 + 4
    c2 = se.cache(B, Hq, H, D, D, cap, dtype)
    k_out = torch.zeros((B, H, cap, D), dtype=dt, device="cuda")
    v_out = torch.zeros_like(k_out)
    kept = torch.zeros((B, H, budget), dtype=torch.int32, device="cuda")
    olen = torch.zeros((B,), dtype=torch.int32, device="cuda")
    qo = gen.obs_queries(cfg, CHAIN_TAGS[0], att)
    se.se_snapkv_score_compact(c1, dev(qo, dt), dev(Klog[:, :, :L1], dt), dev(Vlog[:, :, :L1], dt), L1, W, pool, budget,
                               cfg.softmax_scale, c2, k_out, v_out, kept, None, olen, se.workspace(se.SE_OP_SNAPKV, c1,
                                                                                                   L1, W))
    pos = torch.full((B, H, cap), -7, dtype=torch.int32, device="cuda")
    se.se_chain_remap(c2, None, kept, olen, pos)
    torch.cuda.synchronize()
    n1 = int(host(olen)[0])
    assert n1 == budget
    g_kept, g_pos = host(kept), host(pos)
    r_kept = {}
    for b in range(B):
        for h in range(H):
            r_kept[b, h] = oracle_kept(cfg, qo[b, h * G:(h + 1) * G], Klog[b, h], L1, budget, f"turn 1 b={b} h={h}")
            np.testing.assert_array_equal(g_kept[b, h], r_kept[b, h], err_msg=f"turn 1 kept b={b} h={h}")
            ref = och.compose_positions(None, np.concatenate([r_kept[b, h], np.full(cap - budget, -1)]), n1)
            np.testing.assert_array_equal(g_pos[b, h], ref)
            np.testing.assert_array_equal(host(k_out)[b, h, :n1], Klog[b, h][ref[:n1]])
    # turn 2: the prefix is reused, only the new tokens are appended (logical positions L1 ..)
    logical_len = torch.full((B,), L1, dtype=torch.int32, device="cuda")
    se.se_chain_append_positions(c2, pos, olen, logical_len, n2)
    for j in range(n2):
        se.se_kv_append(c2, k_out, v_out, dev(Klog[:, :, L1 + j], dt), dev(Vlog[:, :, L1 + j], dt), None, olen)
    torch.cuda.synchronize()
    n = n1 + n2
    assert np.all(host(olen) == n)
    g_pos = host(pos)
    r_pos = {}
    for b in range(B):
        for h in range(H):
            r_pos[b, h] = och.append_positions(np.concatenate([r_kept[b, h], np.full(cap - budget, -1)]), n1, L1, n2)
            np.testing.assert_array_equal(g_pos[b, h], r_pos[b, h])
            np.testing.assert_array_equal(host(k_out)[b, h, :n], Klog[b, h][r_pos[b, h][:n]])
            np.testing.assert_array_equal(host(v_out)[b, h, :n], Vlog[b, h][r_pos[b, h][:n]])
    # decode over the chained cache = attention over the logical rows it keeps
    q = gen.decode_query(cfg, 31, 0)
    out, lse = zeros((B, Hq, D)), zeros((B, Hq))
    se.se_sparse_decode_attn(c2, dev(q, dt), k_out, v_out, olen, None, None, 0, 1, cfg.softmax_scale, out, lse,
                             ws=se.workspace(se.SE_OP_ATTN, c2, cap, 0))
    torch.cuda.synchronize()
    Ksel = np.stack([np.stack([Klog[b, h][r_pos[b, h][:n]] for h in range(H)]) for b in range(B)])
    Vsel = np.stack([np.stack([Vlog[b, h][r_pos[b, h][:n]] for h in range(H)]) for b in range(B)])
    ref_o, ref_l, _ = oatt.decode_attention(q, Ksel, Vsel, [n] * B, cfg.softmax_scale)
    np.testing.assert_allclose(host(out), ref_o, atol=TOL[dtype], rtol=0)
    np.testing.assert_allclose(host(lse), ref_l, atol=TOL[dtype], rtol=0)
    # end of turn 2: a second compaction of the chained cache composes the map
    budget2 = CHAIN_BUDGET2
    c3 = se.cache(B, Hq, H, D, D, budget2, dtype)
    k3 = torch.zeros((B, H, budget2, D), dtype=dt, device="cuda")
    v3 = torch.zeros_like(k3)
    kept2 = torch.zeros((B, H, budget2), dtype=torch.int32, device="cuda")
    olen2 = torch.zeros((B,), dtype=torch.int32, device="cuda")
    qo2 = gen.obs_queries(cfg, CHAIN_TAGS[1], att)
    se.se_snapkv_score_compact(c2, dev(qo2, dt), k_out, v_out, n, W, pool, budget2, cfg.softmax_scale, c3, k3, v3,
                               kept2, None, olen2, se.workspace(se.SE_OP_SNAPKV, c2, n, W))
    pos2 = torch.full((B, H, budget2), -7, dtype=torch.int32, device="cuda")
    se.se_chain_remap(c3, pos, kept2, olen2, pos2)
    torch.cuda.synchronize()
    g_kept2, g_pos2 = host(kept2), host(pos2)
    for b in range(B):
        for h in range(H):
            rows = Klog[b, h][r_pos[b, h][:n]]          # the chained cache's physical rows, by the oracle's map
            k2 = oracle_kept(cfg, qo2[b, h * G:(h + 1) * G], rows, n, budget2, f"turn 2 b={b} h={h}")
            np.testing.assert_array_equal(g_kept2[b, h], k2, err_msg=f"turn 2 kept b={b} h={h}")
            ref2 = och.compose_positions(r_pos[b, h], k2, budget2)
            np.testing.assert_array_equal(g_pos2[b, h], ref2)
            np.testing.assert_array_equal(host(k3)[b, h], Klog[b, h][ref2])
            np.testing.assert_array_equal(host(v3)[b, h], Vlog[b, h][ref2])
            assert set(range(L1 + n2 - W, L1 + n2)) <= set(ref2.tolist())   # the newest window kept
