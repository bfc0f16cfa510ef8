"""GPU parity of se_snapkv_score_compact (window votes, max-pool, top-k, compaction)
against the CPU oracle, through the C ABI."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import boundary_gap
from oracle import snapkv as osnap
from tests.gpu_util import TOL, banner, dev, host, zeros
from workloads import generator as gen
from workloads import get_config

pytestmark = pytest.mark.gpu

ATTEMPTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "attempts.json")))
GAP = ATTEMPTS["gap"]


def attempts_of(name):
    return {tuple(int(x) for x in k.split(",")): v for k, v in ATTEMPTS.get(name, {}).items()}


def run_snap(se, cfg, units, attempts, cap=None, budget=None, check_gap=True, decode=False):
    """decode: then one decode step over the compacted cache as the bench runs it (the
    new row appended and attended in one launch), checked on the sampled units."""
    B, H, Hq, D = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k
    L, W, pool = cfg.context, cfg.snap_window, cfg.snap_pool
    budget = cfg.snap_budget if budget is None else budget
    cap = L if cap is None else cap
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    K, V = gen.cache_kv(cfg, 0, cap, length=L)
    qo = gen.obs_queries(cfg, 0, attempts)
    c = se.cache(B, Hq, H, D, D, cap, cfg.dtype)
    nkeep = min(budget, L)
    oc = se.cache(B, Hq, H, D, D, nkeep + 3, cfg.dtype)
    k_out = torch.zeros((B, H, nkeep + 3, D), dtype=dt, device="cuda")
    v_out = torch.zeros_like(k_out)
    kept = torch.zeros((B, H, budget), dtype=torch.int32, device="cuda")
    votes = torch.zeros((B, H, L - W), device="cuda")
    olen = torch.zeros((B,), dtype=torch.int32, device="cuda")
    ws = se.workspace(se.SE_OP_SNAPKV, c, L, W)
    se.se_snapkv_score_compact(c, dev(qo, dt), dev(K, dt), dev(V, dt), L, W, pool, budget, cfg.softmax_scale, oc,
                               k_out, v_out, kept, votes, olen, ws)
    torch.cuda.synchronize()
    g_kept, g_votes, g_k, g_v = host(kept), host(votes), host(k_out), host(v_out)
    assert np.all(host(olen) == nkeep)
    G = cfg.group
    kept_ref = {}
    for u in units:
        b, h = divmod(u, H)
        ref_votes = osnap.unit_votes(qo[b, h * G:(h + 1) * G], K[b, h], L, W, cfg.softmax_scale)
        pooled = osnap.snapkv_pool(ref_votes, pool)
        if check_gap and budget < L:
            assert boundary_gap(pooled, budget - W) >= GAP, f"unit {u}: generated input has a near-tie"
        ref_kept = osnap.snapkv_keep(pooled, L, W, budget)
        np.testing.assert_allclose(g_votes[b, h], ref_votes, rtol=1e-4, atol=1e-30, err_msg=f"unit {u} votes")
        np.testing.assert_array_equal(g_kept[b, h, :nkeep], ref_kept, err_msg=f"unit {u} kept")
        assert np.all(g_kept[b, h, nkeep:] == -1)
        np.testing.assert_array_equal(g_k[b, h, :nkeep], K[b, h][ref_kept])
        np.testing.assert_array_equal(g_v[b, h, :nkeep], V[b, h][ref_kept])
        if decode:
            kept_ref[u] = ref_kept
    if decode:
        q = gen.decode_query(cfg, 0, 0)
        kn, vn = gen.decode_kv_new(cfg, 0, 0)
        out, lse = zeros((B, Hq, D)), zeros((B, Hq))
        se.se_kv_append_decode_attn(oc, dev(q, dt), k_out, v_out, dev(kn, dt), dev(vn, dt), None, olen, None, None, 0,
                                    1, cfg.softmax_scale, out, lse,
                                    ws=se.workspace(se.SE_OP_APPEND_ATTN, oc, nkeep + 3, 0))
        torch.cuda.synchronize()
        assert np.all(host(olen) == nkeep + 1)
        g_out, g_lse = host(out), host(lse)
        kq = torch.from_numpy(np.asarray(kn, np.float32)).to(dt).float().numpy()   # rows as stored
        vq = torch.from_numpy(np.asarray(vn, np.float32)).to(dt).float().numpy()
        for u in units:
            b, h = divmod(u, H)
            Ku = np.concatenate([K[b, h][kept_ref[u]], kq[b, h][None]])[None, None]
            Vu = np.concatenate([V[b, h][kept_ref[u]], vq[b, h][None]])[None, None]
            ro, rl, _ = oatt.decode_attention(q[b:b + 1, h * G:(h + 1) * G], Ku, Vu, [nkeep + 1], cfg.softmax_scale)
            tol = TOL[cfg.dtype]
            np.testing.assert_allclose(g_out[b, h * G:(h + 1) * G], ro[0], atol=tol, rtol=0, err_msg=f"unit {u} out")
            np.testing.assert_allclose(g_lse[b, h * G:(h + 1) * G], rl[0], atol=tol, rtol=0, err_msg=f"unit {u} lse")
    return g_kept


def test_snapkv_tiny_f32_all_units(se):
    cfg = get_config(0)
    banner("snapkv tiny f32")
    run_snap(se, cfg, range(cfg.units), attempts_of("snapkv_tiny"), cap=cfg.context + 5)


def mid_config():
    # bf16, MFMA path (G * W = 64 rows), a scaled-down vote ladder keeps the boundary clear
    return get_config(2, batch=2, context=4096, snap_window=8, snap_budget=400, snap_peaks=100,
                      snap_peak_spacing=40, snap_peak_levels=10)


def test_snapkv_bf16_mfma_mid(se):
    cfg = mid_config()
    banner("snapkv bf16 mid")
    run_snap(se, cfg, range(cfg.units), {})


def test_snapkv_bf16_rows_128_and_256(se):
    for W in (16, 32):
        cfg = get_config(2, batch=1, context=3000, snap_window=W, snap_budget=300, snap_peaks=60,
                          snap_peak_spacing=40, snap_peak_levels=8)
        banner(f"snapkv bf16 rows {cfg.group * W}")
        run_snap(se, cfg, range(cfg.units), {})


def test_snapkv_bf16_rows_192_and_d64(se):
    """The MFMA passes with three 16-row blocks per wave (192 window rows) and with
    64-wide heads (128 rows)."""
    for W, d in ((24, 128), (16, 64)):
        cfg = get_config(2, batch=1, context=3000, d_k=d, d_v=d, snap_window=W, snap_budget=300, snap_peaks=60,
                          snap_peak_spacing=40, snap_peak_levels=8)
        banner(f"snapkv bf16 rows {cfg.group * W} d {d}")
        run_snap(se, cfg, range(cfg.units), {})


def test_snapkv_budget_covers_prompt_and_window_only(se):
    cfg = get_config(0, context=300)
    banner("snapkv edges")
    kept = run_snap(se, cfg, range(cfg.units), {}, budget=400, check_gap=False)
    assert np.all(kept[:, :, :300] == np.arange(300))
    kept = run_snap(se, cfg, range(cfg.units), {}, budget=cfg.snap_window, check_gap=False)
    assert np.all(kept[:, :, :cfg.snap_window] == np.arange(300 - cfg.snap_window, 300))


def test_snapkv_128k_all_units(se):
    """The 128K SnapKV workload at full size through the bench's calls: the eviction of
    every unit's 131072-token prompt to 8192 tokens (votes, kept set, compacted rows),
    then 128 decode steps over the compacted cache (append and attention in one launch),
    every unit compared with the oracle at the first, a middle and the last step."""
    from tests import oracle_pool
    from tests.parity_jobs import snap_unit
    cfg = get_config(2)
    B, H, Hq, D, G = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.group
    L, W, pool, budget = cfg.context, cfg.snap_window, cfg.snap_pool, cfg.snap_budget
    attempts = attempts_of("snapkv_128k")
    checks = (0, 63, cfg.decode_steps - 1)
    jobs = [oracle_pool.pool().submit(snap_unit, ((2, {}), u, attempts.get((0, 0, u), 0), budget, checks))
            for u in range(cfg.units)]
    banner("snapkv 128K: 8 x 4 units, 131072 -> 8192, then 128 decode steps")
    K, V = gen.cache_kv(cfg, 0, L)
    qo = gen.obs_queries(cfg, 0, attempts)
    c = se.cache(B, Hq, H, D, D, L, "bf16")
    cap_out = budget + cfg.decode_steps + 3
    oc = se.cache(B, Hq, H, D, D, cap_out, "bf16")
    k_out = torch.zeros((B, H, cap_out, D), dtype=torch.bfloat16, device="cuda")
    v_out = torch.zeros_like(k_out)
    kept = torch.zeros((B, H, budget), dtype=torch.int32, device="cuda")
    votes = torch.zeros((B, H, L - W), device="cuda")
    olen = torch.zeros((B,), dtype=torch.int32, device="cuda")
    se.se_snapkv_score_compact(c, dev(qo, torch.bfloat16), dev(K, torch.bfloat16), dev(V, torch.bfloat16), L, W, pool,
                               budget, cfg.softmax_scale, oc, k_out, v_out, kept, votes, olen,
                               se.workspace(se.SE_OP_SNAPKV, c, L, W))
    torch.cuda.synchronize()
    assert np.all(host(olen) == budget)
    g_kept, g_votes, g_k, g_v = host(kept), host(votes), host(k_out), host(v_out)
    out, lse = zeros((B, Hq, D)), zeros((B, Hq))
    ws = se.workspace(se.SE_OP_APPEND_ATTN, oc, cap_out, 0)
    dec = {}
    for s in range(cfg.decode_steps):
        q = gen.decode_query(cfg, 0, s)
        kn, vn = gen.decode_kv_new(cfg, 0, s)
        se.se_kv_append_decode_attn(oc, dev(q, torch.bfloat16), k_out, v_out, dev(kn, torch.bfloat16),
                                    dev(vn, torch.bfloat16), None, olen, None, None, 0, 1, cfg.softmax_scale, out, lse,
                                    ws=ws)
        if s in checks:
            torch.cuda.synchronize()
            assert np.all(host(olen) == budget + s + 1)
            dec[s] = (host(out), host(lse))
    banner("snapkv 128K: comparing with the oracle")
    for u, job in enumerate(jobs):
        r = job.result()
        b, h = divmod(u, H)
        assert r["gap"] >= GAP, f"unit {u}: generated input has a near-tie ({r['gap']:.2e})"
        np.testing.assert_allclose(g_votes[b, h], r["votes"], rtol=1e-4, atol=1e-30, err_msg=f"unit {u} votes")
        np.testing.assert_array_equal(g_kept[b, h], r["kept"], err_msg=f"unit {u} kept")
        np.testing.assert_array_equal(g_k[b, h, :budget], K[b, h][r["kept"]], err_msg=f"unit {u} K rows")
        np.testing.assert_array_equal(g_v[b, h, :budget], V[b, h][r["kept"]], err_msg=f"unit {u} V rows")
        for s in checks:
            ro, rl = r["decode"][s]
            np.testing.assert_allclose(dec[s][0][b, h * G:(h + 1) * G], ro, atol=TOL["bf16"], rtol=0,
                                       err_msg=f"unit {u} step {s} out")
            np.testing.assert_allclose(dec[s][1][b, h * G:(h + 1) * G], rl, atol=TOL["bf16"], rtol=0,
                                       err_msg=f"unit {u} step {s} lse")
