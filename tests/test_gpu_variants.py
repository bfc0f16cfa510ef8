"""GPU parity of the StreamingLLM view (se_streaming_view, then the decode
attention over it) and of PyramidKV layers (se_pyramid_budgets driving the
SnapKV call per layer) against the CPU oracle, through the C ABI."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import boundary_gap
from oracle import snapkv as osnap
from oracle import variants as ov
from tests.gpu_util import TOL, banner, dev, host, tdtype, zeros
from tests.h2o_omni_cases import PYRAMID_CASES, PYRAMID_LAYERS
from workloads import generator as gen
from workloads import get_config

pytestmark = pytest.mark.gpu

GAP = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "attempts.json")))["gap"]


@pytest.mark.parametrize("sink,recent", [(4, 60), (0, 33), (7, 0), (1, 1), (16, 2032)])
def test_streaming_view_matches_oracle(se, sink, recent):
    banner(f"streaming view sink={sink} recent={recent}")
    B, H, cap = 5, 3, 3000
    lens = [0, 1, sink + recent, sink + recent + 1, cap]
    c = se.cache(B, 2 * H, H, 64, 64, cap, "bf16")
    vc = sink + recent + 3
    view = torch.full((B, H, vc), 77, dtype=torch.int32, device="cuda")
    vlen = torch.full((B, H), 77, dtype=torch.int32, device="cuda")
    se.se_streaming_view(c, torch.tensor(lens, dtype=torch.int32, device="cuda"), sink, recent, view, vlen)
    torch.cuda.synchronize()
    rv, rl = ov.streaming_view(lens, H, sink, recent, vc)
    np.testing.assert_array_equal(host(vlen), rl)
    np.testing.assert_array_equal(host(view), rv)


@pytest.mark.parametrize("pending", [1, 3])
def test_streaming_view_ahead_of_appends(se, pending):
    """pending > 0: the view of the length seq_len + pending (capped at the capacity)."""
    banner(f"streaming view pending={pending}")
    B, H, cap, sink, recent = 5, 3, 3000, 4, 60
    lens = [0, 1, sink + recent - 1, cap - 2, cap]
    c = se.cache(B, 2 * H, H, 64, 64, cap, "bf16")
    vc = sink + recent
    view = torch.full((B, H, vc), 77, dtype=torch.int32, device="cuda")
    vlen = torch.full((B, H), 77, dtype=torch.int32, device="cuda")
    se.se_streaming_view(c, torch.tensor(lens, dtype=torch.int32, device="cuda"), sink, recent, view, vlen, pending)
    torch.cuda.synchronize()
    rv, rl = ov.streaming_view([min(x + pending, cap) for x in lens], H, sink, recent, vc)
    np.testing.assert_array_equal(host(vlen), rl)
    np.testing.assert_array_equal(host(view), rv)


def test_streaming_step_with_fused_append(se):
    """The view taken one append ahead, then se_kv_append_decode_attn, gives the same
    caches, lengths and outputs (bit for bit) as append, view, attention."""
    cfg = get_config(0, dtype="bf16", batch=2, n_q_heads=16, n_kv_heads=2, d_k=128, d_v=128, context=900)
    banner("streaming step with the fused append")
    B, H, Hq, D = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k
    cap, sink, recent = cfg.context + 8, 4, 200
    vc = sink + recent
    K, V = gen.cache_kv(cfg, 6, cap)
    side = {}
    for t in ("fused", "sep"):
        side[t] = dict(k=dev(K, torch.bfloat16), v=dev(V, torch.bfloat16),
                       seq=torch.tensor([cfg.context, 150], dtype=torch.int32, device="cuda"),
                       view=torch.zeros((B, H, vc), dtype=torch.int32, device="cuda"),
                       vlen=torch.zeros((B, H), dtype=torch.int32, device="cuda"),
                       out=zeros((B, Hq, D)), lse=zeros((B, Hq)))
    c = se.cache(B, Hq, H, D, D, cap, "bf16")
    ws_f = se.workspace(se.SE_OP_APPEND_ATTN, c, vc, 0)
    ws_s = se.workspace(se.SE_OP_ATTN, c, vc, 0)
    for step in range(4):
        q = dev(gen.decode_query(cfg, 6, step), torch.bfloat16)
        kn, vn = gen.decode_kv_new(cfg, 6, step)
        knd, vnd = dev(kn, torch.bfloat16), dev(vn, torch.bfloat16)
        f, s_ = side["fused"], side["sep"]
        se.se_streaming_view(c, f["seq"], sink, recent, f["view"], f["vlen"], 1)
        se.se_kv_append_decode_attn(c, q, f["k"], f["v"], knd, vnd, None, f["seq"], f["view"], f["vlen"], vc, 1,
                                    cfg.softmax_scale, f["out"], f["lse"], ws=ws_f)
        se.se_kv_append(c, s_["k"], s_["v"], knd, vnd, None, s_["seq"])
        se.se_streaming_view(c, s_["seq"], sink, recent, s_["view"], s_["vlen"])
        se.se_sparse_decode_attn(c, q, s_["k"], s_["v"], s_["seq"], s_["view"], s_["vlen"], vc, 1, cfg.softmax_scale,
                                 s_["out"], s_["lse"], ws=ws_s)
        torch.cuda.synchronize()
        for key in ("k", "v", "seq", "view", "vlen", "out", "lse"):
            x, y = f[key], s_[key]
            dt = torch.int16 if x.element_size() == 2 else torch.int32
            assert torch.equal(x.view(dt), y.view(dt)), f"step {step}: {key} differ"


ATTN_CFGS = {
    "bf16_d128_g8": (get_config(0, dtype="bf16", batch=2, n_q_heads=16, n_kv_heads=2, d_k=128, d_v=128,
                                context=3000), 4, 700),
    "f32_d64_g4": (get_config(0, batch=2, n_q_heads=8, n_kv_heads=2, context=500), 4, 60),
    "mla_576": (get_config(4, batch=2, context=1500), 8, 256),
}


@pytest.mark.parametrize("name", list(ATTN_CFGS))
def test_streaming_decode_attention(se, name):
    """Attention over the StreamingLLM view equals the oracle's attention over the kept
    positions; with sink + recent covering the history it is dense attention."""
    cfg, sink, recent = ATTN_CFGS[name]
    banner(f"streaming attention {name}")
    dt = tdtype(cfg)
    B, H, Hq, D, Dv = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.d_v
    cap = cfg.context + 4
    c = se.cache(B, Hq, H, D, Dv, cap, cfg.dtype, cfg.latent)
    K, V = gen.cache_kv(cfg, 3, cap)
    q = gen.decode_query(cfg, 3, 0)
    k = dev(K, dt)
    v = None if cfg.latent else dev(V, dt)
    qd = dev(q, dt)
    for lens, sk, rc in (([cfg.context, cfg.context - 77], sink, recent), ([40, 13], sink, recent),
                         ([cfg.context, 9], cfg.context, 4)):
        seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
        vc = sk + rc
        view = torch.zeros((B, H, vc), dtype=torch.int32, device="cuda")
        vlen = torch.zeros((B, H), dtype=torch.int32, device="cuda")
        se.se_streaming_view(c, seq, sk, rc, view, vlen)
        out, lse = zeros((B, Hq, Dv)), zeros((B, Hq))
        ws = se.workspace(se.SE_OP_ATTN, c, vc, 0)
        se.se_sparse_decode_attn(c, qd, k, v, seq, view, vlen, vc, 1, cfg.softmax_scale, out, lse, ws=ws)
        torch.cuda.synchronize()
        rv, rl = ov.streaming_view(lens, H, sk, rc, vc)
        ref, ref_lse, _ = oatt.decode_attention(q, K, V, lens, cfg.softmax_scale, rv, rl, 1,
                                                latent_dv=Dv if cfg.latent else None)
        tol = TOL[cfg.dtype]
        np.testing.assert_allclose(host(out), ref, atol=tol, rtol=0, err_msg=f"lens {lens}")
        np.testing.assert_allclose(host(lse), ref_lse, atol=tol, rtol=0)
        if sk >= cfg.context:   # the whole history is kept: dense attention
            dense, _, _ = oatt.decode_attention(q, K, V, lens, cfg.softmax_scale, latent_dv=Dv if cfg.latent else None)
            np.testing.assert_allclose(host(out), dense, atol=tol, rtol=0)


def pyramid_attempts(name):
    """(layer, 0, unit) -> attempt of the window queries of one PyramidKV case."""
    att = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "attempts.json")))
    return {tuple(int(x) for x in k.split(",")): v for k, v in att.get("pyramid", {}).get(name, {}).items()}


@pytest.mark.parametrize("name", list(PYRAMID_CASES))
def test_pyramid_layers(se, name):
    """Four layers with the schedule's budgets: each layer's kept set (window plus its
    budget's best pooled votes) and compacted rows against the oracle, for every unit
    (the window queries are drawn so that no unit's vote boundary is a near-tie)."""
    cfg, avg, bmin = PYRAMID_CASES[name]
    banner(f"pyramid layers {name}")
    dt = tdtype(cfg)
    B, H, Hq, D = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k
    L, W, pool, G = cfg.context, cfg.snap_window, cfg.snap_pool, cfg.group
    budgets = se.se_pyramid_budgets(PYRAMID_LAYERS, avg, bmin)
    assert budgets == ov.pyramid_budgets(PYRAMID_LAYERS, avg, bmin)
    attempts = pyramid_attempts(name)
    c = se.cache(B, Hq, H, D, D, L, cfg.dtype)
    ws = se.workspace(se.SE_OP_SNAPKV, c, L, W)
    for layer, budget in enumerate(budgets):
        K, V = gen.cache_kv(cfg, layer, L, length=L)
        qo = gen.obs_queries(cfg, layer, attempts)
        nkeep = min(budget, L)
        oc = se.cache(B, Hq, H, D, D, nkeep, cfg.dtype)
        k_out = torch.zeros((B, H, nkeep, D), dtype=dt, device="cuda")
        v_out = torch.zeros_like(k_out)
        kept = torch.zeros((B, H, budget), dtype=torch.int32, device="cuda")
        olen = torch.zeros((B,), dtype=torch.int32, device="cuda")
        se.se_snapkv_score_compact(c, dev(qo, dt), dev(K, dt), dev(V, dt), L, W, pool, budget, cfg.softmax_scale,
                                   oc, k_out, v_out, kept, None, olen, ws)
        torch.cuda.synchronize()
        assert np.all(host(olen) == nkeep)
        g_kept, g_k, g_v = host(kept), host(k_out), host(v_out)
        for u in range(B * H):
            b, h = divmod(u, H)
            row = g_kept[b, h, :nkeep]
            votes = osnap.unit_votes(qo[b, h * G:(h + 1) * G], K[b, h], L, W, cfg.softmax_scale)
            pooled = osnap.snapkv_pool(votes, pool)
            if budget < L:
                assert boundary_gap(pooled, budget - W) >= GAP, f"layer {layer} unit {u}: generated input near-tie"
            np.testing.assert_array_equal(row, osnap.snapkv_keep(pooled, L, W, budget),
                                          err_msg=f"layer {layer} unit {u}")
            np.testing.assert_array_equal(g_k[b, h], K[b, h][row])      # rows are bit copies
            np.testing.assert_array_equal(g_v[b, h], V[b, h][row])
