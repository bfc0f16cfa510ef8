"""GPU parity of the H2O accumulate-evict step and the OmniKV cross-layer top-k
sweep against the CPU oracle, through the C ABI."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import h2o as oh2o
from oracle import omnikv as oomni
from tests.gpu_util import TOL, banner, dev, host, zeros
from tests.h2o_omni_cases import h2o_config, h2o_step_inputs, h2o_unit_start, omni_config, omni_layer_kv
from tests.sampled_units import H2O_UNITS, OMNI_STEPS, OMNI_UNITS
from workloads import generator as gen

pytestmark = pytest.mark.gpu

ATTEMPTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "attempts.json")))


def attempts_of(name):
    return {tuple(int(x) for x in k.split(",")): v for k, v in ATTEMPTS.get(name, {}).items()}


# ------------------------------------------------------------------ H2O

def run_h2o(se, cfg, units, attempts, fused=False):
    """fused: the step's append and attention through se_kv_append_decode_attn (the
    bench's call) instead of se_kv_append then se_sparse_decode_attn."""
    B, H, Hq, D = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k
    G = cfg.group
    cap = cfg.h2o_heavy + cfg.h2o_recent + 1
    K = np.zeros((B, H, cap, D), np.float32)
    V = np.zeros_like(K)
    pos = np.zeros((B, H, cap), np.int32)
    acc = np.zeros((B, H, cap), np.float32)
    for u in range(B * H):
        K[u // H, u % H], V[u // H, u % H], pos[u // H, u % H], acc[u // H, u % H] = h2o_unit_start(cfg, u)
    c = se.cache(B, Hq, H, D, D, cap, "bf16")
    k, v = dev(K, torch.bfloat16), dev(V, torch.bfloat16)
    slot_pos, acc_d = dev(pos, torch.int32), dev(acc)
    seq = torch.full((B,), cap, dtype=torch.int32, device="cuda")
    evict = torch.full((B, H), cap - 1, dtype=torch.int32, device="cuda")
    out, lse, logits = zeros((B, Hq, D)), zeros((B, Hq)), zeros((B, Hq, cap))
    ws = se.workspace(se.SE_OP_APPEND_ATTN if fused else se.SE_OP_ATTN, c, cap, 0)
    # oracle state of the compared units
    ost = {u: dict(zip(("k", "v", "pos", "acc"), h2o_unit_start(cfg, u))) for u in units}
    for u in units:
        ost[u]["acc"] = ost[u]["acc"].astype(np.float64)
        ost[u]["n"], ost[u]["free"] = cap, cap - 1
    for t in range(cfg.decode_steps):
        q, kn, vn = h2o_step_inputs(cfg, t, attempts)
        if fused:
            se.se_kv_append_decode_attn(c, dev(q, torch.bfloat16), k, v, dev(kn, torch.bfloat16),
                                        dev(vn, torch.bfloat16), evict, seq, None, None, 0, 1, cfg.softmax_scale, out,
                                        lse, logits, cap, 0, ws)
        else:
            se.se_kv_append(c, k, v, dev(kn, torch.bfloat16), dev(vn, torch.bfloat16), evict, seq)
            se.se_sparse_decode_attn(c, dev(q, torch.bfloat16), k, v, seq, None, None, 0, 1, cfg.softmax_scale, out,
                                     lse, logits, cap, 0, ws)
        se.se_h2o_accumulate_evict(c, logits, lse, cap, seq, slot_pos, acc_d, cfg.context + t, cfg.h2o_heavy,
                                   cfg.h2o_recent, evict)
        torch.cuda.synchronize()
        g_ev, g_pos, g_acc, g_out = host(evict), host(slot_pos), host(acc_d), host(out)
        for u in units:
            b, h = divmod(u, H)
            s = ost[u]
            o, l, s["pos"], s["acc"], s["n"], s["free"] = oh2o.h2o_step(
                s["k"], s["v"], s["pos"], s["acc"], s["n"], s["free"], q[b, h * G:(h + 1) * G], kn[b, h], vn[b, h],
                cfg.context + t, cfg.h2o_heavy, cfg.h2o_recent, cfg.softmax_scale)
            assert g_ev[b, h] == s["free"], f"step {t} unit {u}: evicted slot"
            np.testing.assert_array_equal(g_pos[b, h], s["pos"])
            np.testing.assert_allclose(g_acc[b, h], s["acc"], rtol=1e-4, atol=1e-6)
            np.testing.assert_allclose(g_out[b, h * G:(h + 1) * G], o, rtol=0, atol=TOL["bf16"])
    # invariants over every unit
    g_pos = host(slot_pos)
    last = cfg.context + cfg.decode_steps - 1
    for u in range(B * H):
        p = g_pos[u // H, u % H]
        assert (p >= 0).sum() == cfg.h2o_heavy + cfg.h2o_recent
        assert set(range(last - cfg.h2o_recent + 1, last + 1)) <= set(p.tolist())


@pytest.mark.parametrize("fused", [False, True])
def test_h2o_tiny_all_units_all_steps(se, fused):
    cfg = h2o_config(False)
    banner(f"h2o tiny fused={fused}")
    run_h2o(se, cfg, range(cfg.units), {}, fused)


def test_h2o_16k_sampled_units(se):
    """The bench's step: the append into the freed slot and the attention in one launch."""
    cfg = h2o_config(True)
    banner("h2o 16K: 64 x 4 units, 128 steps")
    run_h2o(se, cfg, H2O_UNITS, attempts_of("h2o_16k"), fused=True)


# ------------------------------------------------------------------ OmniKV

def run_omni(se, cfg, units, check_steps, attempts, fused=False):
    B, H, Hq, D = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k
    G = cfg.group
    n_steps = max(check_steps) + 1
    cap = cfg.context + cfg.extra["omni_steps"]
    plan = oomni.omnikv_layer_views(cfg.omni_layers, cfg.omni_filters)
    c = se.cache(B, Hq, H, D, D, cap, "bf16")
    ks, vs, host_units = [], [], []
    for layer in range(cfg.omni_layers):
        K, V = omni_layer_kv(cfg, layer)
        ks.append(dev(K, torch.bfloat16))
        vs.append(dev(V, torch.bfloat16))
        host_units.append({u: (K[u // H, u % H].copy(), V[u // H, u % H].copy()) for u in units})
        del K, V
    seqs = [torch.full((B,), cfg.context, dtype=torch.int32, device="cuda") for _ in range(cfg.omni_layers)]
    views = {f: torch.zeros((B, H, cfg.omni_top_k), dtype=torch.int32, device="cuda") for f in cfg.omni_filters}
    vlens = {f: torch.zeros((B, H), dtype=torch.int32, device="cuda") for f in cfg.omni_filters}
    out, lse, logits = zeros((B, Hq, D)), zeros((B, Hq)), zeros((B, Hq, cap))
    op = se.SE_OP_APPEND_ATTN if fused else se.SE_OP_ATTN
    ws_dense = se.workspace(op, c, cap, 0)
    ws_sparse = se.workspace(op, c, cfg.omni_top_k, 0)
    ws_topk = se.workspace(se.SE_OP_OMNIKV, c, cap, cfg.omni_top_k)
    for s in range(n_steps):
        outs, qs = {}, []
        for layer, (mode, src) in enumerate(plan):
            q = gen.decode_query(cfg, layer, s, attempts)
            qs.append(q)
            kn, vn = gen.decode_kv_new(cfg, layer, s)
            for u in units:
                hk, hv = host_units[layer][u]
                hk[cfg.context + s], hv[cfg.context + s] = kn[u // H, u % H], vn[u // H, u % H]
            knd, vnd = dev(kn, torch.bfloat16), dev(vn, torch.bfloat16)
            if not fused:
                se.se_kv_append(c, ks[layer], vs[layer], knd, vnd, None, seqs[layer])
            qd = dev(q, torch.bfloat16)
            lg = logits if mode == "filter" else None
            vi, vl, vc = (views[src], vlens[src], cfg.omni_top_k) if mode == "sparse" else (None, None, 0)
            wsx = ws_sparse if mode == "sparse" else ws_dense
            if fused:
                se.se_kv_append_decode_attn(c, qd, ks[layer], vs[layer], knd, vnd, None, seqs[layer], vi, vl, vc, 1,
                                            cfg.softmax_scale, out, lse, lg, cap if lg is not None else 0, 0, wsx)
            else:
                se.se_sparse_decode_attn(c, qd, ks[layer], vs[layer], seqs[layer], vi, vl, vc, 1, cfg.softmax_scale,
                                         out, lse, lg, cap if lg is not None else 0, 0, wsx)
            if mode == "filter":
                se.se_omnikv_topk(c, logits, lse, cap, seqs[layer], cfg.omni_top_k, views[layer], vlens[layer], None,
                                  ws_topk)
            if s in check_steps:
                outs[layer] = host(out)
        if s not in check_steps:
            continue
        torch.cuda.synchronize()
        banner(f"omnikv: checking step {s}")
        g_views = {f: host(views[f]) for f in cfg.omni_filters}
        n = cfg.context + s + 1
        for u in units:
            b, h = divmod(u, H)
            o_outs, o_views = oomni.unit_sweep(
                [qq[b, h * G:(h + 1) * G] for qq in qs], [host_units[l][u][0] for l in range(cfg.omni_layers)],
                [host_units[l][u][1] for l in range(cfg.omni_layers)], n, cfg.omni_filters, cfg.omni_top_k,
                cfg.softmax_scale)
            for f in cfg.omni_filters:
                np.testing.assert_array_equal(g_views[f][b, h], o_views[f], err_msg=f"step {s} unit {u} layer {f}")
            for layer in range(cfg.omni_layers):
                np.testing.assert_allclose(outs[layer][b, h * G:(h + 1) * G], o_outs[layer], rtol=0,
                                           atol=TOL["bf16"], err_msg=f"step {s} unit {u} layer {layer}")


@pytest.mark.parametrize("fused", [False, True])
def test_omnikv_tiny_all_units(se, fused):
    cfg = omni_config(False)
    banner(f"omnikv tiny fused={fused}")
    run_omni(se, cfg, range(cfg.units), range(cfg.extra["omni_steps"]), {}, fused)


def test_omnikv_16k_sampled_units(se):
    """The bench's sweep: each layer's append and attention in one launch."""
    cfg = omni_config(True)
    banner("omnikv 16K: 64 x 4 units, 18 layers, filters 2/8/16, top-2048")
    run_omni(se, cfg, OMNI_UNITS, OMNI_STEPS, attempts_of("omnikv_16k"), fused=True)
