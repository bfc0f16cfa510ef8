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
from tests.h2o_omni_cases import OMNI_STEPS, OMNI_UNITS, h2o_config, h2o_step_inputs, h2o_unit_start, omni_config, \
    omni_layer_kv
from workloads import generator as gen

pytestmark = pytest.mark.gpu

ATTEMPTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "attempts.json")))
GAP = ATTEMPTS["gap"]


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


def test_h2o_16k_all_units(se):
    """The 16K H2O workload at full size through the bench's call (se_h2o_decode_step:
    the append into the freed slot, the attention and the accumulate + evict in one
    launch): every unit's evicted slot, slot positions, scores and output compared
    with the oracle at every one of the 128 steps."""
    from tests import oracle_pool
    from tests.parity_jobs import h2o_unit
    cfg = h2o_config(True)
    B, H, Hq, D, G = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.group
    T = cfg.decode_steps
    att = attempts_of("h2o_16k")
    per_unit = [{t: a for (l, t, u2), a in att.items() if u2 == u} for u in range(cfg.units)]
    jobs = [oracle_pool.pool().submit(h2o_unit, ((3, {}), u, per_unit[u])) for u in range(cfg.units)]
    banner("h2o 16K: 64 x 4 units, 128 steps")
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
    ev = [torch.full((B, H), cap - 1, dtype=torch.int32, device="cuda"),
          torch.full((B, H), -1, dtype=torch.int32, device="cuda")]
    out, lse = zeros((B, Hq, D)), zeros((B, Hq))
    ws = se.workspace(se.SE_OP_H2O_STEP, c, 0, 0)
    g_ev = np.zeros((T, B, H), np.int32)
    g_pos = np.zeros((T, B, H, cap), np.int32)
    g_acc = np.zeros((T, B, H, cap), np.float32)
    g_out = np.zeros((T, B, Hq, D), np.float32)
    for t in range(T):
        q, kn, vn = h2o_step_inputs(cfg, t, att)
        se.se_h2o_decode_step(c, dev(q, torch.bfloat16), k, v, dev(kn, torch.bfloat16), dev(vn, torch.bfloat16),
                              ev[t % 2], seq, slot_pos, acc_d, cfg.context + t, cfg.h2o_heavy, cfg.h2o_recent,
                              cfg.softmax_scale, out, lse, ev[(t + 1) % 2], ws)
        g_ev[t], g_pos[t], g_acc[t], g_out[t] = host(ev[(t + 1) % 2]), host(slot_pos), host(acc_d), host(out)
    banner("h2o 16K: comparing with the oracle")
    for u, job in enumerate(jobs):
        r = job.result()
        b, h = divmod(u, H)
        assert np.all(r["gaps"] >= GAP), f"unit {u}: an eviction decision is a near-tie (steps " \
            f"{np.nonzero(r['gaps'] < GAP)[0].tolist()})"
        np.testing.assert_array_equal(g_ev[:, b, h], r["evict"], err_msg=f"unit {u}: evicted slots")
        np.testing.assert_array_equal(g_pos[:, b, h], r["pos"], err_msg=f"unit {u}: slot positions")
        np.testing.assert_allclose(g_acc[:, b, h], r["acc"], rtol=1e-4, atol=1e-6, err_msg=f"unit {u}: scores")
        np.testing.assert_allclose(g_out[:, b, h * G:(h + 1) * G], r["out"], rtol=0, atol=TOL["bf16"],
                                   err_msg=f"unit {u}: outputs")
    last = cfg.context + T - 1
    for u in range(B * H):
        p = g_pos[-1, u // H, u % H]
        assert (p >= 0).sum() == cfg.h2o_heavy + cfg.h2o_recent
        assert set(range(last - cfg.h2o_recent + 1, last + 1)) <= set(p.tolist())


def test_h2o_16k_resume_from_saved_state(se):
    """Checkpoint / resume at full size: after 8 steps every caller-owned buffer of the
    H2O state (cache rows, slot positions, scores, length, evicted slot) is saved to host
    memory; 8 more steps run on, then the saved state is restored into freshly allocated
    buffers and the same 8 steps run again: outputs, evictions and state agree bit for
    bit."""
    cfg = h2o_config(True)
    B, H, Hq, D = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k
    cap = cfg.h2o_heavy + cfg.h2o_recent + 1
    banner("h2o 16K resume: 8 steps, save, 8 steps, restore, 8 steps")
    K = np.zeros((B, H, cap, D), np.float32)
    V = np.zeros_like(K)
    pos = np.zeros((B, H, cap), np.int32)
    acc = np.zeros((B, H, cap), np.float32)
    for u in range(B * H):
        K[u // H, u % H], V[u // H, u % H], pos[u // H, u % H], acc[u // H, u % H] = h2o_unit_start(cfg, u)
    c = se.cache(B, Hq, H, D, D, cap, "bf16")
    state = dict(k=dev(K, torch.bfloat16), v=dev(V, torch.bfloat16), slot_pos=dev(pos, torch.int32), acc=dev(acc),
                 seq=torch.full((B,), cap, dtype=torch.int32, device="cuda"),
                 ev0=torch.full((B, H), cap - 1, dtype=torch.int32, device="cuda"),
                 ev1=torch.full((B, H), -1, dtype=torch.int32, device="cuda"))
    ws = se.workspace(se.SE_OP_H2O_STEP, c, 0, 0)

    def run(st, steps):
        outs = []
        out, lse = zeros((B, Hq, D)), zeros((B, Hq))
        for t in steps:
            q, kn, vn = h2o_step_inputs(cfg, t)
            ev_in, ev_out = (st["ev0"], st["ev1"]) if t % 2 == 0 else (st["ev1"], st["ev0"])
            se.se_h2o_decode_step(c, dev(q, torch.bfloat16), st["k"], st["v"], dev(kn, torch.bfloat16),
                                  dev(vn, torch.bfloat16), ev_in, st["seq"], st["slot_pos"], st["acc"],
                                  cfg.context + t, cfg.h2o_heavy, cfg.h2o_recent, cfg.softmax_scale, out, lse, ev_out,
                                  ws)
            outs.append(torch.cat([out.flatten().view(torch.int32), lse.flatten().view(torch.int32),
                                   ev_out.flatten()]).cpu())
        torch.cuda.synchronize()
        return outs, {n: t.cpu() for n, t in st.items()}

    run(state, range(8))
    saved = {n: t.cpu() for n, t in state.items()}
    first, end1 = run(state, range(8, 16))
    restored = {n: t.to("cuda").clone() for n, t in saved.items()}
    second, end2 = run(restored, range(8, 16))
    for i, (a, b) in enumerate(zip(first, second)):
        assert torch.equal(a, b), f"step {8 + i}: outputs / evictions differ after the restore"
    for n in end1:
        assert torch.equal(end1[n].view(torch.uint8), end2[n].view(torch.uint8)), f"{n} differs after the restore"


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


def dev_grid_fill_(t, seed):
    """Fill a device tensor with seeded grid values (round(32 x) / 32 clipped to +-255/32,
    x ~ N(0, 1)) drawn on the device: rows no oracle check reads."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn(t.shape, generator=g, device="cuda", dtype=torch.float32)
    x.mul_(32.0).round_().clamp_(-255.0, 255.0).div_(32.0)
    t.copy_(x)


def test_omnikv_16k_48_layers(se):
    """The 16K OmniKV workload at full size through the bench's sweep (each layer's
    append and attention in one launch; filter layers 2/8/16 select top-2048 views that
    the following layers reuse): all 48 layers of 64 x 4 units run for 64 decode
    steps; at steps 0, 1 and 63 every layer's output and every filter view of the
    checked units are compared with the oracle's sweep."""
    from concurrent.futures import ThreadPoolExecutor
    from tests import oracle_pool
    from tests.parity_jobs import omni_unit
    cfg = omni_config(True)
    B, H, Hq, D, G = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.group
    nL, checks = cfg.omni_layers, OMNI_STEPS
    n_steps = max(checks) + 1
    att = attempts_of("omnikv_16k")
    jobs = [oracle_pool.pool().submit(omni_unit, ((3, {}), u, checks,
                                                  {(l, t): a for (l, t, u2), a in att.items() if u2 == u}))
            for u in OMNI_UNITS]
    plan = oomni.omnikv_layer_views(nL, cfg.omni_filters)
    cap = cfg.context + n_steps
    c = se.cache(B, Hq, H, D, D, cap, "bf16")
    banner(f"omnikv 16K: filling {nL} layers of 64 x 4 units")
    ks, vs = [], []
    with ThreadPoolExecutor(oracle_pool.n_workers()) as ex:
        for layer in range(nL):
            k = torch.empty((B, H, cap, D), dtype=torch.bfloat16, device="cuda")
            v = torch.empty_like(k)
            dev_grid_fill_(k, 7000 + 2 * layer)
            dev_grid_fill_(v, 7001 + 2 * layer)
            for u, (kk, vv) in zip(OMNI_UNITS, ex.map(lambda u: gen.unit_kv(cfg, layer, u, cfg.context), OMNI_UNITS)):
                k[u // H, u % H, :cfg.context] = torch.from_numpy(kk).to("cuda", torch.bfloat16)
                v[u // H, u % H, :cfg.context] = torch.from_numpy(vv).to("cuda", torch.bfloat16)
            ks.append(k)
            vs.append(v)
    seqs = [torch.full((B,), cfg.context, dtype=torch.int32, device="cuda") for _ in range(nL)]
    views = {f: torch.zeros((B, H, cfg.omni_top_k), dtype=torch.int32, device="cuda") for f in cfg.omni_filters}
    vlens = {f: torch.zeros((B, H), dtype=torch.int32, device="cuda") for f in cfg.omni_filters}
    out, lse, logits = zeros((B, Hq, D)), zeros((B, Hq)), zeros((B, Hq, cap))
    ws_dense = se.workspace(se.SE_OP_APPEND_ATTN, c, cap, 0)
    ws_sparse = se.workspace(se.SE_OP_APPEND_ATTN, c, cfg.omni_top_k, 0)
    ws_topk = se.workspace(se.SE_OP_OMNIKV, c, cap, cfg.omni_top_k)
    qs = [None] * nL
    got = {}
    for s in range(n_steps):
        if s in checks or s == 0:
            qs = [dev(gen.decode_query(cfg, layer, s, att), torch.bfloat16) for layer in range(nL)]
        outs = {}
        for layer, (mode, src) in enumerate(plan):
            kn, vn = gen.decode_kv_new(cfg, layer, s)
            lg = logits if mode == "filter" else None
            vi, vl, vc = (views[src], vlens[src], cfg.omni_top_k) if mode == "sparse" else (None, None, 0)
            se.se_kv_append_decode_attn(c, qs[layer], ks[layer], vs[layer], dev(kn, torch.bfloat16),
                                        dev(vn, torch.bfloat16), None, seqs[layer], vi, vl, vc, 1, cfg.softmax_scale,
                                        out, lse, lg, cap if lg is not None else 0, 0,
                                        ws_sparse if mode == "sparse" else ws_dense)
            if mode == "filter":
                se.se_omnikv_topk(c, logits, lse, cap, seqs[layer], cfg.omni_top_k, views[layer], vlens[layer], None,
                                  ws_topk)
            if s in checks:
                outs[layer] = host(out)
        if s in checks:
            torch.cuda.synchronize()
            got[s] = (outs, {f: host(views[f]) for f in cfg.omni_filters},
                      {f: host(vlens[f]) for f in cfg.omni_filters})
            banner(f"omnikv 16K: step {s} captured")
    banner("omnikv 16K: comparing with the oracle")
    for u, job in zip(OMNI_UNITS, jobs):
        r = job.result()
        b, h = divmod(u, H)
        for s in checks:
            g_outs, g_views, g_vlens = got[s]
            for f in cfg.omni_filters:
                assert r[s]["gaps"][f] >= GAP, f"unit {u} step {s} layer {f}: near-tie ({r[s]['gaps'][f]:.2e})"
                assert g_vlens[f][b, h] == cfg.omni_top_k
                np.testing.assert_array_equal(g_views[f][b, h], r[s]["views"][f], err_msg=f"step {s} unit {u} layer {f}")
            for layer in range(nL):
                np.testing.assert_allclose(g_outs[layer][b, h * G:(h + 1) * G], r[s]["outs"][layer], rtol=0,
                                           atol=TOL["bf16"], err_msg=f"step {s} unit {u} layer {layer}")
