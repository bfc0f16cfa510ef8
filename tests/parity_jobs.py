"""Per-unit oracle jobs for the full-size parity tests (test infrastructure).

Each job rebuilds one unit's inputs from the seeded generator (the same calls
the GPU side makes to fill its buffers) and runs the oracle on them, step by
step in the workload's order.  Only small results leave the job: indices,
outputs and scores, and SHA-256 digests of the large bit-exact arrays (page
metadata, FP8 codes), which the tests compare with digests of the GPU's arrays
taken the same way.  Every decision and number comes from `oracle/`.
"""
import hashlib

import numpy as np

import oracle
from oracle import fp8 as ofp8
from oracle import h2o as oh2o
from oracle import omnikv as oomni
from oracle import quest as oquest
from oracle import snapkv as osnap
from workloads import generator as gen
from workloads import get_config


def digest(a):
    """SHA-256 of an array's float32 (or int32 / uint8) bytes, with its shape."""
    a = np.asarray(a)
    if a.dtype.kind == "f":
        a = a.astype(np.float32)
    elif a.dtype.kind in "iu" and a.dtype != np.uint8:
        a = a.astype(np.int32)
    a = np.ascontiguousarray(a)
    return f"{a.shape}:{a.dtype}:" + hashlib.sha256(a.tobytes()).hexdigest()


def cfg_of(spec):
    cfg_id, kw = spec
    return get_config(cfg_id, **kw)


def appended_rows(cfg, layer, unit, steps):
    """(k_new, v_new) rows [steps][d] the decode steps 0..steps-1 append to one unit."""
    b, h = divmod(unit, cfg.n_kv_heads)
    ks, vs = [], []
    for s in range(steps):
        kn, vn = gen.decode_kv_new(cfg, layer, s)
        ks.append(kn[b, h])
        vs.append(None if vn is None else vn[b, h])
    return ks, vs


# ------------------------------------------------------------------ Quest over FP8 rows

def fp8_quest_unit(job):
    """One unit of the Quest decode over FP8 rows: the prompt rows and every appended
    row quantized by the oracle's rule, then at each checked step the page metadata of
    the stored values, the Quest view and the attention over the stored rows."""
    spec, unit, check_steps = job
    cfg = cfg_of(spec)
    P, k, G = cfg.page_size, cfg.top_pages, cfg.group
    n_steps = max(check_steps) + 1
    K, V = gen.unit_kv(cfg, 0, unit, cfg.context)
    ks, vs = appended_rows(cfg, 0, unit, n_steps)
    K = np.concatenate([K, np.stack(ks)])
    V = np.concatenate([V, np.stack(vs)])
    kc, ksb = ofp8.quantize_rows(K)
    vc, vsb = ofp8.quantize_rows(V)
    Ks, Vs = ofp8.dequantize_rows(kc, ksb), ofp8.dequantize_rows(vc, vsb)
    res = {}
    for s in check_steps:
        L = cfg.context + s + 1
        qg = gen.unit_query(cfg, 0, s, unit)
        kmin, kmax = oquest.page_meta(Ks[None, None, :L], [L], P)
        view, vlen, S = oquest.quest_select(qg[None], kmin, kmax, [L], P, k)
        out, lse, _ = oracle.decode_attention(qg[None], Ks[None, None, :L], Vs[None, None, :L], [L],
                                              cfg.softmax_scale, view, vlen, P)
        npv = oquest.n_pages(L, P)
        res[s] = dict(codes=digest(np.stack([kc[:L], vc[:L]])), scales=digest(np.stack([ksb[:L], vsb[:L]])),
                      meta=digest(np.stack([kmin[0, 0, :npv], kmax[0, 0, :npv]])), score=S[0, 0, :npv],
                      view=view[0, 0], vlen=int(vlen[0, 0]), out=out[0], lse=lse[0])
    return res


# ------------------------------------------------------------------ SnapKV

def snap_unit(job):
    """One unit of the SnapKV eviction: window votes, kept positions and the boundary
    gap of the kept set (the input's distance from a near-tie); then decode steps over
    the compacted cache (the kept rows, one appended row per step) with the attention
    output and lse at each checked step."""
    spec, unit, attempt, budget, decode_checks = job
    cfg = cfg_of(spec)
    L, W = cfg.context, cfg.snap_window
    K, V = gen.unit_kv(cfg, 0, unit, L)
    qo = gen.unit_obs_queries(cfg, 0, unit, attempt)
    votes = osnap.unit_votes(qo, K, L, W, cfg.softmax_scale)
    pooled = osnap.snapkv_pool(votes, cfg.snap_pool)
    kept = osnap.snapkv_keep(pooled, L, W, budget)
    gap = np.inf if budget >= L else oracle.boundary_gap(pooled, budget - W)
    decode = {}
    if decode_checks:
        ks, vs = appended_rows(cfg, 0, unit, max(decode_checks) + 1)
        Kc = np.concatenate([osnap.snapkv_compact(K, kept), np.stack(ks)])
        Vc = np.concatenate([osnap.snapkv_compact(V, kept), np.stack(vs)])
        for s in decode_checks:
            n = len(kept) + s + 1
            qg = gen.unit_query(cfg, 0, s, unit)
            out, lse, _ = oracle.unit_attention(qg, Kc[:n], Vc[:n], cfg.softmax_scale)
            decode[s] = (out, lse)
    return dict(votes=votes, kept=kept, gap=gap, decode=decode)


# ------------------------------------------------------------------ H2O

def h2o_start(cfg, unit):
    cap = cfg.h2o_heavy + cfg.h2o_recent + 1
    k = gen.unit_rows(cfg, 0, gen.T_K, unit, cap, cfg.d_k)
    v = gen.unit_rows(cfg, 0, gen.T_V, unit, cap, cfg.d_v)
    pos, acc = gen.h2o_initial_state(cfg, 0, unit)
    return k, v, pos, acc


def h2o_unit(job):
    """Every decode step of one H2O unit from its post-prefill state: evicted slot, slot
    positions, scores and output per step, and the eviction decision's gap per step."""
    spec, unit, attempts = job
    cfg = cfg_of(spec)
    b, h = divmod(unit, cfg.n_kv_heads)
    k, v, pos, acc = h2o_start(cfg, unit)
    acc = acc.astype(np.float64)
    n, free = k.shape[0], k.shape[0] - 1
    T = cfg.decode_steps
    ev = np.zeros(T, np.int32)
    P = np.zeros((T, n), np.int32)
    A = np.zeros((T, n))
    O = np.zeros((T, cfg.group, cfg.d_v))
    gaps = np.full(T, np.inf)
    for t in range(T):
        qg = gen.unit_query(cfg, 0, t, unit, attempts.get(t, 0))
        kn, vn = gen.decode_kv_new(cfg, 0, t)
        g = []
        o, _, pos, acc, n, free = oh2o.h2o_step(k, v, pos, acc, n, free, qg, kn[b, h], vn[b, h], cfg.context + t,
                                                cfg.h2o_heavy, cfg.h2o_recent, cfg.softmax_scale, g)
        ev[t], P[t], A[t], O[t] = free, pos, acc, o
        if g:
            gaps[t] = g[0]
    return dict(evict=ev, pos=P, acc=A, out=O, gaps=gaps)


# ------------------------------------------------------------------ OmniKV

def omni_unit(job):
    """The whole layer sweep of one OmniKV unit at each checked decode step: every
    layer's output, each filter layer's view and its top-k boundary gap."""
    spec, unit, check_steps, attempts = job
    cfg = cfg_of(spec)
    b, h = divmod(unit, cfg.n_kv_heads)
    cap = cfg.context + max(check_steps) + 1
    Ks, Vs = [], []
    for layer in range(cfg.omni_layers):
        kk, vv = gen.unit_kv(cfg, layer, unit, cfg.context)
        Kl = np.zeros((cap, cfg.d_k), np.float32)
        Vl = np.zeros((cap, cfg.d_v), np.float32)
        Kl[:cfg.context], Vl[:cfg.context] = kk, vv
        Ks.append(Kl)
        Vs.append(Vl)
    res = {}
    for s in range(max(check_steps) + 1):
        for layer in range(cfg.omni_layers):
            kn, vn = gen.decode_kv_new(cfg, layer, s)
            Ks[layer][cfg.context + s], Vs[layer][cfg.context + s] = kn[b, h], vn[b, h]
        if s not in check_steps:
            continue
        n = cfg.context + s + 1
        qs = [gen.unit_query(cfg, layer, s, unit, attempts.get((layer, s), 0)) for layer in range(cfg.omni_layers)]
        gaps = {}
        outs, views = oomni.unit_sweep(qs, Ks, Vs, n, cfg.omni_filters, cfg.omni_top_k, cfg.softmax_scale, gaps=gaps)
        res[s] = dict(outs=outs, views=views, gaps=gaps)
    return res


# ------------------------------------------------------------------ MLA

def mla_row(job):
    """One batch row of the MLA latent Quest decode at each checked step: metadata
    digest, page scores, view, and the attention output and lse."""
    spec, row, check_steps = job
    cfg = cfg_of(spec)
    P, k, Dv = cfg.page_size, cfg.top_pages, cfg.d_v
    C, _ = gen.unit_kv(cfg, 0, row, cfg.context)
    ks, _ = appended_rows(cfg, 0, row, max(check_steps) + 1)
    C = np.concatenate([C, np.stack(ks)])
    res = {}
    for s in check_steps:
        L = cfg.context + s + 1
        q = gen.unit_query(cfg, 0, s, row)[None]                    # [1][32][576]
        Cb = C[None, None, :L]
        kmin, kmax = oquest.page_meta(Cb, [L], P)
        view, vlen, S = oquest.quest_select(q, kmin, kmax, [L], P, k)
        out, lse, _ = oracle.decode_attention(q, Cb, None, [L], cfg.softmax_scale, view, vlen, P, latent_dv=Dv)
        npv = oquest.n_pages(L, P)
        res[s] = dict(meta=digest(np.stack([kmin[0, 0, :npv], kmax[0, 0, :npv]])), score=S[0, 0, :npv],
                      view=view[0, 0], vlen=int(vlen[0, 0]), out=out[0], lse=lse[0])
    return res
