"""Finds, with the CPU oracle only, the seeded query draws that keep every
selection decision of the parity cases clear of near-ties, and writes them to
attempts.json beside this script.

A decision (top-k boundary, H2O argmin) is accepted when the oracle's float64
scores put at least GAP relative distance between the kept side and the rest;
otherwise the unit's query of that step is redrawn with attempt + 1.  float32
rounding of the GPU scores (a few ulp of accumulated error) cannot reorder such
decisions.  The searches are independent per unit and run in a process pool.
Run: python tests/golden/make_attempts.py [--only SECTION[,SECTION..]]
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import boundary_gap  # noqa: E402
from oracle import h2o as oh2o  # noqa: E402
from oracle import omnikv as oomni  # noqa: E402
from oracle import snapkv as osnap  # noqa: E402
from oracle.attention import unit_attention  # noqa: E402
from tests.h2o_omni_cases import (CHAIN_BUDGET2, CHAIN_CASES, CHAIN_TAGS, CHAIN_TURN2, OMNI_STEPS,  # noqa: E402
                                  OMNI_UNITS, PREFILL_CASES, PREFILL_DECODE_CFG, PREFILL_DECODE_LAYER,
                                  PREFILL_KV_LAYER, PYRAMID_CASES, PYRAMID_LAYERS, h2o_config, omni_config,
                                  prefill_unit_queries)
from workloads import generator as gen  # noqa: E402
from workloads import get_config  # noqa: E402

GAP = 1e-4
MAX_ATTEMPTS = 64
OUT = os.path.join(HERE, "attempts.json")


def key(*parts):
    return ",".join(str(int(p)) for p in parts)


def h2o_steps_from(cfg, layer, unit, k, v, pos, acc, t_steps, cur0):
    """Attempt per step of one unit's H2O decode from the given slot state: the step's
    query is redrawn until its eviction decision clears GAP.  Returns {step: attempt}."""
    b, h = divmod(unit, cfg.n_kv_heads)
    acc = np.asarray(acc, np.float64)
    n, free = k.shape[0], k.shape[0] - 1
    found = {}
    for t in range(t_steps):
        kn, vn = gen.decode_kv_new(cfg, layer, t)
        for attempt in range(MAX_ATTEMPTS):
            qg = gen.unit_query(cfg, layer, t, unit, attempt)
            k2, v2 = k.copy(), v.copy()
            gaps = []
            res = oh2o.h2o_step(k2, v2, pos, acc, n, free, qg, kn[b, h], vn[b, h], cur0 + t, cfg.h2o_heavy,
                                cfg.h2o_recent, cfg.softmax_scale, gaps)
            if not gaps or gaps[0] >= GAP:
                break
        else:
            raise RuntimeError(f"no clear draw for h2o unit {unit} step {t}")
        if attempt:
            found[t] = attempt
        k, v = k2, v2
        _, _, pos, acc, n, free = res
    return found


def h2o_unit_job(unit):
    """The 16K H2O workload, one unit, every decode step from the synthetic prefill state."""
    cfg = h2o_config(True)
    cap = cfg.h2o_heavy + cfg.h2o_recent + 1
    k = gen.unit_rows(cfg, 0, gen.T_K, unit, cap, cfg.d_k)
    v = gen.unit_rows(cfg, 0, gen.T_V, unit, cap, cfg.d_v)
    pos, acc = gen.h2o_initial_state(cfg, 0, unit)
    found = h2o_steps_from(cfg, 0, unit, k, v, pos, acc, cfg.decode_steps, cfg.context)
    return {key(0, t, unit): a for t, a in found.items()}


def omni_unit_job(unit):
    """The 16K OmniKV workload, one unit: per checked step and filter layer, the query
    draw whose top-k boundary clears GAP (a filter layer's view depends on its own
    query and rows only)."""
    cfg = omni_config(True)
    b, h = divmod(unit, cfg.n_kv_heads)
    cap = cfg.context + max(OMNI_STEPS) + 1
    layers = {}
    for f in cfg.omni_filters:
        kk, vv = gen.unit_kv(cfg, f, unit, cfg.context)
        K = np.zeros((cap, cfg.d_k), np.float32)
        V = np.zeros((cap, cfg.d_v), np.float32)
        K[:cfg.context], V[:cfg.context] = kk, vv
        for s in range(cap - cfg.context):
            kn, vn = gen.decode_kv_new(cfg, f, s)
            K[cfg.context + s], V[cfg.context + s] = kn[b, h], vn[b, h]
        layers[f] = (K, V)
    found = {}
    for s in OMNI_STEPS:
        n = cfg.context + s + 1
        for f in cfg.omni_filters:
            K, V = layers[f]
            for attempt in range(MAX_ATTEMPTS):
                qg = gen.unit_query(cfg, f, s, unit, attempt)
                _, lse, logits = unit_attention(qg, K[:n], V[:n], cfg.softmax_scale)
                if boundary_gap(oomni.omnikv_scores(logits, lse, n), cfg.omni_top_k) >= GAP:
                    break
            else:
                raise RuntimeError(f"no clear draw for omnikv unit {unit} step {s} layer {f}")
            if attempt:
                found[key(f, s, unit)] = attempt
    return found


def snap_unit_job(args):
    """A SnapKV eviction, one unit: the window-query draw whose kept-set boundary clears GAP."""
    cfg_id, kw, layer, unit, budget = args
    cfg = get_config(cfg_id, **kw)
    L, W = cfg.context, cfg.snap_window
    k, _ = gen.unit_kv(cfg, layer, unit, L)
    for attempt in range(MAX_ATTEMPTS):
        qo = gen.unit_obs_queries(cfg, layer, unit, attempt)
        votes = osnap.unit_votes(qo, k, L, W, cfg.softmax_scale)
        pooled = osnap.snapkv_pool(votes, cfg.snap_pool)
        if budget >= L or boundary_gap(pooled, budget - W) >= GAP:
            return {key(layer, 0, unit): attempt} if attempt else {}
    raise RuntimeError(f"no clear draw for snapkv unit {unit} layer {layer}")


def prefill_unit_job(args):
    """The prefill-end H2O state, one unit: the prompt-query draw whose heavy-hitter
    boundary clears GAP."""
    name, unit = args
    cfg, L, heavy, recent = PREFILL_CASES[name]
    tag = list(PREFILL_CASES).index(name)
    K, _ = gen.cache_kv(cfg, PREFILL_KV_LAYER, L + 7, length=L + 7)
    b, h = divmod(unit, cfg.n_kv_heads)
    scale = 1.0 / np.sqrt(cfg.d_k)
    if heavy + recent >= L:
        return name, unit, 0
    for attempt in range(MAX_ATTEMPTS):
        q = prefill_unit_queries(cfg, tag, L, unit, attempt)
        acc0 = oh2o.prefill_scores(q, K[b, h], L, scale)
        if boundary_gap(acc0[:L - recent], heavy) >= GAP:
            return name, unit, attempt
    raise RuntimeError(f"no clear draw for prefill case {name} unit {unit}")


def prefill_decode_unit_job(unit):
    """The prefill-end state continued by H2O decode steps, one unit: first the prompt
    draw, then each step's query draw, all from the oracle's own state."""
    cfg = PREFILL_DECODE_CFG
    L, heavy, recent = cfg.context, cfg.h2o_heavy, cfg.h2o_recent
    cap = heavy + recent + 1
    b, h = divmod(unit, cfg.n_kv_heads)
    K, V = gen.cache_kv(cfg, PREFILL_DECODE_LAYER, L, length=L)
    for attempt in range(MAX_ATTEMPTS):
        q = prefill_unit_queries(cfg, 99, L, unit, attempt)
        acc0 = oh2o.prefill_scores(q, K[b, h], L, cfg.softmax_scale)
        if boundary_gap(acc0[:L - recent], heavy) >= GAP:
            break
    else:
        raise RuntimeError(f"no clear prompt draw for unit {unit}")
    kept, pos, acc = oh2o.prefill_state(acc0, L, heavy, recent, cap)
    k = np.zeros((cap, cfg.d_k))
    v = np.zeros((cap, cfg.d_v))
    k[:len(kept)], v[:len(kept)] = K[b, h][kept], V[b, h][kept]
    steps = h2o_steps_from(cfg, PREFILL_DECODE_LAYER, unit, k, v, pos, acc, cfg.decode_steps, L)
    return unit, attempt, steps


def chain_unit_job(args):
    """Chain Cache over two turns, one unit: the window-query draw of the turn-1
    compaction, then (over the oracle's chained rows: the kept prompt rows and the
    turn-2 rows) the draw of the turn-2 compaction, each clearing GAP."""
    name, unit = args
    cfg = CHAIN_CASES[name]
    b, h = divmod(unit, cfg.n_kv_heads)
    L1, W = cfg.context, cfg.snap_window
    Klog, _ = gen.cache_kv(cfg, CHAIN_TAGS[0], L1 + CHAIN_TURN2, length=L1 + CHAIN_TURN2)
    found = {}

    def search(tag, rows, n, budget):
        for attempt in range(MAX_ATTEMPTS):
            qo = gen.unit_obs_queries(cfg, tag, unit, attempt)
            pooled = osnap.snapkv_pool(osnap.unit_votes(qo, rows, n, W, cfg.softmax_scale), cfg.snap_pool)
            if boundary_gap(pooled, budget - W) >= GAP:
                if attempt:
                    found[key(tag, 0, unit)] = attempt
                return osnap.snapkv_keep(pooled, n, W, budget)
        raise RuntimeError(f"no clear draw for chain {name} unit {unit} tag {tag}")

    kept = search(CHAIN_TAGS[0], Klog[b, h], L1, cfg.snap_budget)
    pos = np.concatenate([kept, np.arange(L1, L1 + CHAIN_TURN2)])
    search(CHAIN_TAGS[1], Klog[b, h][pos], len(pos), CHAIN_BUDGET2)
    return name, found


def section_h2o_16k(pool, out, t0):
    cfg = h2o_config(True)
    out["h2o_16k"] = {}
    for d in pool.map(h2o_unit_job, range(cfg.units)):
        out["h2o_16k"].update(d)
    print(f"h2o_16k: {len(out['h2o_16k'])} redraws ({time.time() - t0:.0f}s)", flush=True)


def section_omnikv_16k(pool, out, t0):
    out["omnikv_16k"] = {}
    for d in pool.map(omni_unit_job, OMNI_UNITS):
        out["omnikv_16k"].update(d)
    print(f"omnikv_16k: {len(out['omnikv_16k'])} redraws ({time.time() - t0:.0f}s)", flush=True)


def section_snapkv(pool, out, t0):
    for name, cfg_id in (("snapkv_128k", 2), ("snapkv_tiny", 0)):
        c = get_config(cfg_id)
        out[name] = {}
        for d in pool.map(snap_unit_job, [(cfg_id, {}, 0, u, c.snap_budget) for u in range(c.units)]):
            out[name].update(d)
        print(f"{name}: {len(out[name])} redraws ({time.time() - t0:.0f}s)", flush=True)


def section_pyramid(pool, out, t0):
    out["pyramid"] = {}
    from oracle import variants as ov
    for name, (c, avg, bmin) in PYRAMID_CASES.items():
        budgets = ov.pyramid_budgets(PYRAMID_LAYERS, avg, bmin)
        kw = {f: getattr(c, f) for f in ("dtype", "batch", "n_q_heads", "n_kv_heads", "d_k", "d_v", "context",
                                         "snap_window", "snap_pool", "snap_budget", "snap_peaks", "snap_peak_spacing",
                                         "snap_peak_levels")}
        jobs = [(c.cfg_id, kw, layer, u, budgets[layer]) for layer in range(PYRAMID_LAYERS) for u in range(c.units)]
        out["pyramid"][name] = {}
        for d in pool.map(snap_unit_job, jobs):
            out["pyramid"][name].update(d)
        print(f"pyramid {name}: {len(out['pyramid'][name])} redraws ({time.time() - t0:.0f}s)", flush=True)


def section_h2o_prefill(pool, out, t0):
    out["h2o_prefill"] = {name: {} for name in PREFILL_CASES}
    jobs = [(name, u) for name, (c, _, _, _) in PREFILL_CASES.items() for u in range(c.units)]
    for name, unit, attempt in pool.map(prefill_unit_job, jobs):
        if attempt:
            out["h2o_prefill"][name][str(unit)] = attempt
    print(f"h2o_prefill: {out['h2o_prefill']} ({time.time() - t0:.0f}s)", flush=True)


def section_h2o_prefill_decode(pool, out, t0):
    dec = {"prompt": {}, "steps": {}}
    for unit, attempt, steps in pool.map(prefill_decode_unit_job, range(PREFILL_DECODE_CFG.units)):
        if attempt:
            dec["prompt"][str(unit)] = attempt
        for t, a in steps.items():
            dec["steps"][key(t, unit)] = a
    out["h2o_prefill_decode"] = dec
    print(f"h2o_prefill_decode: {dec} ({time.time() - t0:.0f}s)", flush=True)


def section_chain(pool, out, t0):
    out["chain"] = {name: {} for name in CHAIN_CASES}
    for name, found in pool.map(chain_unit_job, [(n, u) for n, c in CHAIN_CASES.items() for u in range(c.units)]):
        out["chain"][name].update(found)
    print(f"chain: {out['chain']} ({time.time() - t0:.0f}s)", flush=True)


SECTIONS = {"h2o_16k": section_h2o_16k, "omnikv_16k": section_omnikv_16k, "snapkv": section_snapkv,
            "pyramid": section_pyramid, "h2o_prefill": section_h2o_prefill,
            "h2o_prefill_decode": section_h2o_prefill_decode, "chain": section_chain}


def main(argv=None):
    """Every section, or with --only NAME[,NAME..] those sections recomputed into the
    existing attempts.json (the others kept as they are)."""
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--only", default="", help="comma-separated sections: " + ", ".join(SECTIONS))
    args = ap.parse_args(argv)
    only = [n for n in args.only.split(",") if n]
    for n in only:
        if n not in SECTIONS:
            raise SystemExit(f"unknown section {n}; sections: {', '.join(SECTIONS)}")
    from tests import oracle_pool
    t0 = time.time()
    pool = oracle_pool.pool()
    if only:
        with open(OUT) as f:
            out = json.load(f)
        assert out["gap"] == GAP, "the stored draws were searched with another gap"
    else:
        out = {"gap": GAP}
    for name, fn in SECTIONS.items():
        if not only or name in only:
            fn(pool, out, t0)
    oracle_pool.shutdown()
    with open(OUT, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print("wrote", OUT)


if __name__ == "__main__":
    from tests.golden.make_attempts import main as _main   # jobs pickled by this module's name
    _main()
