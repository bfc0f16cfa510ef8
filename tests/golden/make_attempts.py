"""Finds, with the CPU oracle only, the seeded query draws that keep every
selection decision of the full-size parity cases clear of near-ties, and writes
them to attempts.json beside this script.

A decision (top-k boundary, H2O argmin) is accepted when the oracle's float64
scores put at least GAP relative distance between the kept side and the rest;
otherwise the unit's query of that step is redrawn with attempt + 1.  float32
rounding of the GPU scores (a few ulp of accumulated error) cannot reorder such
decisions.  Run: python tests/golden/make_attempts.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import h2o as oh2o  # noqa: E402
from oracle import omnikv as oomni  # noqa: E402
from oracle import snapkv as osnap  # noqa: E402
from oracle import boundary_gap  # noqa: E402
from oracle.attention import unit_attention  # noqa: E402
from tests.h2o_omni_cases import h2o_config, h2o_step_inputs, h2o_unit_start, omni_config  # noqa: E402
from tests.sampled_units import H2O_UNITS, OMNI_STEPS, OMNI_UNITS, SNAP_UNITS  # noqa: E402
from workloads import generator as gen  # noqa: E402
from workloads import get_config  # noqa: E402

GAP = 1e-4
OUT = os.path.join(HERE, "attempts.json")


def key(layer, step, unit):
    return f"{layer},{step},{unit}"


def h2o_attempts(cfg, units):
    """Sequential per unit: redraw the step's query until the eviction gap clears GAP."""
    found = {}
    G = cfg.group
    for unit in units:
        b, h = divmod(unit, cfg.n_kv_heads)
        k, v, pos, acc = h2o_unit_start(cfg, unit)
        acc = acc.astype(np.float64)
        n, free = k.shape[0], k.shape[0] - 1
        for t in range(cfg.decode_steps):
            _, kn, vn = h2o_step_inputs(cfg, t)
            for attempt in range(64):
                qg = gen.unit_query(cfg, 0, t, unit, attempt)
                k2, v2 = k.copy(), v.copy()
                gaps = []
                res = oh2o.h2o_step(k2, v2, pos, acc, n, free, qg, kn[b, h], vn[b, h], cfg.context + t,
                                    cfg.h2o_heavy, cfg.h2o_recent, cfg.softmax_scale, gaps)
                if not gaps or gaps[0] >= GAP:
                    break
            else:
                raise RuntimeError(f"no clear draw for h2o unit {unit} step {t}")
            if attempt:
                found[key(0, t, unit)] = attempt
            k, v = k2, v2
            _, _, pos, acc, n, free = res
    return found


def omni_attempts(cfg, units, steps):
    """Per (unit, step): redraw the filter layers' queries until every boundary gap clears GAP."""
    found = {}
    G = cfg.group
    cap = cfg.context + cfg.extra["omni_steps"]
    last_filter = max(cfg.omni_filters)
    for unit in units:
        b, h = divmod(unit, cfg.n_kv_heads)
        Ks, Vs = [], []
        for layer in range(last_filter + 1):
            k, v = gen.unit_kv(cfg, layer, unit, cap)
            k[cfg.context:] = 0
            v[cfg.context:] = 0
            Ks.append(k)
            Vs.append(v)
        for s in range(max(steps) + 1):
            for layer in range(last_filter + 1):
                kn, vn = gen.decode_kv_new(cfg, layer, s)
                Ks[layer][cfg.context + s], Vs[layer][cfg.context + s] = kn[b, h], vn[b, h]
            if s not in steps:
                continue
            n = cfg.context + s + 1
            for f in cfg.omni_filters:
                for attempt in range(64):
                    qg = gen.unit_query(cfg, f, s, unit, attempt)
                    _, lse, logits = unit_attention(qg, Ks[f][:n], Vs[f][:n], cfg.softmax_scale)
                    if boundary_gap(oomni.omnikv_scores(logits, lse, n), cfg.omni_top_k) >= GAP:
                        break
                else:
                    raise RuntimeError(f"no clear draw for omnikv unit {unit} step {s} layer {f}")
                if attempt:
                    found[key(f, s, unit)] = attempt
    return found


def snap_attempts(cfg, units):
    found = {}
    L, W = cfg.context, cfg.snap_window
    for unit in units:
        k, _ = gen.unit_kv(cfg, 0, unit, L)
        for attempt in range(64):
            qo = gen.unit_obs_queries(cfg, 0, unit, attempt)
            votes = osnap.unit_votes(qo, k, L, W, cfg.softmax_scale)
            pooled = osnap.snapkv_pool(votes, cfg.snap_pool)
            if cfg.snap_budget >= L or boundary_gap(pooled, cfg.snap_budget - W) >= GAP:
                break
        else:
            raise RuntimeError(f"no clear draw for snapkv unit {unit}")
        if attempt:
            found[key(0, 0, unit)] = attempt
        print(f"snapkv unit {unit}: attempt {attempt}", flush=True)
    return found


def main():
    out = {}
    out["h2o_16k"] = h2o_attempts(h2o_config(True), H2O_UNITS)
    print("h2o", out["h2o_16k"], flush=True)
    out["omnikv_16k"] = omni_attempts(omni_config(True), OMNI_UNITS, OMNI_STEPS)
    print("omnikv", out["omnikv_16k"], flush=True)
    out["snapkv_128k"] = snap_attempts(get_config(2), SNAP_UNITS)
    out["snapkv_tiny"] = snap_attempts(get_config(0), range(get_config(0).units))
    print("snapkv", out["snapkv_128k"], flush=True)
    out["gap"] = GAP
    with open(OUT, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
