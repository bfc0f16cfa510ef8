"""Workload builders shared by the H2O / OmniKV parity tests and the attempt search
(input assembly only: every score and decision comes from the oracle or the GPU)."""
import numpy as np

from workloads import generator as gen
from workloads import get_config


def h2o_config(full: bool):
    if full:
        return get_config(3)
    return get_config(3, batch=2, n_q_heads=8, n_kv_heads=2, context=96, h2o_heavy=12, h2o_recent=6,
                      decode_steps=24)


def omni_config(full: bool):
    if full:
        return get_config(3, omni_layers=18)
    return get_config(3, batch=2, n_q_heads=8, n_kv_heads=2, context=200, omni_layers=6, omni_filters=(1, 3),
                      omni_top_k=40, extra={"omni_steps": 3})


def h2o_unit_start(cfg, unit):
    """(K slots [cap][D], V slots [cap][D], slot_pos [cap], acc [cap]) of one unit after prefill."""
    cap = cfg.h2o_heavy + cfg.h2o_recent + 1
    k = gen.unit_rows(cfg, 0, gen.T_K, unit, cap, cfg.d_k)
    v = gen.unit_rows(cfg, 0, gen.T_V, unit, cap, cfg.d_v)
    pos, acc = gen.h2o_initial_state(cfg, 0, unit)
    return k, v, pos, acc


def h2o_step_inputs(cfg, step, attempts=None):
    """q [B][Hq][D], k_new / v_new [B][Hkv][D] of decode step `step` (layer 0)."""
    q = gen.decode_query(cfg, 0, step, attempts)
    kn, vn = gen.decode_kv_new(cfg, 0, step)
    return q, kn, vn


def omni_layer_kv(cfg, layer, units=None):
    """[B][Hkv][ctx + steps][D] K and V of one layer (float32, zero past the prompt)."""
    cap = cfg.context + cfg.extra["omni_steps"]
    return gen.cache_kv(cfg, layer, cap, units=units)


def relative_gap(values, lo_value):
    values = np.asarray(values, np.float64)
    d = np.abs(values - lo_value)
    d = d[d > 0]
    return float(d.min() / abs(lo_value)) if d.size and lo_value != 0 else np.inf
