"""Workload builders shared by the parity tests and the attempt search in
tests/golden/make_attempts.py (input assembly only: every score and decision comes
from the oracle or the GPU)."""
import numpy as np

from workloads import generator as gen
from workloads import get_config


def h2o_config(full: bool):
    if full:
        return get_config(3)
    return get_config(3, batch=2, n_q_heads=8, n_kv_heads=2, context=96, h2o_heavy=12, h2o_recent=6,
                      decode_steps=24)


# OmniKV units (batch row x KV head) compared one by one at full size: every other batch
# row, the KV head rotating, and the decode steps compared (steps 0 .. 63 run)
OMNI_UNITS = tuple(8 * i + (i % 4) for i in range(32))
OMNI_STEPS = (0, 1, 63)


def omni_config(full: bool):
    if full:
        return get_config(3)
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


# ------------------------------------------------------------------ H2O at the end of a prefill

# name -> (config, prompt length, heavy budget, recent window)
PREFILL_CASES = {
    "d128_g8": (get_config(0, dtype="bf16", batch=2, n_q_heads=16, n_kv_heads=2, d_k=128, d_v=128), 700, 64, 32),
    "d128_g16_ragged": (get_config(0, dtype="bf16", batch=1, n_q_heads=32, n_kv_heads=2, d_k=128, d_v=128), 1033, 100,
                        50),
    "d64_g4": (get_config(0, dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2), 333, 40, 16),
    # G = 6: the (position, head) query rows straddle the 16-row MFMA column blocks
    "d128_g6_ragged": (get_config(0, dtype="bf16", batch=2, n_q_heads=12, n_kv_heads=2, d_k=128, d_v=128), 1111, 90,
                       33),
    "keep_all": (get_config(0, dtype="bf16", batch=1, n_q_heads=8, n_kv_heads=2), 90, 64, 32),
    # past one 512-key column block: the column pass's whole-tile path with 64-wide heads
    "d64_g4_long": (get_config(0, dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2), 900, 60, 24),
    # one query head per KV head: the query rows are the positions themselves, two row
    # blocks and three column blocks per unit
    "d128_g1_long": (get_config(0, dtype="bf16", batch=2, n_q_heads=3, n_kv_heads=3, d_k=128, d_v=128), 1500, 120,
                     40),
}
PREFILL_KV_LAYER = 41

# the prefill-end state continued by H2O decode steps
PREFILL_DECODE_CFG = get_config(3, batch=2, n_q_heads=8, n_kv_heads=2, context=200, h2o_heavy=24, h2o_recent=12,
                                decode_steps=6)
PREFILL_DECODE_LAYER = 43


def prefill_unit_queries(cfg, tag, L, unit, attempt=0):
    """[G][L][d] grid queries of every prompt position for the G heads of one KV head."""
    return gen.grid_normal((cfg.cfg_id, 50 + tag, L, unit, attempt), (cfg.group, L, cfg.d_k))


def prefill_queries(cfg, tag, L, attempts=None):
    """[B][Hq][L][d] prompt queries; attempts maps unit -> attempt."""
    B, H, G = cfg.batch, cfg.n_kv_heads, cfg.group
    q = np.empty((B, H * G, L, cfg.d_k), np.float32)
    for u in range(B * H):
        q[u // H, (u % H) * G:(u % H + 1) * G] = prefill_unit_queries(cfg, tag, L, u, (attempts or {}).get(u, 0))
    return q


# ------------------------------------------------------------------ PyramidKV layers

# name -> (config, average budget, smallest budget); four layers each
PYRAMID_CASES = {
    "tiny_f32": (get_config(0), 128, 64),
    "mid_bf16": (get_config(2, batch=2, context=4096, snap_window=8, snap_budget=400, snap_peaks=100,
                            snap_peak_spacing=40, snap_peak_levels=10), 400, 200),
}
PYRAMID_LAYERS = 4


# ------------------------------------------------------------------ Chain Cache over two turns

# dtype -> config: SnapKV at the end of turn 1 (window queries of layer tag 31), turn 2
# appends CHAIN_TURN2 tokens, a second SnapKV (layer tag 32) keeps CHAIN_BUDGET2 rows
CHAIN_CASES = {"f32": get_config(0),
               "bf16": get_config(0, dtype="bf16", batch=2, n_q_heads=16, n_kv_heads=2, d_k=128, d_v=128)}
CHAIN_TURN2, CHAIN_BUDGET2, CHAIN_TAGS = 40, 64, (31, 32)
