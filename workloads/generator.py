"""Seeded grid-valued inputs.

Every value is round(32 x) / 32 clipped to +-255/32 with x ~ N(0, 1): such a
value has at most 8 significant bits, so it is exact in bf16 and fp32, and
every product of two of them is a multiple of 2^-10.  Sums of such products
are then exact in fp32 in any order while their absolute sum stays below
2^14, which is what lets a GPU and a CPU reach bit-identical dot products.

Each (config, layer, tensor, unit, step, attempt) block is drawn from its own
PCG64 stream, so any one unit (a batch row and KV head) can be regenerated on
its own, and a unit's decode query can be redrawn (attempt + 1) without
touching anything else.  The attempt numbers are plain data handed in by the
caller.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from typing import Dict, Iterable, Optional, Tuple

import numpy as np

from .configs import WorkloadConfig

GRID = 32.0
CLIP = 255.0
_ROOT = 0x5E5D0C0DE

# tensor tags
T_K, T_V, T_Q, T_KNEW, T_VNEW, T_QOBS, T_DIR, T_PLANT, T_PLANTSEL, T_HEAVY, T_ACC = range(1, 12)

Attempts = Dict[Tuple[int, int, int], int]   # (layer, step, unit) -> attempt


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def rng_for(*words: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([_ROOT, *[int(w) for w in words]])))


def quantize_(x: np.ndarray) -> np.ndarray:
    """In place: x -> clip(round(32 x), -255, 255) / 32 (float32, exact, no negative zero)."""
    np.multiply(x, GRID, out=x)
    np.rint(x, out=x)
    np.clip(x, -CLIP, CLIP, out=x)
    np.multiply(x, 1.0 / GRID, out=x)
    np.add(x, 0.0, out=x)          # -0.0 -> +0.0
    return x


def grid_normal(words: Iterable[int], shape) -> np.ndarray:
    x = rng_for(*words).standard_normal(shape, dtype=np.float32)
    return quantize_(x)


def _parallel(fn, items):
    items = list(items)
    if len(items) <= 1:
        return [fn(i) for i in items]
    with _cf.ThreadPoolExecutor(_threads()) as ex:
        return list(ex.map(fn, items))


# ---------------------------------------------------------------- KV caches

def unit_rows(cfg: WorkloadConfig, layer: int, tensor: int, unit: int, length: int, width: int) -> np.ndarray:
    """[length][width] grid rows of one unit's K (or V) cache."""
    return grid_normal((cfg.cfg_id, layer, tensor, unit), (length, width))


def _planted(cfg: WorkloadConfig, layer: int, unit: int):
    """Direction u and the planted page ids of one unit (Quest workload)."""
    r = rng_for(cfg.cfg_id, layer, T_DIR, unit)
    u = r.standard_normal(cfg.d_k, dtype=np.float32)
    region = min(cfg.planted_region_pages, cfg.context // cfg.page_size)
    pages = np.sort(rng_for(cfg.cfg_id, layer, T_PLANTSEL, unit).choice(region, cfg.planted_pages, replace=False))
    return u, pages


def planted_pages(cfg: WorkloadConfig, layer: int, unit: int) -> np.ndarray:
    return _planted(cfg, layer, unit)[1]


def unit_kv(cfg: WorkloadConfig, layer: int, unit: int, length: Optional[int] = None):
    """(K, V) rows of one unit at prefill end: [length][d_k], [length][d_v] (V None for latent caches)."""
    L = cfg.context if length is None else length
    k = unit_rows(cfg, layer, T_K, unit, L, cfg.d_k)
    if cfg.planted_pages:
        u, pages = _planted(cfg, layer, unit)
        P = cfg.page_size
        noise = rng_for(cfg.cfg_id, layer, T_PLANT, unit).standard_normal((len(pages), P, cfg.d_k), dtype=np.float32)
        for i, p in enumerate(pages):
            if (p + 1) * P <= L:
                rows = 0.8 * u[None, :] + 0.2 * noise[i]
                k[p * P:(p + 1) * P] = quantize_(rows.astype(np.float32))
    if cfg.snap_peaks:
        for pos, key in zip(*_snap_peaks(cfg, layer, unit)):
            if pos < L:
                k[pos] = key
    v = None if cfg.latent else unit_rows(cfg, layer, T_V, unit, L, cfg.d_v)
    return k, v


def _snap_direction(cfg: WorkloadConfig, layer: int, unit: int) -> np.ndarray:
    return rng_for(cfg.cfg_id, layer, T_DIR, unit).standard_normal(cfg.d_k, dtype=np.float32)


def _snap_peaks(cfg: WorkloadConfig, layer: int, unit: int):
    """Planted SnapKV keys of one unit: (positions, rows).  Peak j sits at position
    48 + spacing * j and its key is a_l * sign(u) with level l = j mod levels and
    a_l = 2 + l / 32 (exact grid values), u being the unit's query direction.  With
    the window queries drawn around u, the peaks' votes form a ladder of distinct
    levels far above the random keys, so the kept set's boundary falls between
    well-separated vote levels."""
    sgn = np.where(_snap_direction(cfg, layer, unit) >= 0, 1.0, -1.0).astype(np.float32)
    j = np.arange(cfg.snap_peaks)
    pos = 48 + cfg.snap_peak_spacing * j
    a = (2.0 + (j % cfg.snap_peak_levels) / 32.0).astype(np.float32)
    return pos, a[:, None] * sgn[None, :]


def snap_peak_positions(cfg: WorkloadConfig) -> np.ndarray:
    return 48 + cfg.snap_peak_spacing * np.arange(cfg.snap_peaks)


def cache_kv(cfg: WorkloadConfig, layer: int, capacity: int, length: Optional[int] = None,
             units: Optional[Iterable[int]] = None):
    """Full caches [B][Hkv][capacity][d] (float32, zero past `length`); V is None for latent caches."""
    L = cfg.context if length is None else length
    B, H = cfg.batch, cfg.n_kv_heads
    K = np.zeros((B, H, capacity, cfg.d_k), np.float32)
    V = None if cfg.latent else np.zeros((B, H, capacity, cfg.d_v), np.float32)
    todo = list(range(B * H)) if units is None else list(units)

    def one(u):
        k, v = unit_kv(cfg, layer, u, L)
        K[u // H, u % H, :L] = k
        if V is not None:
            V[u // H, u % H, :L] = v
    _parallel(one, todo)
    return K, V


# ---------------------------------------------------------------- decode inputs

def unit_query(cfg: WorkloadConfig, layer: int, step: int, unit: int, attempt: int = 0) -> np.ndarray:
    """[G][d_k] decode queries of the G query heads that read KV head `unit`."""
    G = cfg.group
    if cfg.planted_pages:
        u, _ = _planted(cfg, layer, unit)
        eps = rng_for(cfg.cfg_id, layer, T_Q, step, unit, attempt).standard_normal((G, cfg.d_k), dtype=np.float32)
        return quantize_((u[None, :] + 0.5 * eps).astype(np.float32))
    return grid_normal((cfg.cfg_id, layer, T_Q, step, unit, attempt), (G, cfg.d_k))


def decode_query(cfg: WorkloadConfig, layer: int, step: int, attempts: Optional[Attempts] = None) -> np.ndarray:
    """q [B][Hq][d_k]; query head h reads KV head h // G."""
    B, H, G = cfg.batch, cfg.n_kv_heads, cfg.group
    q = np.empty((B, H * G, cfg.d_k), np.float32)
    for u in range(B * H):
        a = (attempts or {}).get((layer, step, u), 0)
        q[u // H, (u % H) * G:(u % H + 1) * G] = unit_query(cfg, layer, step, u, a)
    return q


def decode_kv_new(cfg: WorkloadConfig, layer: int, step: int):
    """Rows appended at this step: k_new [B][Hkv][d_k], v_new [B][Hkv][d_v] (None for latent)."""
    B, H = cfg.batch, cfg.n_kv_heads
    k = grid_normal((cfg.cfg_id, layer, T_KNEW, step), (B, H, cfg.d_k))
    v = None if cfg.latent else grid_normal((cfg.cfg_id, layer, T_VNEW, step), (B, H, cfg.d_v))
    return k, v


# ---------------------------------------------------------------- SnapKV

def unit_obs_queries(cfg: WorkloadConfig, layer: int, unit: int, attempt: int = 0) -> np.ndarray:
    """[G][window][d_k]: queries of the last `window` prompt tokens for the G heads of one KV head.
    With planted peaks the queries are u + 0.5 eps around the unit's direction u."""
    shape = (cfg.group, cfg.snap_window, cfg.d_k)
    if cfg.snap_peaks:
        u = _snap_direction(cfg, layer, unit)
        eps = rng_for(cfg.cfg_id, layer, T_QOBS, unit, attempt).standard_normal(shape, dtype=np.float32)
        return quantize_((u + 0.5 * eps).astype(np.float32))
    return grid_normal((cfg.cfg_id, layer, T_QOBS, unit, attempt), shape)


def obs_queries(cfg: WorkloadConfig, layer: int, attempts: Optional[Attempts] = None) -> np.ndarray:
    """q_obs [B][Hq][window][d_k]."""
    B, H, G = cfg.batch, cfg.n_kv_heads, cfg.group
    q = np.empty((B, H * G, cfg.snap_window, cfg.d_k), np.float32)
    for u in range(B * H):
        a = (attempts or {}).get((layer, 0, u), 0)
        q[u // H, (u % H) * G:(u % H + 1) * G] = unit_obs_queries(cfg, layer, u, a)
    return q


# ---------------------------------------------------------------- H2O state after prefill

def h2o_initial_state(cfg: WorkloadConfig, layer: int, unit: int):
    """Synthetic post-prefill H2O state of one unit.

    Returns (slot_pos [cap] int32 with -1 for the one free slot, acc [cap] float32).
    The heavy hitters are `heavy` distinct positions drawn uniformly below the
    recent window, the recent window holds the last `recent` prompt positions,
    and the accumulated scores start as G * U(0, 1)."""
    heavy, recent, L = cfg.h2o_heavy, cfg.h2o_recent, cfg.context
    cap = heavy + recent + 1
    pos = np.sort(rng_for(cfg.cfg_id, layer, T_HEAVY, unit).choice(L - recent, heavy, replace=False)).astype(np.int32)
    slot_pos = np.full(cap, -1, np.int32)
    slot_pos[:heavy] = pos
    slot_pos[heavy:heavy + recent] = np.arange(L - recent, L, dtype=np.int32)
    acc = np.zeros(cap, np.float32)
    acc[:heavy + recent] = cfg.group * rng_for(cfg.cfg_id, layer, T_ACC, unit).random(heavy + recent, dtype=np.float32)
    return slot_pos, acc
