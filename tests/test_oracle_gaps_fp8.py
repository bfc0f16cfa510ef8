"""Pins of the near-tie certification (boundary_gap, argmin_gap) and of the
exactness precondition behind bit-exact Quest selection over FP8 rows.

boundary_gap and argmin_gap decide which generated inputs the bit-exact parity
tests may use, so each is pinned twice: against a brute force over all
(kept, dropped) pairs on tiny inputs, and by what the gap promises — moving
every distinct score by less than half the gap (equal scores moved together)
never changes the selected set or the argmin.
"""
import itertools

import numpy as np
import pytest

from oracle import argmin_gap, argmin_lower, boundary_gap, top_k_ascending
from oracle import fp8 as ofp8
from oracle import quest as oquest
from workloads import generator as gen
from workloads import get_config


def brute_boundary_gap(score, k, valid=None):
    """min over kept a and dropped b with different scores of (a - b) / |k-th best|,
    the kept set taken by Python's sort on (-score, index); inf when nothing or
    everything is kept, or no such pair exists."""
    idx = [i for i in range(len(score)) if valid is None or valid[i]]
    order = sorted(idx, key=lambda i: (-float(score[i]), i))
    if k <= 0 or k >= len(order):
        return np.inf
    kept, dropped = order[:k], order[k:]
    kth = float(score[order[k - 1]])
    gaps = [(float(score[a]) - float(score[b])) / abs(kth) for a in kept for b in dropped
            if float(score[a]) != float(score[b])]
    return min(gaps) if gaps else np.inf


def brute_argmin_gap(score, valid):
    cand = [i for i in range(len(score)) if valid[i]]
    if len(cand) < 2:
        return np.inf
    lo = min(float(score[i]) for i in cand)
    gaps = [(float(score[j]) - lo) / abs(lo) for j in cand if float(score[j]) != lo]
    return min(gaps) if gaps else np.inf


def tiny_scores(rng, n):
    """Nonzero scores from a small value set, so exact duplicates are common."""
    vals = rng.choice([-3.0, -1.5, -0.25, 0.5, 0.75, 1.0, 1.0009, 2.0, 2.5, 7.0], size=n)
    return vals * rng.choice([1.0, 1.0, 1e-3, 3.0])


def test_boundary_gap_equals_brute_force_over_pairs():
    rng = np.random.default_rng(11)
    for _ in range(3000):
        n = int(rng.integers(1, 9))
        s = tiny_scores(rng, n)
        valid = rng.random(n) < 0.8 if rng.random() < 0.3 else None
        for k in range(0, n + 2):
            assert boundary_gap(s, k, valid) == brute_boundary_gap(s, k, valid), (s, k, valid)


def test_boundary_gap_hand_cases():
    s = np.array([5.0, 3.0, 4.0, 1.0])
    assert boundary_gap(s, 2) == pytest.approx((4.0 - 3.0) / 4.0)     # kept {5, 4}, nearest dropped 3
    # equal scores straddle the boundary: distances to the nearest different score either side
    s = np.array([6.0, 2.0, 2.0, 2.0, 1.0])
    assert boundary_gap(s, 2) == pytest.approx(min(6.0 - 2.0, 2.0 - 1.0) / 2.0)
    assert boundary_gap(np.array([2.0, 2.0, 2.0]), 1) == np.inf        # all equal: no different score
    assert boundary_gap(s, 0) == np.inf and boundary_gap(s, 5) == np.inf


def test_argmin_gap_equals_brute_force():
    rng = np.random.default_rng(12)
    for _ in range(3000):
        n = int(rng.integers(1, 9))
        s = tiny_scores(rng, n)
        valid = rng.random(n) < 0.75
        assert argmin_gap(s, valid) == brute_argmin_gap(s, valid), (s, valid)
    assert argmin_gap(np.array([1.0, 3.0, 1.5]), np.array([True, True, True])) == pytest.approx(0.5)
    assert argmin_gap(np.array([1.0, 3.0]), np.array([True, False])) == np.inf


def perturb_groups(rng, s, bound):
    """Move every distinct value by the same random amount below `bound` in size."""
    out = s.astype(np.float64).copy()
    for v in np.unique(s):
        out[s == v] = v + rng.uniform(-bound, bound)
    return out


def test_boundary_gap_is_a_decision_margin():
    """Perturbing the distinct scores by less than gap * |k-th| / 2 keeps the selected set."""
    rng = np.random.default_rng(13)
    checked = 0
    for _ in range(2000):
        n = int(rng.integers(2, 9))
        s = tiny_scores(rng, n)
        k = int(rng.integers(1, n))
        gap = boundary_gap(s, k)
        if not np.isfinite(gap):
            continue
        kth = np.sort(s)[::-1][k - 1]
        sel = top_k_ascending(s, k)
        for _ in range(5):
            p = perturb_groups(rng, s, 0.499 * gap * abs(kth))
            np.testing.assert_array_equal(top_k_ascending(p, k), sel)
        checked += 1
    assert checked > 500


def test_argmin_gap_is_a_decision_margin():
    rng = np.random.default_rng(14)
    checked = 0
    for _ in range(2000):
        n = int(rng.integers(2, 9))
        s = tiny_scores(rng, n)
        valid = rng.random(n) < 0.8
        gap = argmin_gap(s, valid)
        if not np.isfinite(gap):
            continue
        lo = s[valid].min()
        pos = np.arange(n)
        ev = argmin_lower(s, pos, valid)
        for _ in range(5):
            p = perturb_groups(rng, s, 0.499 * gap * abs(lo))
            assert argmin_lower(p, pos, valid) == ev
        checked += 1
    assert checked > 500


def lowest_bit_exponent(x):
    """Per nonzero value, the exponent p of its lowest set bit (x = odd * 2^p)."""
    x = np.abs(np.asarray(x, np.float64))
    x = x[x > 0]
    m, e = np.frexp(x)                               # x = m * 2^e, m in [0.5, 1)
    mant = (m * 2.0 ** 53).astype(np.uint64)         # exact: m has at most 53 significant bits
    tz = np.zeros(mant.shape, np.int64)
    for b in range(53):
        tz += ((mant >> np.uint64(b)) & np.uint64(1) == 0) & (tz == b)
    return e - 53 + tz


def test_lowest_bit_exponent_hand_values():
    np.testing.assert_array_equal(lowest_bit_exponent([1.0, 0.75, 3 / 32, 448.0, 2.0 ** -9, 0.0]),
                                  [0, -2, -5, 6, -9])


@pytest.mark.parametrize("unit", [0, 21, 42, 63])
def test_fp8_stored_quest_bounds_are_exact_in_fp32(unit):
    """The Quest bound over FP8 rows is a sum of products q_d * v with v a stored value
    (code * 2^e, per-row e).  If every such product is a multiple of 2^p and the sum of
    the products' magnitudes stays below 2^(24 + p), every partial sum in any order is
    exact in fp32, so the GPU's bounds (any summation order, MFMA included) equal the
    oracle's exactly.  Checked on the 32K Quest workload's rows and queries as stored."""
    cfg = get_config(1)
    P = cfg.page_size
    K, _ = gen.unit_kv(cfg, 0, unit, cfg.context)
    kn = np.stack([gen.decode_kv_new(cfg, 0, s)[0][divmod(unit, cfg.n_kv_heads)] for s in range(cfg.decode_steps)])
    K = np.concatenate([K, kn])
    codes, sb = ofp8.quantize_rows(K)
    Ks = ofp8.dequantize_rows(codes, sb)
    L = K.shape[0]
    kmin, kmax = oquest.page_meta(Ks[None, None], [L], P)
    p_v = int(lowest_bit_exponent(np.concatenate([kmin.ravel(), kmax.ravel()])).min())
    worst, p_q = 0.0, 0
    for s in range(0, cfg.decode_steps, 7):
        q = gen.unit_query(cfg, 0, s, unit).astype(np.float64)             # [G][D]
        p_q = min(p_q, int(lowest_bit_exponent(q).min()))
        mag = np.maximum(np.abs(kmin[0, 0]), np.abs(kmax[0, 0]))          # [pages][D]
        worst = max(worst, float((np.abs(q) @ mag.T).max()))
        # and directly: float32 sums in two orders equal the exact float64 bound
        U64 = np.maximum(q[:, None, :] * kmin[0, 0][None], q[:, None, :] * kmax[0, 0][None])   # [G][pages][D]
        exact = U64.sum(axis=2)
        seq32 = np.zeros(exact.shape, np.float32)
        for d in range(U64.shape[2]):
            seq32 += U64[:, :, d].astype(np.float32)
        rev32 = np.zeros(exact.shape, np.float32)
        for d in reversed(range(U64.shape[2])):
            rev32 += U64[:, :, d].astype(np.float32)
        np.testing.assert_array_equal(seq32.astype(np.float64), exact)
        np.testing.assert_array_equal(rev32.astype(np.float64), exact)
    p = p_q + p_v
    assert worst < 2.0 ** (24 + p), f"sum of |q v| {worst} reaches 2^(24 + {p})"
