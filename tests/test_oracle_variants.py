"""Pins of the StreamingLLM and PyramidKV oracle (no GPU): special cases that
reduce to plain windows, dense attention or library routines, invariants of
the kept sets and budget schedules, and hand-worked schedules.  Also checks the
library's host-side budget schedule against the oracle."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import variants as ov

import sparse_attention_kv_quest_amd as se


@pytest.mark.parametrize("L,sink,recent", [(0, 4, 8), (1, 4, 8), (12, 4, 8), (13, 4, 8), (100, 4, 8),
                                           (100, 0, 8), (100, 4, 0), (7, 10, 3), (3000, 4, 2044)])
def test_streaming_kept_invariants(L, sink, recent):
    kept = ov.streaming_kept(L, sink, recent)
    assert len(kept) == min(L, sink + recent)
    assert np.all(np.diff(kept) > 0) and (len(kept) == 0 or (kept[0] >= 0 and kept[-1] < L))
    assert set(range(min(sink, L))) <= set(kept.tolist())                 # the sink
    assert set(range(max(0, L - recent), L)) <= set(kept.tolist())        # the recent window


def test_streaming_kept_special_cases():
    # nothing dropped while the history fits
    np.testing.assert_array_equal(ov.streaming_kept(50, 10, 40), np.arange(50))
    # no sink: a plain sliding window (numpy slicing)
    np.testing.assert_array_equal(ov.streaming_kept(50, 0, 7), np.arange(50)[-7:])
    # no window: the first tokens only
    np.testing.assert_array_equal(ov.streaming_kept(50, 5, 0), np.arange(5))
    # hand-worked: 20 tokens, sink 2, recent 3
    assert ov.streaming_kept(20, 2, 3).tolist() == [0, 1, 17, 18, 19]


def test_streaming_view_shapes_and_padding():
    view, vlen = ov.streaming_view([20, 3, 0], 2, 2, 3, 6)
    assert view.shape == (3, 2, 6) and vlen.tolist() == [[5, 5], [3, 3], [0, 0]]
    assert view[0, 1].tolist() == [0, 1, 17, 18, 19, -1]
    assert view[1, 0].tolist() == [0, 1, 2, -1, -1, -1]
    assert np.all(view[2] == -1)


def test_streaming_attention_full_budget_equals_dense():
    """sink + recent >= length: attention over the StreamingLLM view equals dense attention
    (torch's scaled-dot-product attention in float64)."""
    rng = np.random.default_rng(4)
    B, H, G, D, L = 2, 2, 3, 16, 40
    q = rng.normal(size=(B, H * G, D))
    K = rng.normal(size=(B, H, L, D))
    V = rng.normal(size=(B, H, L, D))
    view, vlen = ov.streaming_view([L, L - 5], H, 8, 40, 48)
    out, _, _ = oatt.decode_attention(q, K, V, [L, L - 5], 0.25, view, vlen, 1)
    for b, n in enumerate([L, L - 5]):
        qt = torch.from_numpy(q[b]).reshape(H, G, 1, D)
        kt = torch.from_numpy(K[b, :, :n]).reshape(H, 1, n, D).expand(H, G, n, D)
        vt = torch.from_numpy(V[b, :, :n]).reshape(H, 1, n, D).expand(H, G, n, D)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.25).reshape(H * G, D)
        np.testing.assert_allclose(out[b], ref.numpy(), atol=1e-12)


@pytest.mark.parametrize("n,avg,bmin,expect", [(4, 10, 4, [16, 12, 8, 4]), (4, 10, 5, [15, 12, 8, 5]),
                                               (3, 10, 5, [15, 10, 5]), (1, 7, 2, [7]), (5, 9, 9, [9] * 5),
                                               (2, 10, 0, [20, 0])])
def test_pyramid_budgets_hand_worked(n, avg, bmin, expect):
    assert ov.pyramid_budgets(n, avg, bmin) == expect


@pytest.mark.parametrize("n,avg,bmin", [(32, 2048, 512), (48, 8192, 1024), (7, 100, 33), (13, 1000, 999),
                                        (3, 5, 0), (64, 333, 111)])
def test_pyramid_budgets_invariants(n, avg, bmin):
    b = ov.pyramid_budgets(n, avg, bmin)
    assert len(b) == n and sum(b) == n * avg                            # the mean is the average budget
    assert all(x >= y for x, y in zip(b, b[1:]))                         # shrinks with depth
    real = np.linspace(2 * avg - bmin, bmin, n)                          # the arithmetic sequence
    assert np.all(np.abs(np.array(b) - real) < 1.0 + 1e-9)


@pytest.mark.parametrize("seed", range(6))
def test_library_pyramid_budgets_match_oracle(seed):
    """The library's host-side schedule (C ABI, no GPU work) equals the oracle's."""
    lib = se.load()
    rng = np.random.default_rng(seed)
    for _ in range(200):
        n = int(rng.integers(1, 80))
        avg = int(rng.integers(0, 20000))
        bmin = int(rng.integers(0, avg + 1))
        out = (ctypes.c_int32 * n)()
        assert lib.se_pyramid_budgets(n, avg, bmin, out) == 0
        assert list(out) == ov.pyramid_budgets(n, avg, bmin), (n, avg, bmin)


def test_library_pyramid_budgets_rejects_bad_arguments():
    lib = se.load()
    out = (ctypes.c_int32 * 4)()
    assert lib.se_pyramid_budgets(0, 10, 5, out) == -2          # no layer
    assert lib.se_pyramid_budgets(4, 10, 11, out) == -5         # min above the average
    assert lib.se_pyramid_budgets(4, 10, -1, out) == -5
    assert lib.se_pyramid_budgets(4, 10, 5, None) == -1
