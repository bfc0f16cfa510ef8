"""Pins of the Chain Cache oracle (no GPU): prefix matching against
os.path.commonprefix, the position maps against a simulated multi-turn history
(every physical row must hold the row of its logical position), and the library's
host-side matcher against the oracle."""
import ctypes
import os

import numpy as np

from oracle import chain as och

import sparse_attention_kv_quest_amd as se


def test_match_prefix_hand_worked_and_commonprefix():
    stored = [[1, 2, 3], [1, 2], [1, 2, 3, 4, 5], [], [9, 9]]
    assert och.match_prefix(stored, [1, 2, 3, 4, 5, 6]) == (2, 5)
    assert och.match_prefix(stored, [1, 2, 3, 7]) == (0, 3)
    assert och.match_prefix(stored, [1, 2]) == (1, 2)
    assert och.match_prefix(stored, [5]) == (3, 0)                # only the empty prefix continues
    assert och.match_prefix([[4], [4]], [4, 4]) == (0, 1)          # equal lengths: the lower index
    assert och.match_prefix([[1, 2]], [1]) == (-1, 0)
    rng = np.random.default_rng(5)
    for _ in range(300):
        base = list(rng.integers(0, 4, 12))
        stored = [base[: int(rng.integers(0, 13))] if rng.random() < 0.7 else list(rng.integers(0, 4, 5))
                  for _ in range(6)]
        req = base[: int(rng.integers(0, 13))]
        s, n = och.match_prefix(stored, req)
        ok = [i for i, p in enumerate(stored) if os.path.commonprefix([p, req]) == p]
        if not ok:
            assert (s, n) == (-1, 0)
        else:
            best = max(len(stored[i]) for i in ok)
            assert n == best and s == min(i for i in ok if len(stored[i]) == best)


def test_position_maps_track_rows_through_turns():
    """Rows of a logical history (row t = [t, t]) through compaction, appends and a
    second compaction: the physical row i always holds the row of position map[i]."""
    rng = np.random.default_rng(6)
    logical = np.stack([np.arange(1000.0)] * 2, axis=1)
    L1 = 300
    phys = logical[:L1].copy()
    kept1 = np.sort(rng.choice(L1, 90, replace=False))
    m = och.compose_positions(None, np.concatenate([kept1, [-1] * 10]), 90)
    phys = phys[kept1]
    assert np.all(m[90:] == -1)
    np.testing.assert_array_equal(phys, logical[m[:90]])
    # turn 2: 50 new tokens at logical positions 300..349
    m = np.concatenate([m[:90], np.full(60, -1)])
    m = och.append_positions(m, 90, L1, 50)
    phys = np.concatenate([phys, logical[L1:L1 + 50]])
    np.testing.assert_array_equal(phys, logical[m[:140]])
    # turn-2 end: a second compaction keeps 40 of the 140 physical rows
    kept2 = np.sort(rng.choice(140, 40, replace=False))
    m2 = och.compose_positions(m, kept2, 40)
    np.testing.assert_array_equal(phys[kept2], logical[m2])
    # composing twice equals composing once with the composed selection
    np.testing.assert_array_equal(m2, och.compose_positions(None, np.concatenate([kept1, np.arange(L1, L1 + 50)])[kept2],
                                                            40))


def test_library_chain_match_matches_oracle():
    lib = se.load()
    rng = np.random.default_rng(7)
    for _ in range(300):
        base = list(int(x) for x in rng.integers(0, 3, 10))
        stored = [base[: int(rng.integers(0, 11))] if rng.random() < 0.7 else [int(x) for x in rng.integers(0, 3, 4)]
                  for _ in range(int(rng.integers(0, 7)))]
        req = base[: int(rng.integers(0, 11))]
        arrs = [(ctypes.c_int32 * max(1, len(p)))(*p) for p in stored]
        ptrs = (ctypes.c_void_p * max(1, len(stored)))(*[ctypes.cast(a, ctypes.c_void_p) for a in arrs])
        lens = (ctypes.c_int32 * max(1, len(stored)))(*[len(p) for p in stored])
        toks = (ctypes.c_int32 * max(1, len(req)))(*req)
        got_s, got_len = ctypes.c_int32(-5), ctypes.c_int32(-5)
        assert lib.se_chain_match(toks, len(req), ptrs, lens, len(stored), ctypes.byref(got_s), ctypes.byref(got_len)) == 0
        assert (got_s.value, got_len.value) == och.match_prefix(stored, req), (stored, req)


def test_library_chain_match_rejects_bad_arguments():
    lib = se.load()
    s, n = ctypes.c_int32(), ctypes.c_int32()
    lens = (ctypes.c_int32 * 1)(-1)
    ptrs = (ctypes.c_void_p * 1)(ctypes.c_void_p(0x10000))
    tok = (ctypes.c_int32 * 1)(1)
    assert lib.se_chain_match(None, 3, ptrs, lens, 1, ctypes.byref(s), ctypes.byref(n)) == -1    # tokens missing
    assert lib.se_chain_match(tok, 1, ptrs, lens, 1, None, ctypes.byref(n)) == -1                 # no output
    assert lib.se_chain_match(tok, 1, ptrs, lens, 1, ctypes.byref(s), ctypes.byref(n)) == -2      # negative length
    assert lib.se_chain_match(tok, -1, ptrs, lens, 0, ctypes.byref(s), ctypes.byref(n)) == -2
