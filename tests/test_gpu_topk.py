"""GPU parity of the Quest page top-k on designed score patterns: with
kmin = kmax = (s_p, 0, ..., 0) and q = (1, 0, ..., 0) every head's bound of
page p is exactly s_p, so ties, all-equal scores, signed zeros, negative
scores and every page-count regime of the selection kernel can be set up
directly.  The view is compared with the oracle's selection."""
import numpy as np
import pytest
import torch

from oracle import quest as oquest
from tests.gpu_util import banner, dev, host

pytestmark = pytest.mark.gpu

D, G, P = 64, 4, 16


def run_select(se, scores_per_unit, lens, k):
    """scores_per_unit: [units][n_cap_pages] bf16-exact page scores; lens: seq_len per batch row."""
    B, H = len(lens), scores_per_unit.shape[0] // len(lens)
    ncp = scores_per_unit.shape[1]
    cap = ncp * P
    meta = np.zeros((B, H, ncp, D), np.float32)
    meta[:, :, :, 0] = scores_per_unit.reshape(B, H, ncp)
    q = np.zeros((B, H * G, D), np.float32)
    q[:, :, 0] = 1.0
    c = se.cache(B, H * G, H, D, D, cap, "bf16")
    view = torch.zeros((B, H, k), dtype=torch.int32, device="cuda")
    vlen = torch.zeros((B, H), dtype=torch.int32, device="cuda")
    ws = se.workspace(se.SE_OP_QUEST, c, P, k)
    md = dev(meta, torch.bfloat16)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    se.se_quest_select(c, dev(q, torch.bfloat16), md, md, seq, P, k, view, vlen, None, ws)
    torch.cuda.synchronize()
    rv, rl, _ = oquest.quest_select(q, meta, meta, lens, P, k)
    return host(view), host(vlen), rv, rl


def bf16_exact(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("n_pages", [37, 2048, 2052, 4000, 4096, 8000, 8192, 9000])
def test_topk_random_scores_all_regimes(se, n_pages):
    """Register paths (n <= 2048, 4096, 8192 pages) and the LDS / global path above."""
    banner(f"topk random n={n_pages}")
    rng = np.random.default_rng(n_pages)
    B, H = 2, 2
    s = bf16_exact(rng.normal(0, 8, (B * H, n_pages)))
    lens = [n_pages * P, n_pages * P - 7]
    for k in (1, 128, n_pages - 1, n_pages + 3):
        gv, gl, rv, rl = run_select(se, s, lens, k)
        np.testing.assert_array_equal(gl, rl)
        np.testing.assert_array_equal(gv, rv, err_msg=f"k={k}")


def test_topk_ties_and_equal_scores(se):
    banner("topk ties")
    n = 2052
    rng = np.random.default_rng(3)
    B, H = 2, 2
    s = np.zeros((B * H, n), np.float32)
    s[0] = 1.5                                           # every score equal: the first k pages
    s[1] = rng.choice([-2.0, 0.5, 3.0], n)               # three values: the boundary falls inside a tie
    s[2] = rng.choice([0.0, -0.0, 1.0], n)               # signed zeros tie with each other
    s[3] = bf16_exact(-np.abs(rng.normal(0, 1, n)))      # all negative
    lens = [n * P, n * P]
    for k in (1, 5, 128, 700, 2051):
        gv, gl, rv, rl = run_select(se, s, lens, k)
        np.testing.assert_array_equal(gl, rl)
        np.testing.assert_array_equal(gv, rv, err_msg=f"k={k}")
    gv, _, _, _ = run_select(se, s, lens, 128)
    np.testing.assert_array_equal(gv[0, 0], np.arange(128))


def test_topk_short_and_empty_units(se):
    banner("topk short units")
    n = 300
    rng = np.random.default_rng(9)
    s = bf16_exact(rng.normal(0, 1, (3, n)))
    lens = [0, 1, 17 * P + 3]                            # no page, one page, a partial last page
    gv, gl, rv, rl = run_select(se, s, lens, 20)
    np.testing.assert_array_equal(gl, rl)
    np.testing.assert_array_equal(gv, rv)
    assert gl[0, 0] == 0 and np.all(gv[0, 0] == -1)
    assert gl[1, 0] == 1 and gv[1, 0, 0] == 0
