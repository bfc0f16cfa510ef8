"""GPU checks of the Quest scoring of 576-column latent rows at grid shapes that
select each groups-per-wave variant of its kernel (1 to 4 groups of 16 pages per
wave, two blocks per CU): page bounds of sampled units against the CPU oracle's
bounds over the stored metadata, the views against the oracle's top-k of the
kernel's own scores (the decision taken in the kernel's precision), and the fused
decode call (append, fold into the last page, score, select) against the separate
calls, bit for bit, for every unit."""
import numpy as np
import pytest
import torch

from oracle import quest as oquest
from oracle.selection import top_k_ascending
from tests.gpu_util import banner

pytestmark = pytest.mark.gpu

D, DV, HQ, P, TOP = 576, 512, 32, 16, 8

# (units, capacity): 40, 200, 132 and 240 pages -> 1, 2, 3 and 4 groups per wave
CASES = {"g1": (512, 40 * P), "g2": (256, 200 * P), "g3": (512, 132 * P + 7), "g4": (512, 240 * P)}


def grid_groups(ncp, units):
    """Groups per wave the launcher picks (two 4-wave blocks per CU, pages split
    evenly, at most 4 groups per wave): only used to label the cases."""
    n = max(1, min(512 // units, -(-ncp // 16)))
    p = min(-(-(-(-ncp // n)) // 16) * 16, 256)
    return -(-p // 64)


def same_bits(x, y):
    """Bitwise equality on the device (signed zeros and infinities compare exactly)."""
    dt = torch.int16 if x.element_size() == 2 else torch.int32
    return torch.equal(x.contiguous().view(dt), y.contiguous().view(dt))


def make(se, units, cap, lens, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    c = se.cache(units, HQ, 1, D, DV, cap, "bf16", latent=True)
    k = torch.randn((units, 1, cap, D), generator=g, device="cuda").to(torch.bfloat16)
    ncp = -(-cap // P)
    kmin = torch.zeros((units, 1, ncp, D), dtype=torch.bfloat16, device="cuda")
    kmax = torch.zeros_like(kmin)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    se.se_page_meta_update(c, k, kmin, kmax, seq, P, 0)
    return c, k, kmin, kmax, seq


@pytest.mark.parametrize("name", list(CASES))
def test_wide_scoring_grid_variants(se, name):
    units, cap = CASES[name]
    ncp = -(-cap // P)
    banner(f"latent quest scoring {name}: units {units}, {ncp} pages, {grid_groups(ncp, units)} groups per wave")
    rng = np.random.default_rng(ncp)
    # mixed lengths: one short of full, ragged, one token, a fresh page on append, full
    lens = rng.integers(1, cap - 1, size=units)
    lens[:5] = [cap - 1, 1, P, 5 * P, cap]
    g = torch.Generator(device="cuda").manual_seed(7)
    q = torch.randn((units, HQ, D), generator=g, device="cuda").to(torch.bfloat16)
    kn = torch.randn((units, 1, D), generator=g, device="cuda").to(torch.bfloat16)
    sample = sorted({0, 1, 2, 3, 4, units // 2, units - 1, int(rng.integers(units))})

    # the selection alone
    c, k, kmin, kmax, seq = make(se, units, cap, lens, 11)
    view = torch.full((units, 1, TOP), -7, dtype=torch.int32, device="cuda")
    vlen = torch.full((units, 1), -7, dtype=torch.int32, device="cuda")
    score = torch.zeros((units, 1, ncp), device="cuda")
    se.se_quest_select(c, q, kmin, kmax, seq, P, TOP, view, vlen, score, se.workspace(se.SE_OP_QUEST, c, P, TOP))
    torch.cuda.synchronize()
    qh = q.float().cpu().numpy()[sample]
    mn = kmin.float().cpu().numpy()[sample]
    mx = kmax.float().cpu().numpy()[sample]
    _, S = oquest.quest_bounds(qh, mn, mx, lens[sample], P)
    got = score.cpu().numpy()[sample]
    for i, u in enumerate(sample):
        npv = -(-int(lens[u]) // P)
        np.testing.assert_allclose(got[i, 0, :npv], S[i, 0, :npv], rtol=1e-5, atol=1e-3, err_msg=f"unit {u}")
        ref = top_k_ascending(got[i, 0, :npv], TOP)
        np.testing.assert_array_equal(view.cpu().numpy()[u, 0, :ref.size], ref, err_msg=f"view unit {u}")
        assert vlen.cpu().numpy()[u, 0] == ref.size
    del k, kmin, kmax, score

    # the fused decode call against the separate calls, every unit
    st = {}
    for tag in ("fused", "separate"):
        st[tag] = make(se, units, cap, lens, 11) + (torch.zeros((units, 1, ncp), device="cuda"),
                                                    torch.full((units, 1, TOP), -7, dtype=torch.int32, device="cuda"),
                                                    torch.full((units, 1), -7, dtype=torch.int32, device="cuda"))
    c, k, kmin, kmax, seq, sc, vw, vl = st["fused"]
    se.se_quest_append_select(c, q, k, None, kn, None, seq, kmin, kmax, P, TOP, vw, vl, sc,
                              se.workspace(se.SE_OP_QUEST_APPEND, c, P, 0))
    c, k, kmin, kmax, seq, sc, vw, vl = st["separate"]
    se.se_kv_append_meta(c, k, None, kn, None, None, seq, kmin, kmax, P)
    se.se_quest_select(c, q, kmin, kmax, seq, P, TOP, vw, vl, sc, se.workspace(se.SE_OP_QUEST, c, P, TOP))
    torch.cuda.synchronize()
    a, b = st["fused"], st["separate"]
    assert np.array_equal(a[4].cpu().numpy(), np.minimum(lens + 1, cap))
    for x, y, what in zip(a[1:], b[1:], ("rows", "min", "max", "seq_len", "scores", "view", "view_len")):
        assert same_bits(x, y), f"{what} differ"
