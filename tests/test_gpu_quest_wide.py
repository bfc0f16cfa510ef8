"""GPU checks of the Quest scoring of 576-column latent rows at grid shapes that
select each groups-per-wave variant of its kernel (1 to 4 groups of 16 pages per
wave, two blocks per CU): on grid-valued rows and queries (every bound exact in
fp32), page bounds and views of sampled units against the CPU oracle's, bit for
bit, and the fused decode call (append, fold into the last page, score, select)
against the separate calls, bit for bit, for every unit."""
import numpy as np
import pytest
import torch

from oracle import quest as oquest
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


def grid_randn(shape, g):
    """round(32 x) / 32 clipped to +-255/32, x ~ N(0, 1), drawn on the device: exact in
    bf16, and every sum of products of two such values below 2^14 is exact in fp32."""
    x = torch.randn(shape, generator=g, device="cuda")
    return x.mul_(32.0).round_().clamp_(-255.0, 255.0).div_(32.0).add_(0.0).to(torch.bfloat16)


def make(se, units, cap, lens, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    c = se.cache(units, HQ, 1, D, DV, cap, "bf16", latent=True)
    k = grid_randn((units, 1, cap, D), g)
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
    q = grid_randn((units, HQ, D), g)
    kn = grid_randn((units, 1, D), g)
    sample = sorted({0, 1, 2, 3, 4, units // 2, units - 1, int(rng.integers(units))})

    # the selection alone
    c, k, kmin, kmax, seq = make(se, units, cap, lens, 11)
    view = torch.full((units, 1, TOP), -7, dtype=torch.int32, device="cuda")
    vlen = torch.full((units, 1), -7, dtype=torch.int32, device="cuda")
    score = torch.zeros((units, 1, ncp), device="cuda")
    se.se_quest_select(c, q, kmin, kmax, seq, P, TOP, view, vlen, score, se.workspace(se.SE_OP_QUEST, c, P, TOP))
    torch.cuda.synchronize()
    qh = q.float().cpu().numpy()[sample]
    kh = k.float().cpu().numpy()[sample]
    mn, mx = oquest.page_meta(kh, lens[sample], P)
    np.testing.assert_array_equal(kmin.float().cpu().numpy()[sample][:, :, :mn.shape[2]][~np.isnan(mn)],
                                  mn[~np.isnan(mn)])
    assert float((np.abs(qh).sum(-1).max()) * np.abs(kh).max()) < 2 ** 14     # the exactness precondition
    rview, rlen, S = oquest.quest_select(qh, mn, mx, lens[sample], P, TOP)
    got = score.cpu().numpy()[sample]
    for i, u in enumerate(sample):
        npv = -(-int(lens[u]) // P)
        np.testing.assert_array_equal(got[i, 0, :npv], S[i, 0, :npv].astype(np.float32), err_msg=f"unit {u}")
        np.testing.assert_array_equal(view.cpu().numpy()[u, 0], rview[i, 0], err_msg=f"view unit {u}")
        assert vlen.cpu().numpy()[u, 0] == rlen[i, 0]
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
