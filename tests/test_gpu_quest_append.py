"""GPU parity of the fused Quest decode call (se_quest_append_select: append the
new K / V rows, rebuild the appended page's min / max, score and select pages)
against the separate calls it stands for (se_kv_append_meta, then
se_quest_select) bit for bit, and of its views against the CPU oracle."""
import numpy as np
import pytest
import torch

from oracle import quest as oquest
from tests.gpu_util import banner, dev, tdtype
from workloads import generator as gen
from workloads import get_config

pytestmark = pytest.mark.gpu

CFGS = {
    "bf16_d128_g8": get_config(0, dtype="bf16", batch=3, n_q_heads=16, n_kv_heads=2, d_k=128, d_v=128),
    "bf16_d128_g32": get_config(0, dtype="bf16", batch=2, n_q_heads=64, n_kv_heads=2, d_k=128, d_v=128),
    "bf16_d64_g4": get_config(0, dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2),
    "f32_d64": get_config(0, batch=2, n_q_heads=4, n_kv_heads=2),
    "mla_576": get_config(4, batch=2, context=200, page_size=64),
}


def bits(t):
    """Raw bits of a device tensor (signed zeros and NaN payloads compare exactly)."""
    t = t.detach().contiguous()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


class Layer:
    def __init__(self, se, cfg, cap, lens0, seed):
        dt = tdtype(cfg)
        B, H, D, P = cfg.batch, cfg.n_kv_heads, cfg.d_k, cfg.page_size
        self.c = se.cache(B, cfg.n_q_heads, H, D, cfg.d_v, cap, cfg.dtype, cfg.latent)
        K, V = gen.cache_kv(cfg, seed, cap, length=cap)
        self.k = dev(K, dt)
        self.v = None if cfg.latent else dev(V, dt)
        ncp = (cap + P - 1) // P
        self.kmin = torch.zeros((B, H, ncp, D), dtype=dt, device="cuda")
        self.kmax = torch.zeros_like(self.kmin)
        self.seq = torch.tensor(lens0, dtype=torch.int32, device="cuda")
        self.view = torch.full((B, H, TOP), -7, dtype=torch.int32, device="cuda")
        self.vlen = torch.full((B, H), -7, dtype=torch.int32, device="cuda")
        self.score = torch.zeros((B, H, ncp), device="cuda")
        se.se_page_meta_update(self.c, self.k, self.kmin, self.kmax, self.seq, P, 0)

    def state(self):
        out = [self.k, self.kmin, self.kmax, self.seq, self.view, self.vlen, self.score]
        return out + ([] if self.v is None else [self.v])


TOP = 3


def run_pair(se, cfg, cap, lens0, steps, seed, check_oracle=True):
    P = cfg.page_size
    dt = tdtype(cfg)
    fused, sep = Layer(se, cfg, cap, lens0, seed), Layer(se, cfg, cap, lens0, seed)
    ws_f = se.workspace(se.SE_OP_QUEST_APPEND, fused.c, P, 0)
    ws_s = se.workspace(se.SE_OP_QUEST, sep.c, P, TOP)
    for step in range(steps):
        q = gen.decode_query(cfg, seed, step)
        kn, vn = gen.decode_kv_new(cfg, seed, step)
        qd, knd = dev(q, dt), dev(kn, dt)
        vnd = None if cfg.latent else dev(vn, dt)
        se.se_quest_append_select(fused.c, qd, fused.k, fused.v, knd, vnd, fused.seq, fused.kmin, fused.kmax, P, TOP,
                                  fused.view, fused.vlen, fused.score, ws_f)
        se.se_kv_append_meta(sep.c, sep.k, sep.v, knd, vnd, None, sep.seq, sep.kmin, sep.kmax, P)
        se.se_quest_select(sep.c, qd, sep.kmin, sep.kmax, sep.seq, P, TOP, sep.view, sep.vlen, sep.score, ws_s)
        torch.cuda.synchronize()
        for a, b in zip(fused.state(), sep.state()):
            np.testing.assert_array_equal(bits(a), bits(b), err_msg=f"step {step}")
        if check_oracle:
            lens = fused.seq.cpu().numpy()
            Kh = fused.k.float().cpu().numpy()
            mn, mx = oquest.page_meta(Kh, lens, P)
            rv, rl, _ = oquest.quest_select(q, mn, mx, lens, P, TOP)
            np.testing.assert_array_equal(fused.vlen.cpu().numpy(), rl)
            np.testing.assert_array_equal(fused.view.cpu().numpy(), rv)
    return fused


@pytest.mark.parametrize("name", list(CFGS))
def test_append_select_matches_separate_calls(se, name):
    """Ragged lengths: a partial page filling up, a fresh page, a cache running full
    (no append once seq_len == capacity)."""
    cfg = CFGS[name]
    banner(f"quest append+select {name}")
    P = cfg.page_size
    cap = 4 * P + 3
    lens0 = [P - 1, 2 * P, cap - 2][: cfg.batch] if cfg.batch == 3 else [2 * P, cap - 2]
    f = run_pair(se, cfg, cap, lens0, 5, 11)
    assert list(f.seq.cpu().numpy()) == [min(l + 5, cap) for l in lens0]


@pytest.mark.parametrize("pages", [1500, 3000, 8000])
def test_append_select_long_caches(se, pages):
    """Page counts that take the in-launch selection's wider register paths (9, 16, 32
    keys per thread)."""
    cfg = get_config(0, dtype="bf16", batch=1, n_q_heads=4, n_kv_heads=1)
    banner(f"quest append+select pages={pages}")
    P = cfg.page_size
    cap = pages * P
    run_pair(se, cfg, cap, [cap - 20], 2, 12, check_oracle=(pages <= 3000))


def test_append_select_workspace_counters_return_to_zero(se):
    cfg = CFGS["bf16_d128_g8"]
    banner("quest append+select counters")
    P = cfg.page_size
    cap = 6 * P
    lay = Layer(se, cfg, cap, [P, 2 * P + 1, 3 * P - 1], 13)
    ws = se.workspace(se.SE_OP_QUEST_APPEND, lay.c, P, 0)
    dt = tdtype(cfg)
    for step in range(3):
        q = gen.decode_query(cfg, 13, step)
        kn, vn = gen.decode_kv_new(cfg, 13, step)
        se.se_quest_append_select(lay.c, dev(q, dt), lay.k, lay.v, dev(kn, dt), dev(vn, dt), lay.seq, lay.kmin,
                                  lay.kmax, P, TOP, lay.view, lay.vlen, None, ws)
        torch.cuda.synchronize()
        ctr = ws[: 4 * cfg.batch].view(torch.int32).cpu().numpy()   # one ticket counter per batch row
        assert np.all(ctr == 0), ctr
