"""GPU parity of se_sparse_decode_attn over identity, page and token views,
with logits / lse outputs, split-K variations and degenerate views."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import TOL, banner, dev, host, tdtype, zeros
from workloads import generator as gen
from workloads import get_config

pytestmark = pytest.mark.gpu


def make(se, cfg, cap, lens, seed_layer=0):
    dt = tdtype(cfg)
    K, V = gen.cache_kv(cfg, seed_layer, cap, length=cap)
    q = gen.decode_query(cfg, seed_layer, 0)
    c = se.cache(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.d_k, cfg.d_v, cap, cfg.dtype, cfg.latent)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    return c, K, V, q, dev(K, dt), (None if V is None else dev(V, dt)), dev(q, dt), seq


def run_attn(se, c, qd, kd, vd, seq, view=None, vlen=None, view_cap=0, g=1, scale=0.1, logit_cap=0, splits=0):
    B, Hq = c.batch, c.n_q_heads
    out, lse = zeros((B, Hq, c.d_v)), zeros((B, Hq))
    logits = torch.full((B, Hq, logit_cap), 7.0, device="cuda") if logit_cap else None
    slots = view_cap * g if view is not None else c.capacity
    ws = se.workspace(se.SE_OP_ATTN, c, slots, splits)
    se.se_sparse_decode_attn(c, qd, kd, vd if vd is not None else kd, seq, view, vlen, view_cap, g, scale, out,
                             lse, logits, logit_cap, splits, ws)
    torch.cuda.synchronize()
    return host(out), host(lse), (host(logits) if logit_cap else None)


CFGS = {
    "f32_d64_g4": get_config(0),
    "bf16_d128_g8": get_config(0, dtype="bf16", batch=3, n_q_heads=16, n_kv_heads=2, d_k=128, d_v=128),
    "bf16_d64_g2": get_config(0, dtype="bf16", batch=2, n_q_heads=4, n_kv_heads=2, d_k=64, d_v=64),
    "bf16_mla": get_config(4, batch=2, context=700),
}


@pytest.mark.parametrize("name", list(CFGS))
@pytest.mark.parametrize("splits", [0, 1, 5])
def test_identity_view_with_logits(se, name, splits):
    cfg = CFGS[name]
    banner(f"identity view {name} splits={splits}")
    cap = 700 if cfg.latent else 333
    lens = [cap - 3 * i for i in range(cfg.batch)]
    c, K, V, q, kd, vd, qd, seq = make(se, cfg, cap, lens)
    scale = cfg.softmax_scale
    out, lse, lg = run_attn(se, c, qd, kd, vd, seq, scale=scale, logit_cap=cap + 5, splits=splits)
    ro, rl, rlg = oracle.decode_attention(q, K, V, lens, scale, latent_dv=cfg.d_v if cfg.latent else None,
                                          logit_cap=cap + 5)
    tol = TOL[cfg.dtype]
    np.testing.assert_allclose(out, ro, rtol=0, atol=tol)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=tol)
    for b, L in enumerate(lens):
        np.testing.assert_allclose(lg[b, :, :L], rlg[b, :, :L], rtol=0, atol=tol)
        assert np.all(lg[b, :, cap:] == 7.0)   # past the view's slots: not written


@pytest.mark.parametrize("name", ["f32_d64_g4", "bf16_d128_g8"])
def test_token_view_scattered(se, name):
    cfg = CFGS[name]
    banner(f"token view {name}")
    cap = 400
    rng = np.random.default_rng(3)
    lens = [cap - 17 * i for i in range(cfg.batch)]
    c, K, V, q, kd, vd, qd, seq = make(se, cfg, cap, lens)
    H, vc = cfg.n_kv_heads, 97
    view = np.full((cfg.batch, H, vc), -1, np.int32)
    vlen = np.zeros((cfg.batch, H), np.int32)
    for b in range(cfg.batch):
        for h in range(H):
            n = int(rng.integers(0, vc + 1))
            view[b, h, :n] = np.sort(rng.choice(lens[b], n, replace=False))
            vlen[b, h] = n
    vlen[0, 0] = 0                                       # an empty view
    out, lse, lg = run_attn(se, c, qd, kd, vd, seq, dev(view, torch.int32), dev(vlen, torch.int32), vc, 1,
                            cfg.softmax_scale, logit_cap=vc)
    ro, rl, rlg = oracle.decode_attention(q, K, V, lens, cfg.softmax_scale, view, vlen, 1, logit_cap=vc)
    tol = TOL[cfg.dtype]
    np.testing.assert_allclose(out, ro, rtol=0, atol=tol)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=tol)
    G = cfg.group
    assert np.all(out[0, :G] == 0) and np.all(np.isneginf(lse[0, :G]))
    for b in range(cfg.batch):
        for h in range(H):
            n = vlen[b, h]
            np.testing.assert_allclose(lg[b, h * G:(h + 1) * G, :n], rlg[b, h * G:(h + 1) * G, :n], atol=tol)


def test_page_view_pages_past_seq_len_and_empty_cache(se):
    cfg = CFGS["bf16_d128_g8"]
    banner("page view past seq_len")
    cap = 256
    lens = [200, 0, 17]
    c, K, V, q, kd, vd, qd, seq = make(se, cfg, cap, lens)
    H = cfg.n_kv_heads
    view = np.tile(np.array([0, 3, 12, 15], np.int32), (cfg.batch, H, 1))   # pages 12..15 lie past 200
    vlen = np.full((cfg.batch, H), 4, np.int32)
    out, lse, _ = run_attn(se, c, qd, kd, vd, seq, dev(view, torch.int32), dev(vlen, torch.int32), 4, 16,
                           cfg.softmax_scale)
    ro, rl, _ = oracle.decode_attention(q, K, V, lens, cfg.softmax_scale, view, vlen, 16)
    np.testing.assert_allclose(out, ro, rtol=0, atol=2e-3)
    np.testing.assert_allclose(lse[[0, 2]], rl[[0, 2]], rtol=0, atol=2e-3)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


def test_results_are_deterministic(se):
    cfg = CFGS["bf16_d128_g8"]
    c, K, V, q, kd, vd, qd, seq = make(se, cfg, 333, [333, 300, 1])
    a = run_attn(se, c, qd, kd, vd, seq, scale=0.1, logit_cap=333)
    b = run_attn(se, c, qd, kd, vd, seq, scale=0.1, logit_cap=333)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("name", ["bf16_d128_g8", "f32_d64_g4", "bf16_mla"])
def test_workspace_counters_return_to_zero(se, name):
    """The split tickets at the head of the workspace are zero after every call, so
    one workspace serves repeated calls with any split count, whichever merge path
    (in-kernel or combine kernel) the split count selects."""
    cfg = CFGS[name]
    banner(f"workspace reuse {name}")
    cap = 700 if cfg.latent else 333
    lens = [cap - 5 * i for i in range(cfg.batch)]
    c, K, V, q, kd, vd, qd, seq = make(se, cfg, cap, lens)
    ws = se.workspace(se.SE_OP_ATTN, c, cap, 100)
    ro, rl, _ = oracle.decode_attention(q, K, V, lens, 0.1, latent_dv=cfg.d_v if cfg.latent else None)
    first = None
    # small split counts merge inside the kernel, large ones in the combine kernel
    for splits in (7, 3, 1, 100, 40, 7):
        out, lse = zeros((cfg.batch, cfg.n_q_heads, cfg.d_v)), zeros((cfg.batch, cfg.n_q_heads))
        se.se_sparse_decode_attn(c, qd, kd, vd if vd is not None else kd, seq, None, None, 0, 1, 0.1, out, lse,
                                 None, 0, splits, ws)
        torch.cuda.synchronize()
        assert int(ws[:256].count_nonzero()) == 0
        np.testing.assert_allclose(host(out), ro, rtol=0, atol=TOL[cfg.dtype])
        np.testing.assert_allclose(host(lse), rl, rtol=0, atol=TOL[cfg.dtype])
        if splits == 7:
            if first is None:
                first = host(out)
            else:
                np.testing.assert_array_equal(host(out), first)
