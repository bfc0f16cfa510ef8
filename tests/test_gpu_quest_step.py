"""se_quest_decode_step (a whole Quest decode step: append, page metadata, page
scores, page selection and attention) against se_quest_append_select followed
by se_sparse_decode_attn, bit for bit, over consecutive steps: cache rows, page
metadata, seq_len, page scores, views, outputs and lse.  Shapes that run the
in-launch selection (d_k 128 and 64, ragged and fresh pages, a full cache, page
counts across the selection's key-per-thread variants; MLA latent rows with 32
heads, including more pages than the view holds and a view longer than the
pages, and a group of 24 heads) and shapes that run the two calls' kernels
(fp32, latent rows with 16 heads, a non-power-of-two page size).  The
step call's results against the oracle are checked at full size in
test_gpu_quest.py."""
import numpy as np
import pytest
import torch

from tests.gpu_util import banner, dev, tdtype
from workloads import generator as gen
from workloads import get_config

pytestmark = pytest.mark.gpu

CASES = {
    "d128_g8_ragged": (get_config(0, dtype="bf16", batch=3, n_q_heads=16, n_kv_heads=2, d_k=128, d_v=128,
                                  context=300, top_pages=5), 7),
    "d64_g4": (get_config(0, dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2, context=500, top_pages=9), 5),
    "d128_g16_1500_pages": (get_config(0, dtype="bf16", batch=2, n_q_heads=32, n_kv_heads=2, d_k=128, d_v=128,
                                       context=24000, top_pages=100), 3),
    "d128_g8_3000_pages": (get_config(0, dtype="bf16", batch=1, n_q_heads=16, n_kv_heads=2, d_k=128, d_v=128,
                                      context=48000, top_pages=256), 2),
    "d128_full_cache": (get_config(0, dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2, d_k=128, d_v=128,
                                   context=318, top_pages=4), 4),
    "k_above_pages": (get_config(0, dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=1, d_k=128, d_v=128, context=40,
                                 top_pages=9), 3),
    "f32_fallback": (get_config(0, context=300, top_pages=6), 3),
    "mla_latent": (get_config(4, batch=2, context=1000, page_size=64, top_pages=5), 3),
    "mla_latent_2200_pages": (get_config(4, batch=1, context=140700, page_size=64, top_pages=64), 2),
    "mla_latent_ragged_view": (get_config(4, batch=3, context=900, page_size=64, top_pages=40), 3),
    "mla_g24_latent": (get_config(4, batch=2, n_q_heads=24, context=2000, page_size=64, top_pages=9), 3),
    "mla_g16_fallback": (get_config(4, batch=2, n_q_heads=16, context=1000, page_size=64, top_pages=5), 3),
    "mla_latent_page16": (get_config(4, batch=2, context=1000, page_size=16, top_pages=20), 3),
    "mla_latent_page32": (get_config(4, batch=3, context=1300, page_size=32, top_pages=9), 3),
    "d128_g8_page8": (get_config(0, dtype="bf16", batch=2, n_q_heads=16, n_kv_heads=2, d_k=128, d_v=128,
                                 context=250, page_size=8, top_pages=8), 9),
    "page_12_fallback": (get_config(0, dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2, d_k=128, d_v=128,
                                    context=300, page_size=12, top_pages=6), 3),
}


def same_bits(x, y):
    return torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8))


@pytest.mark.parametrize("name", list(CASES))
def test_step_matches_separate_calls(se, name):
    cfg, steps = CASES[name]
    banner(f"quest decode step vs separate calls: {name}")
    dt = tdtype(cfg)
    B, H, Hq, D, Dv, P, k = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.d_v, cfg.page_size, cfg.top_pages
    cap = cfg.context + (steps if name != "d128_full_cache" else 2)
    c = se.cache(B, Hq, H, D, Dv, cap, cfg.dtype, cfg.latent)
    K, V = gen.cache_kv(cfg, 60, cap)
    ncp = (cap + P - 1) // P
    side = {}
    for tag in ("step", "separate"):
        st = dict(k=dev(K, dt), v=None if cfg.latent else dev(V, dt),
                  seq=torch.full((B,), cfg.context, dtype=torch.int32, device="cuda"),
                  kmin=torch.zeros((B, H, ncp, D), dtype=dt, device="cuda"),
                  view=torch.full((B, H, k), -7, dtype=torch.int32, device="cuda"),
                  vlen=torch.full((B, H), -7, dtype=torch.int32, device="cuda"),
                  score=torch.zeros((B, H, ncp), device="cuda"),
                  out=torch.zeros((B, Hq, Dv), device="cuda"), lse=torch.zeros((B, Hq), device="cuda"))
        st["kmax"] = torch.zeros_like(st["kmin"])
        se.se_page_meta_update(c, st["k"], st["kmin"], st["kmax"], st["seq"], P, 0)
        side[tag] = st
    ws_step = se.workspace(se.SE_OP_QUEST_STEP, c, P, k)
    ws_sel = se.workspace(se.SE_OP_QUEST_APPEND, c, P, 0)
    ws_att = se.workspace(se.SE_OP_ATTN, c, k * P, 0)
    for step in range(steps):
        q = dev(gen.decode_query(cfg, 60, step), dt)
        kn, vn = gen.decode_kv_new(cfg, 60, step)
        knd = dev(kn, dt)
        vnd = None if cfg.latent else dev(vn, dt)
        a = side["step"]
        se.se_quest_decode_step(c, q, a["k"], a["v"], knd, vnd, a["seq"], a["kmin"], a["kmax"], P, k,
                                cfg.softmax_scale, a["out"], a["lse"], a["view"], a["vlen"], a["score"], ws_step)
        b = side["separate"]
        se.se_quest_append_select(c, q, b["k"], b["v"], knd, vnd, b["seq"], b["kmin"], b["kmax"], P, k, b["view"],
                                  b["vlen"], b["score"], ws_sel)
        se.se_sparse_decode_attn(c, q, b["k"], b["v"], b["seq"], b["view"], b["vlen"], k, P, cfg.softmax_scale,
                                 b["out"], b["lse"], ws=ws_att)
        torch.cuda.synchronize()
        for n in ("k", "v", "seq", "kmin", "kmax", "score", "view", "vlen", "out", "lse"):
            if a[n] is not None:
                assert same_bits(a[n], b[n]), f"step {step}: {n} differs"
    lens = side["step"]["seq"].cpu().numpy()
    assert np.all(lens == min(cfg.context + steps, cap))


def test_step_without_view_outputs(se):
    """The view and scores are optional outputs: the same out / lse without them."""
    cfg, steps = CASES["d128_g8_ragged"]
    banner("quest decode step without view outputs")
    dt = tdtype(cfg)
    B, H, Hq, D, P, k = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.page_size, cfg.top_pages
    cap = cfg.context + 1
    c = se.cache(B, Hq, H, D, D, cap, "bf16")
    K, V = gen.cache_kv(cfg, 61, cap)
    res = []
    for with_view in (True, False):
        kk, vv = dev(K, dt), dev(V, dt)
        seq = torch.full((B,), cfg.context, dtype=torch.int32, device="cuda")
        ncp = (cap + P - 1) // P
        kmin = torch.zeros((B, H, ncp, D), dtype=dt, device="cuda")
        kmax = torch.zeros_like(kmin)
        se.se_page_meta_update(c, kk, kmin, kmax, seq, P, 0)
        out, lse = torch.zeros((B, Hq, D), device="cuda"), torch.zeros((B, Hq), device="cuda")
        view = torch.zeros((B, H, k), dtype=torch.int32, device="cuda") if with_view else None
        vlen = torch.zeros((B, H), dtype=torch.int32, device="cuda") if with_view else None
        kn, vn = gen.decode_kv_new(cfg, 61, 0)
        se.se_quest_decode_step(c, dev(gen.decode_query(cfg, 61, 0), dt), kk, vv, dev(kn, dt), dev(vn, dt), seq, kmin,
                                kmax, P, k, cfg.softmax_scale, out, lse, view, vlen, None,
                                se.workspace(se.SE_OP_QUEST_STEP, c, P, k))
        torch.cuda.synchronize()
        res.append((out, lse, seq))
    for x, y in zip(res[0], res[1]):
        assert same_bits(x, y)
