"""GPU parity of the MLA latent path: 64-token latent pages, Quest top-k over
576-wide keys shared by 32 heads, attention with V = the first 512 latent columns."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quest as oquest
from tests.gpu_util import TOL, banner, dev, host, zeros
from workloads import generator as gen
from workloads import get_config

pytestmark = pytest.mark.gpu


def run_mla(se, cfg, units, steps=1, mode="separate"):
    """mode "separate": se_kv_append, se_page_meta_update, se_quest_select, then the
    attention; "fused": se_quest_append_select, then the attention; "step": the whole
    decode step in se_quest_decode_step (the bench's call)."""
    B, Hq, D, Dv, P, k = cfg.batch, cfg.n_q_heads, cfg.d_k, cfg.d_v, cfg.page_size, cfg.top_pages
    cap = cfg.context + steps
    C, _ = gen.cache_kv(cfg, 0, cap)                       # [B][1][cap][576]
    c = se.cache(B, Hq, 1, D, Dv, cap, "bf16", latent=True)
    cd = dev(C, torch.bfloat16)
    seq = torch.full((B,), cfg.context, dtype=torch.int32, device="cuda")
    ncp = (cap + P - 1) // P
    kmin = torch.zeros((B, 1, ncp, D), dtype=torch.bfloat16, device="cuda")
    kmax = torch.zeros_like(kmin)
    view = torch.zeros((B, 1, k), dtype=torch.int32, device="cuda")
    vlen = torch.zeros((B, 1), dtype=torch.int32, device="cuda")
    score = torch.zeros((B, 1, ncp), device="cuda")
    out, lse = zeros((B, Hq, Dv)), zeros((B, Hq))
    ws_q = se.workspace(se.SE_OP_QUEST, c, P, k)
    ws_qa = se.workspace(se.SE_OP_QUEST_APPEND, c, P, 0)
    ws_a = se.workspace(se.SE_OP_ATTN, c, k * P, 0)
    ws_s = se.workspace(se.SE_OP_QUEST_STEP, c, P, k)
    se.se_page_meta_update(c, cd, kmin, kmax, seq, P, 0)
    for s in range(steps):
        q = gen.decode_query(cfg, 0, s)                     # [B][32][576]
        kn, _ = gen.decode_kv_new(cfg, 0, s)
        C[:, :, cfg.context + s] = kn
        qd = dev(q, torch.bfloat16)
        if mode == "step":
            se.se_quest_decode_step(c, qd, cd, None, dev(kn, torch.bfloat16), None, seq, kmin, kmax, P, k,
                                    cfg.softmax_scale, out, lse, view, vlen, score, ws_s)
            continue
        if mode == "fused":
            se.se_quest_append_select(c, qd, cd, None, dev(kn, torch.bfloat16), None, seq, kmin, kmax, P, k, view,
                                      vlen, score, ws_qa)
        else:
            se.se_kv_append(c, cd, None, dev(kn, torch.bfloat16), None, None, seq)
            se.se_page_meta_update(c, cd, kmin, kmax, seq, P, -1)
            se.se_quest_select(c, qd, kmin, kmax, seq, P, k, view, vlen, score, ws_q)
        se.se_sparse_decode_attn(c, qd, cd, None, seq, view, vlen, k, P, cfg.softmax_scale, out, lse, ws=ws_a)
    torch.cuda.synchronize()
    L = cfg.context + steps
    g = {n: host(t) for n, t in (("kmin", kmin), ("kmax", kmax), ("view", view), ("vlen", vlen), ("score", score),
                                 ("out", out), ("lse", lse))}
    for b in units:
        Cb = C[b:b + 1]
        mn, mx = oquest.page_meta(Cb, [L], P)
        npv = oquest.n_pages(L, P)
        np.testing.assert_array_equal(g["kmin"][b, 0, :npv], mn[0, 0, :npv])
        np.testing.assert_array_equal(g["kmax"][b, 0, :npv], mx[0, 0, :npv])
        rv, rl, S = oquest.quest_select(q[b:b + 1], mn, mx, [L], P, k)
        np.testing.assert_array_equal(g["score"][b, 0, :npv], S[0, 0, :npv].astype(np.float32))
        np.testing.assert_array_equal(g["view"][b, 0], rv[0, 0])
        ro, rlse, _ = oracle.decode_attention(q[b:b + 1], Cb, None, [L], cfg.softmax_scale, rv, rl, P, latent_dv=Dv)
        np.testing.assert_allclose(g["out"][b], ro[0], rtol=0, atol=TOL["bf16"])
        np.testing.assert_allclose(g["lse"][b], rlse[0], rtol=0, atol=TOL["bf16"])


@pytest.mark.parametrize("mode", ["separate", "fused", "step"])
def test_mla_small_all_units(se, mode):
    cfg = get_config(4, batch=3, context=3000, top_pages=8)
    banner(f"mla small {mode}")
    run_mla(se, cfg, range(cfg.batch), steps=3, mode=mode)


@pytest.mark.parametrize("mode", ["separate", "step"])
@pytest.mark.parametrize("page", [16, 32])
def test_mla_small_page_sizes(se, page, mode):
    """Latent rows over 16- and 32-token pages, every batch row against the oracle after
    steps that cross a page boundary."""
    cfg = get_config(4, batch=2, context=1000 + page - 3, page_size=page, top_pages=12)
    banner(f"mla small page={page} {mode}")
    run_mla(se, cfg, range(cfg.batch), steps=5, mode=mode)


def test_mla_128k_all_rows(se):
    """The 128K MLA workload at full size through the bench's call (se_quest_decode_step:
    the scoring launch with the append, then the attention launch that selects the
    pages itself): 64 decode steps, every batch row compared with the oracle at steps
    0, 1, 31 and 63 (metadata by digest, page scores and views exactly, output and lse
    at the bf16 tolerance)."""
    from concurrent.futures import ThreadPoolExecutor
    from tests import oracle_pool
    from tests.parity_jobs import digest, mla_row
    cfg = get_config(4)
    B, Hq, D, Dv, P, k = cfg.batch, cfg.n_q_heads, cfg.d_k, cfg.d_v, cfg.page_size, cfg.top_pages
    checks = (0, 1, 31, cfg.decode_steps - 1)
    jobs = [oracle_pool.pool().submit(mla_row, ((4, {}), b, checks)) for b in range(B)]
    banner("mla 128K: 32 x 131072 latent rows, top-64 pages")
    cap = cfg.context + cfg.decode_steps
    c = se.cache(B, Hq, 1, D, Dv, cap, "bf16", latent=True)
    cd = torch.zeros((B, 1, cap, D), dtype=torch.bfloat16, device="cuda")
    with ThreadPoolExecutor(oracle_pool.n_workers()) as ex:
        for b, (rows, _) in enumerate(ex.map(lambda b: gen.unit_kv(cfg, 0, b, cfg.context), range(B))):
            cd[b, 0, :cfg.context] = torch.from_numpy(rows).to("cuda", torch.bfloat16)
    seq = torch.full((B,), cfg.context, dtype=torch.int32, device="cuda")
    ncp = (cap + P - 1) // P
    kmin = torch.zeros((B, 1, ncp, D), dtype=torch.bfloat16, device="cuda")
    kmax = torch.zeros_like(kmin)
    view = torch.zeros((B, 1, k), dtype=torch.int32, device="cuda")
    vlen = torch.zeros((B, 1), dtype=torch.int32, device="cuda")
    score = torch.zeros((B, 1, ncp), device="cuda")
    out, lse = zeros((B, Hq, Dv)), zeros((B, Hq))
    ws_s = se.workspace(se.SE_OP_QUEST_STEP, c, P, k)
    se.se_page_meta_update(c, cd, kmin, kmax, seq, P, 0)
    got = {}
    for s in range(cfg.decode_steps):
        qd = dev(gen.decode_query(cfg, 0, s), torch.bfloat16)
        kn, _ = gen.decode_kv_new(cfg, 0, s)
        se.se_quest_decode_step(c, qd, cd, None, dev(kn, torch.bfloat16), None, seq, kmin, kmax, P, k,
                                cfg.softmax_scale, out, lse, view, vlen, score, ws_s)
        if s in checks:
            torch.cuda.synchronize()
            L = cfg.context + s + 1
            assert np.all(host(seq) == L)
            npv = (L + P - 1) // P
            mn, mx = host(kmin), host(kmax)
            got[s] = dict(meta=[digest(np.stack([mn[b, 0, :npv], mx[b, 0, :npv]])) for b in range(B)],
                          score=host(score), view=host(view), vlen=host(vlen), out=host(out), lse=host(lse))
            banner(f"mla 128K: step {s} captured")
    for b, job in enumerate(jobs):
        r = job.result()
        for s in checks:
            g = got[s]
            L = cfg.context + s + 1
            npv = (L + P - 1) // P
            where = f"row {b} step {s}"
            assert g["meta"][b] == r[s]["meta"], f"{where}: page metadata differs"
            np.testing.assert_array_equal(g["score"][b, 0, :npv], r[s]["score"].astype(np.float32), err_msg=where)
            assert g["vlen"][b, 0] == r[s]["vlen"]
            np.testing.assert_array_equal(g["view"][b, 0], r[s]["view"], err_msg=where)
            np.testing.assert_allclose(g["out"][b], r[s]["out"], rtol=0, atol=TOL["bf16"], err_msg=where)
            np.testing.assert_allclose(g["lse"][b], r[s]["lse"], rtol=0, atol=TOL["bf16"], err_msg=where)
