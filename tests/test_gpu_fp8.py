"""GPU parity of the FP8 KV path (se_kv_quantize_fp8, se_kv_append_fp8,
se_sparse_decode_attn_fp8, and se_quest_select over the stored values) against
the CPU oracle, through the C ABI.  Codes and scale bytes are compared bit for
bit; attention over the stored values at the bf16 tolerance."""
import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import fp8 as ofp8
from oracle import quest as oquest
from tests.gpu_util import TOL, banner, dev, host, zeros
from workloads import generator as gen
from workloads import get_config

pytestmark = pytest.mark.gpu

CFGS = {
    "d128_g8": get_config(0, dtype="bf16", batch=3, n_q_heads=16, n_kv_heads=2, d_k=128, d_v=128, context=700),
    "d64_g4": get_config(0, dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2, context=500),
}


class Fp8Cache:
    def __init__(self, se, cfg, cap, seed, special=False):
        B, H, D, P = cfg.batch, cfg.n_kv_heads, cfg.d_k, cfg.page_size
        self.c = se.cache(B, cfg.n_q_heads, H, D, D, cap, "bf16")
        K, V = gen.cache_kv(cfg, seed, cap, length=cap)
        if special:   # rows the encoder must get right: zero, huge, tiny, signed zeros, 448 exactly
            K[0, 0, 1] = 0.0
            K[0, 0, 2] *= 1e6
            K[0, 0, 3] *= 2.0 ** -40
            K[0, 0, 4] = -0.0
            K[0, 0, 5, :] = 0.0
            K[0, 0, 5, 7] = 448.0
            V[0, 0, 6] *= -3e-3
        self.K = torch.from_numpy(K).to(torch.bfloat16).float().numpy()   # the bf16 source values
        self.V = torch.from_numpy(V).to(torch.bfloat16).float().numpy()
        self.k, self.v = dev(K, torch.bfloat16), dev(V, torch.bfloat16)
        self.kq = torch.full((B, H, cap, D), 0x55, dtype=torch.uint8, device="cuda")
        self.vq = torch.full_like(self.kq, 0x55)
        self.ks = torch.full((B, H, cap), 0x55, dtype=torch.uint8, device="cuda")
        self.vs = torch.full_like(self.ks, 0x55)
        ncp = (cap + P - 1) // P
        self.kmin = torch.zeros((B, H, ncp, D), dtype=torch.bfloat16, device="cuda")
        self.kmax = torch.zeros_like(self.kmin)


def stored(codes, sb):
    return ofp8.dequantize_rows(codes, sb)


@pytest.mark.parametrize("name", list(CFGS))
def test_quantize_matches_oracle(se, name):
    cfg = CFGS[name]
    banner(f"fp8 quantize {name}")
    B, H, P = cfg.batch, cfg.n_kv_heads, cfg.page_size
    cap = cfg.context + 9
    st = Fp8Cache(se, cfg, cap, 21, special=True)
    lens = [cfg.context - 3 * b for b in range(B)]
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    se.se_kv_quantize_fp8(st.c, st.k, st.v, seq, st.kq, st.vq, st.ks, st.vs, st.kmin, st.kmax, P)
    torch.cuda.synchronize()
    kq, vq, ks, vs = st.kq.cpu().numpy(), st.vq.cpu().numpy(), st.ks.cpu().numpy(), st.vs.cpu().numpy()
    Kh = np.zeros_like(st.K)
    for b in range(B):
        L = lens[b]
        rk, rks = ofp8.quantize_rows(st.K[b, :, :L])
        rv, rvs = ofp8.quantize_rows(st.V[b, :, :L])
        np.testing.assert_array_equal(kq[b, :, :L], rk, err_msg=f"K codes b={b}")
        np.testing.assert_array_equal(ks[b, :, :L], rks)
        np.testing.assert_array_equal(vq[b, :, :L], rv, err_msg=f"V codes b={b}")
        np.testing.assert_array_equal(vs[b, :, :L], rvs)
        assert np.all(kq[b, :, L:] == 0x55) and np.all(ks[b, :, L:] == 0x55)      # rows past seq_len untouched
        Kh[b, :, :L] = stored(rk, rks)
    mn, mx = oquest.page_meta(Kh, lens, P)
    for b in range(B):
        npg = (lens[b] + P - 1) // P
        np.testing.assert_array_equal(host(st.kmin)[b, :, :npg], mn[b, :, :npg])
        np.testing.assert_array_equal(host(st.kmax)[b, :, :npg], mx[b, :, :npg])


@pytest.mark.parametrize("name", list(CFGS))
def test_append_matches_oracle(se, name):
    cfg = CFGS[name]
    banner(f"fp8 append {name}")
    B, H, P = cfg.batch, cfg.n_kv_heads, cfg.page_size
    cap = 5 * P + 2
    st = Fp8Cache(se, cfg, cap, 22)
    lens0 = ([P - 2, 2 * P, cap - 2] * 2)[:B]
    seq = torch.tensor(lens0, dtype=torch.int32, device="cuda")
    se.se_kv_quantize_fp8(st.c, st.k, st.v, seq, st.kq, st.vq, st.ks, st.vs, st.kmin, st.kmax, P)
    for step in range(5):          # fills a page, opens a fresh one, runs into the full cache
        kn, vn = gen.decode_kv_new(cfg, 22, step)
        knb = torch.from_numpy(kn).to(torch.bfloat16).float().numpy()
        vnb = torch.from_numpy(vn).to(torch.bfloat16).float().numpy()
        before = seq.cpu().numpy().copy()
        se.se_kv_append_fp8(st.c, st.kq, st.vq, st.ks, st.vs, dev(kn, torch.bfloat16), dev(vn, torch.bfloat16), seq,
                            st.kmin, st.kmax, P)
        torch.cuda.synchronize()
        lens = seq.cpu().numpy()
        kq, vq, ks, vs = st.kq.cpu().numpy(), st.vq.cpu().numpy(), st.ks.cpu().numpy(), st.vs.cpu().numpy()
        for b in range(B):
            if before[b] < cap:
                assert lens[b] == before[b] + 1
                t = before[b]
                rk, rks = ofp8.quantize_rows(knb[b])
                rv, rvs = ofp8.quantize_rows(vnb[b])
                np.testing.assert_array_equal(kq[b, :, t], rk)
                np.testing.assert_array_equal(ks[b, :, t], rks)
                np.testing.assert_array_equal(vq[b, :, t], rv)
                np.testing.assert_array_equal(vs[b, :, t], rvs)
            else:
                assert lens[b] == cap
        Kh = stored(kq, ks)
        mn, mx = oquest.page_meta(Kh, lens, P)
        for b in range(B):
            npg = (lens[b] + P - 1) // P
            np.testing.assert_array_equal(host(st.kmin)[b, :, :npg], mn[b, :, :npg], err_msg=f"step {step}")
            np.testing.assert_array_equal(host(st.kmax)[b, :, :npg], mx[b, :, :npg])


def attention_case(se, cfg, st, lens, view, vlen, vcap, gran, splits, logit_cap=0):
    B, H, Hq, D = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k
    q = gen.decode_query(cfg, 23, 0)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out, lse = zeros((B, Hq, D)), zeros((B, Hq))
    logits = zeros((B, Hq, logit_cap)) if logit_cap else None
    slots = vcap * gran if view is not None else st.c.capacity
    ws = se.workspace(se.SE_OP_ATTN, st.c, slots, splits)
    se.se_sparse_decode_attn_fp8(st.c, dev(q, torch.bfloat16), st.kq, st.vq, st.ks, st.vs, seq,
                                 None if view is None else dev(view, torch.int32),
                                 None if vlen is None else dev(vlen, torch.int32), vcap, gran, cfg.softmax_scale, out,
                                 lse, logits, logit_cap, splits, ws)
    torch.cuda.synchronize()
    Kh = stored(st.kq.cpu().numpy(), st.ks.cpu().numpy())
    Vh = stored(st.vq.cpu().numpy(), st.vs.cpu().numpy())
    ref, ref_lse, ref_lg = oatt.decode_attention(q, Kh, Vh, lens, cfg.softmax_scale, view, vlen, gran,
                                                 logit_cap=logit_cap)
    tol = TOL["bf16"]
    np.testing.assert_allclose(host(out), ref, atol=tol, rtol=0)
    np.testing.assert_allclose(host(lse), ref_lse, atol=tol, rtol=0)
    if logit_cap:   # slots of the view's entries (later slots are not written)
        g, G = host(logits), cfg.group
        for b in range(B):
            for h in range(H):
                n = int(vlen[b, h]) * gran
                np.testing.assert_allclose(g[b, h * G:(h + 1) * G, :n], ref_lg[b, h * G:(h + 1) * G, :n], atol=tol,
                                           rtol=0)


@pytest.mark.parametrize("name", list(CFGS))
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_fp8_attention_views(se, name, splits):
    cfg = CFGS[name]
    banner(f"fp8 attention {name} splits={splits}")
    B, H, P = cfg.batch, cfg.n_kv_heads, cfg.page_size
    cap = cfg.context + 9
    st = Fp8Cache(se, cfg, cap, 24)
    lens = [cfg.context - 5 * b for b in range(B)]
    se.se_kv_quantize_fp8(st.c, st.k, st.v, torch.tensor(lens, dtype=torch.int32, device="cuda"), st.kq, st.vq,
                          st.ks, st.vs)
    rng = np.random.default_rng(splits)
    npg = (cfg.context + P - 1) // P
    # page view: ragged lengths, the partial last page included in some units
    k = 9
    view = np.full((B, H, k), -1, np.int32)
    vlen = np.zeros((B, H), np.int32)
    for b in range(B):
        for h in range(H):
            n = k - (b + h) % 3
            view[b, h, :n] = np.sort(rng.choice(npg, n, replace=False))
            vlen[b, h] = n
    attention_case(se, cfg, st, lens, view, vlen, k, P, splits, logit_cap=k * P)
    # token view
    kt = 77
    tview = np.sort(np.stack([rng.choice(cfg.context - 10, kt, replace=False) for _ in range(B * H)]), axis=1)
    attention_case(se, cfg, st, lens, tview.reshape(B, H, kt).astype(np.int32), np.full((B, H), kt, np.int32), kt, 1,
                   splits)
    # identity view (every valid slot)
    attention_case(se, cfg, st, lens, None, None, 0, 1, splits)


def test_fp8_quest_decode(se):
    """A Quest decode over an FP8 cache: the view from metadata of the stored values, the
    attention over the stored rows, against the oracle at every step."""
    cfg = get_config(0, dtype="bf16", batch=2, n_q_heads=16, n_kv_heads=2, d_k=128, d_v=128, context=1000,
                     top_pages=6)
    banner("fp8 quest decode")
    B, H, Hq, D, P, k = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.page_size, cfg.top_pages
    cap = cfg.context + 8
    st = Fp8Cache(se, cfg, cap, 25)
    seq = torch.full((B,), cfg.context, dtype=torch.int32, device="cuda")
    se.se_kv_quantize_fp8(st.c, st.k, st.v, seq, st.kq, st.vq, st.ks, st.vs, st.kmin, st.kmax, P)
    view = torch.zeros((B, H, k), dtype=torch.int32, device="cuda")
    vlen = torch.zeros((B, H), dtype=torch.int32, device="cuda")
    ws_q = se.workspace(se.SE_OP_QUEST, st.c, P, k)
    ws_a = se.workspace(se.SE_OP_ATTN, st.c, k * P, 0)
    for step in range(4):
        kn, vn = gen.decode_kv_new(cfg, 25, step)
        q = gen.decode_query(cfg, 25, step)
        se.se_kv_append_fp8(st.c, st.kq, st.vq, st.ks, st.vs, dev(kn, torch.bfloat16), dev(vn, torch.bfloat16), seq,
                            st.kmin, st.kmax, P)
        se.se_quest_select(st.c, dev(q, torch.bfloat16), st.kmin, st.kmax, seq, P, k, view, vlen, None, ws_q)
        out, lse = zeros((B, Hq, D)), zeros((B, Hq))
        se.se_sparse_decode_attn_fp8(st.c, dev(q, torch.bfloat16), st.kq, st.vq, st.ks, st.vs, seq, view, vlen, k, P,
                                     cfg.softmax_scale, out, lse, ws=ws_a)
        torch.cuda.synchronize()
        lens = seq.cpu().numpy()
        Kh = stored(st.kq.cpu().numpy(), st.ks.cpu().numpy())
        Vh = stored(st.vq.cpu().numpy(), st.vs.cpu().numpy())
        mn, mx = oquest.page_meta(Kh, lens, P)
        rv, rl, _ = oquest.quest_select(q, mn, mx, lens, P, k)
        np.testing.assert_array_equal(host(vlen), rl)
        np.testing.assert_array_equal(host(view), rv)
        ref, ref_lse, _ = oatt.decode_attention(q, Kh, Vh, lens, cfg.softmax_scale, rv, rl, P)
        np.testing.assert_allclose(host(out), ref, atol=TOL["bf16"], rtol=0)
        np.testing.assert_allclose(host(lse), ref_lse, atol=TOL["bf16"], rtol=0)


def test_fp8_quest_32k_all_units(se):
    """The 32K Quest workload over FP8 rows at full size, through the bench's calls
    (se_kv_quantize_fp8 once, then per step se_quest_decode_step_fp8): at the first, a
    middle and the last of 64 steps, every unit's codes, scale bytes and page metadata
    are compared by digest, its page scores and view exactly, and its attention at the
    bf16 tolerance, with the oracle's."""
    from tests import oracle_pool
    from tests.parity_jobs import digest, fp8_quest_unit
    cfg = get_config(1)
    B, H, Hq, D, P, k, G = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.page_size, cfg.top_pages, cfg.group
    checks = (0, 31, cfg.decode_steps - 1)
    jobs = [oracle_pool.pool().submit(fp8_quest_unit, ((1, {}), u, checks)) for u in range(cfg.units)]
    banner("fp8 quest 32K: building caches")
    cap = cfg.context + cfg.decode_steps
    c = se.cache(B, Hq, H, D, D, cap, "bf16")
    K, V = gen.cache_kv(cfg, 0, cap)
    kq = torch.full((B, H, cap, D), 0x55, dtype=torch.uint8, device="cuda")
    vq = torch.full_like(kq, 0x55)
    ks = torch.full((B, H, cap), 0x55, dtype=torch.uint8, device="cuda")
    vs = torch.full_like(ks, 0x55)
    ncp = (cap + P - 1) // P
    kmin = torch.zeros((B, H, ncp, D), dtype=torch.bfloat16, device="cuda")
    kmax = torch.zeros_like(kmin)
    seq = torch.full((B,), cfg.context, dtype=torch.int32, device="cuda")
    se.se_kv_quantize_fp8(c, dev(K, torch.bfloat16), dev(V, torch.bfloat16), seq, kq, vq, ks, vs, kmin, kmax, P)
    del K, V
    view = torch.zeros((B, H, k), dtype=torch.int32, device="cuda")
    vlen = torch.zeros((B, H), dtype=torch.int32, device="cuda")
    score = torch.zeros((B, H, ncp), device="cuda")
    out, lse = zeros((B, Hq, D)), zeros((B, Hq))
    ws_s = se.workspace(se.SE_OP_QUEST_STEP, c, P, k)
    got = {}
    for step in range(cfg.decode_steps):
        kn, vn = gen.decode_kv_new(cfg, 0, step)
        qd = dev(gen.decode_query(cfg, 0, step), torch.bfloat16)
        se.se_quest_decode_step_fp8(c, qd, kq, vq, ks, vs, dev(kn, torch.bfloat16), dev(vn, torch.bfloat16), seq,
                                    kmin, kmax, P, k, cfg.softmax_scale, out, lse, view, vlen, score, ws_s)
        if step in checks:
            torch.cuda.synchronize()
            L = cfg.context + step + 1
            assert np.all(host(seq) == L)
            npv = (L + P - 1) // P
            hk, hv, hks, hvs = kq.cpu().numpy(), vq.cpu().numpy(), ks.cpu().numpy(), vs.cpu().numpy()
            mn, mx = host(kmin), host(kmax)
            got[step] = dict(
                codes=[digest(np.stack([hk[u // H, u % H, :L], hv[u // H, u % H, :L]])) for u in range(cfg.units)],
                scales=[digest(np.stack([hks[u // H, u % H, :L], hvs[u // H, u % H, :L]])) for u in range(cfg.units)],
                meta=[digest(np.stack([mn[u // H, u % H, :npv], mx[u // H, u % H, :npv]])) for u in range(cfg.units)],
                score=host(score), view=host(view), vlen=host(vlen), out=host(out), lse=host(lse))
            banner(f"fp8 quest 32K: step {step} captured")
    for u, job in enumerate(jobs):
        ref = job.result()
        b, h = divmod(u, H)
        for step in checks:
            g, r = got[step], ref[step]
            L = cfg.context + step + 1
            npv = (L + P - 1) // P
            where = f"unit {u} step {step}"
            assert g["codes"][u] == r["codes"], f"{where}: FP8 codes differ"
            assert g["scales"][u] == r["scales"], f"{where}: scale bytes differ"
            assert g["meta"][u] == r["meta"], f"{where}: page metadata differs"
            np.testing.assert_array_equal(g["score"][b, h, :npv], r["score"].astype(np.float32), err_msg=where)
            assert g["vlen"][b, h] == r["vlen"]
            np.testing.assert_array_equal(g["view"][b, h], r["view"], err_msg=where)
            np.testing.assert_allclose(g["out"][b, h * G:(h + 1) * G], r["out"], atol=TOL["bf16"], rtol=0,
                                       err_msg=where)
            np.testing.assert_allclose(g["lse"][b, h * G:(h + 1) * G], r["lse"], atol=TOL["bf16"], rtol=0,
                                       err_msg=where)
