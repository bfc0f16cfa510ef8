"""GPU parity of the Quest decode path (append -> page metadata -> page top-k ->
sparse decode attention) against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quest as oquest
from tests.gpu_util import TOL, banner, dev, host, tdtype, unit_slices, zeros
from workloads import generator as gen
from workloads import get_config

pytestmark = pytest.mark.gpu


class QuestState:
    """Device buffers of one layer of a Quest cache."""

    def __init__(self, se, cfg, cap):
        self.cfg, self.cap = cfg, cap
        dt = tdtype(cfg)
        B, H, Hq, D, P = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.page_size
        self.c = se.cache(B, Hq, H, D, cfg.d_v, cap, cfg.dtype)
        self.K, self.V = gen.cache_kv(cfg, 0, cap)
        self.k, self.v = dev(self.K, dt), dev(self.V, dt)
        self.seq = torch.full((B,), cfg.context, dtype=torch.int32, device="cuda")
        self.ncp = (cap + P - 1) // P
        self.kmin = torch.zeros((B, H, self.ncp, D), dtype=dt, device="cuda")
        self.kmax = torch.zeros_like(self.kmin)
        self.view = torch.zeros((B, H, cfg.top_pages), dtype=torch.int32, device="cuda")
        self.vlen = torch.zeros((B, H), dtype=torch.int32, device="cuda")
        self.score = torch.zeros((B, H, self.ncp), device="cuda")
        self.out = zeros((B, Hq, cfg.d_v))
        self.lse = zeros((B, Hq))
        self.ws_q = se.workspace(se.SE_OP_QUEST, self.c, P, cfg.top_pages)
        self.ws_qa = se.workspace(se.SE_OP_QUEST_APPEND, self.c, P, 0)
        self.ws_a = se.workspace(se.SE_OP_ATTN, self.c, cfg.top_pages * P, 0)
        self.ws_step = se.workspace(se.SE_OP_QUEST_STEP, self.c, P, cfg.top_pages)
        se.se_page_meta_update(self.c, self.k, self.kmin, self.kmax, self.seq, P, 0)

    def step(self, se, step, splits=0, fused=False, whole=False):
        """fused: append, metadata, scores and view through se_quest_append_select instead
        of se_kv_append, se_page_meta_update, se_quest_select; whole: the whole step
        through se_quest_decode_step (the bench's call)."""
        cfg, dt, P = self.cfg, tdtype(self.cfg), self.cfg.page_size
        q = gen.decode_query(cfg, 0, step)
        kn, vn = gen.decode_kv_new(cfg, 0, step)
        L = cfg.context + step
        self.K[:, :, L], self.V[:, :, L] = kn, vn
        qd = dev(q, dt)
        if whole:
            se.se_quest_decode_step(self.c, qd, self.k, self.v, dev(kn, dt), dev(vn, dt), self.seq, self.kmin,
                                    self.kmax, P, cfg.top_pages, cfg.softmax_scale, self.out, self.lse, self.view,
                                    self.vlen, self.score, self.ws_step)
            return q, L + 1
        if fused:
            se.se_quest_append_select(self.c, qd, self.k, self.v, dev(kn, dt), dev(vn, dt), self.seq, self.kmin,
                                      self.kmax, P, cfg.top_pages, self.view, self.vlen, self.score, self.ws_qa)
        else:
            se.se_kv_append(self.c, self.k, self.v, dev(kn, dt), dev(vn, dt), None, self.seq)
            se.se_page_meta_update(self.c, self.k, self.kmin, self.kmax, self.seq, P, -1)
            se.se_quest_select(self.c, qd, self.kmin, self.kmax, self.seq, P, cfg.top_pages, self.view, self.vlen,
                               self.score, self.ws_q)
        se.se_sparse_decode_attn(self.c, qd, self.k, self.v, self.seq, self.view, self.vlen, cfg.top_pages, P,
                                 cfg.softmax_scale, self.out, self.lse, num_splits=splits,
                                 ws=se.workspace(se.SE_OP_ATTN, self.c, cfg.top_pages * P, splits))
        return q, L + 1


def check_unit(cfg, st, q, L, unit, got):
    """Oracle for one unit at the current state; compares metadata, scores, view and attention."""
    b, h, hs = unit_slices(cfg, unit)
    P = cfg.page_size
    Ku = st.K[b:b + 1, h:h + 1]
    Vu = st.V[b:b + 1, h:h + 1]
    qu = q[b:b + 1, hs]
    kmin, kmax = oquest.page_meta(Ku, [L], P)
    npv = oquest.n_pages(L, P)
    np.testing.assert_array_equal(got["kmin"][b, h, :npv], kmin[0, 0, :npv])
    np.testing.assert_array_equal(got["kmax"][b, h, :npv], kmax[0, 0, :npv])
    view, vlen, S = oquest.quest_select(qu, kmin, kmax, [L], P, cfg.top_pages)
    np.testing.assert_array_equal(got["score"][b, h, :npv], S[0, 0, :npv].astype(np.float32))
    assert np.all(np.isneginf(got["score"][b, h, npv:]))
    assert got["vlen"][b, h] == vlen[0, 0]
    np.testing.assert_array_equal(got["view"][b, h], view[0, 0])
    out, lse, _ = oracle.decode_attention(qu, Ku, Vu, [L], cfg.softmax_scale, view, vlen, P)
    tol = TOL[cfg.dtype]
    np.testing.assert_allclose(got["out"][b, hs], out[0], rtol=0, atol=tol)
    np.testing.assert_allclose(got["lse"][b, hs], lse[0], rtol=0, atol=tol)


def snapshot(st):
    return {"kmin": host(st.kmin), "kmax": host(st.kmax), "score": host(st.score), "view": host(st.view),
            "vlen": host(st.vlen), "out": host(st.out), "lse": host(st.lse)}


def test_tiny_f32_quest_decode_all_units_all_steps(se):
    cfg = get_config(0)
    banner("tiny f32 quest pipeline")
    st = QuestState(se, cfg, cfg.context + cfg.decode_steps)
    for step in range(cfg.decode_steps):
        q, L = st.step(se, step, splits=(0, 1, 3, 7, 64)[step % 5])
        torch.cuda.synchronize()
        got = snapshot(st)
        assert np.all(host(st.seq) == L)
        for unit in range(cfg.units):
            check_unit(cfg, st, q, L, unit, got)


@pytest.mark.parametrize("mode", ["separate", "fused", "whole"])
def test_tiny_bf16_quest_decode_with_partial_pages(se, mode):
    cfg = get_config(0, dtype="bf16", batch=3, n_q_heads=8, n_kv_heads=2, d_k=128, d_v=128, context=300,
                      top_pages=5, decode_steps=20)
    banner(f"tiny bf16 quest pipeline, ragged pages, {mode}")
    st = QuestState(se, cfg, cfg.context + cfg.decode_steps)
    for step in range(cfg.decode_steps):
        q, L = st.step(se, step, fused=mode == "fused", whole=mode == "whole")
        torch.cuda.synchronize()
        got = snapshot(st)
        for unit in range(cfg.units):
            check_unit(cfg, st, q, L, unit, got)


PAGE_CASES = {   # page size: (context, top pages, decode steps, d_k); steps cross page boundaries
    1: (200, 24, 3, 128),
    2: (150, 20, 5, 64),
    4: (201, 10, 6, 128),
    8: (250, 8, 10, 128),
    32: (700, 5, 40, 128),
}


@pytest.mark.parametrize("mode", ["separate", "whole"])
@pytest.mark.parametrize("page", list(PAGE_CASES))
def test_bf16_quest_decode_page_sizes(se, page, mode):
    """Quest over pages of 1 to 32 tokens (token views, slot quads split across
    entries below 4 tokens, within one entry from 4 on), every unit against the
    oracle at every step, through the separate calls and through the whole step."""
    ctx, k, steps, d = PAGE_CASES[page]
    cfg = get_config(0, dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2, d_k=d, d_v=d, context=ctx,
                      page_size=page, top_pages=k, decode_steps=steps)
    banner(f"bf16 quest page={page} {mode}")
    st = QuestState(se, cfg, cfg.context + cfg.decode_steps)
    for step in range(cfg.decode_steps):
        q, L = st.step(se, step, whole=mode == "whole")
        torch.cuda.synchronize()
        got = snapshot(st)
        assert np.all(host(st.seq) == L)
        for unit in range(cfg.units):
            check_unit(cfg, st, q, L, unit, got)


@pytest.mark.parametrize("k_pages", [1, 19, 40])
def test_quest_top_k_edges(se, k_pages):
    # k = 1, k just below the page count, k above the page count (every page selected)
    cfg = get_config(0, dtype="bf16", batch=2, n_q_heads=4, n_kv_heads=2, d_k=64, d_v=64, context=300,
                      page_size=16, top_pages=k_pages, decode_steps=1)
    banner(f"quest top-k edge k={k_pages}")
    st = QuestState(se, cfg, cfg.context + 1)
    q, L = st.step(se, 0)
    torch.cuda.synchronize()
    got = snapshot(st)
    for unit in range(cfg.units):
        check_unit(cfg, st, q, L, unit, got)
    assert np.all(got["vlen"] == min(k_pages, (L + 15) // 16))


def test_quest_32k_decode(se):
    """The 32K Quest workload at full size through the bench's call (se_quest_decode_step:
    the append and page scores, then the page selection and attention in one launch):
    every step runs on the GPU; every unit is compared with the oracle at the first, a
    middle and the last step."""
    cfg = get_config(1)
    banner("quest 32K: building caches")
    st = QuestState(se, cfg, cfg.context + cfg.decode_steps)
    every = range(cfg.units)
    sample_steps = {0: every, 31: every, cfg.decode_steps - 1: every}
    recall = []
    for step in range(cfg.decode_steps):
        q, L = st.step(se, step, whole=True)
        if step in sample_steps:
            torch.cuda.synchronize()
            banner(f"quest 32K: checking step {step}")
            got = snapshot(st)
            for unit in sample_steps[step]:
                check_unit(cfg, st, q, L, unit, got)
            for unit in range(cfg.units):
                b, h = divmod(unit, cfg.n_kv_heads)
                planted = set(gen.planted_pages(cfg, 0, unit).tolist())
                recall.append(len(planted & set(got["view"][b, h].tolist())) / len(planted))
    view = host(st.view)
    assert np.all(np.diff(view, axis=-1) > 0)
    print(f"planted-page recall (diagnostic only): {np.mean(recall):.3f}")


def quest_32k_state_buffers(st):
    return (st.k, st.v, st.kmin, st.kmax, st.seq, st.view, st.vlen, st.score, st.out, st.lse)


def test_quest_32k_step_deterministic_and_resumable(se):
    """At full size (the cross-block split merges run across the chip): a decode step
    replayed from saved caller-owned state gives bit-identical outputs, views, scores,
    lengths, metadata and cache rows; the state is saved to host memory and restored
    into the same buffers, as a caller resuming a sequence would."""
    cfg = get_config(1)
    banner("quest 32K determinism: building caches")
    st = QuestState(se, cfg, cfg.context + 4)
    for step in range(3):
        st.step(se, step, whole=True)
    torch.cuda.synchronize()
    saved = [t.cpu() for t in quest_32k_state_buffers(st)]
    results = []
    for rep in range(2):
        banner(f"quest 32K determinism: run {rep}")
        for t, h in zip(quest_32k_state_buffers(st), saved):
            t.copy_(h)
        st.step(se, 3, whole=True)
        torch.cuda.synchronize()
        results.append([t.cpu() for t in quest_32k_state_buffers(st)])
    for a, b, name in zip(results[0], results[1], ("k", "v", "kmin", "kmax", "seq", "view", "vlen", "score", "out",
                                                   "lse")):
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), \
            f"{name} differs between runs"
    assert torch.equal(results[0][4], torch.full((cfg.batch,), cfg.context + 4, dtype=torch.int32))


APPEND_CFGS = {
    "bf16_d128_g8": get_config(0, dtype="bf16", batch=3, n_q_heads=16, n_kv_heads=2, d_k=128, d_v=128),
    "f32_d64": get_config(0, batch=2, n_q_heads=4, n_kv_heads=2),
    "mla_576": get_config(4, batch=2, context=200, page_size=64),
}


@pytest.mark.parametrize("name", list(APPEND_CFGS))
def test_append_meta_matches_separate_calls(se, name):
    """se_kv_append_meta = se_kv_append + se_page_meta_update(first_page=-1), bit for bit:
    rows, every valid page's min / max and seq_len, across page boundaries and a full cache."""
    cfg = APPEND_CFGS[name]
    banner(f"append+meta {name}")
    dt = tdtype(cfg)
    B, H, D, Dv, P = cfg.batch, cfg.n_kv_heads, cfg.d_k, cfg.d_v, cfg.page_size
    cap = 4 * P + 3
    lens0 = [P - 1, 2 * P, cap - 2][:B] if B == 3 else [P - 1, cap - 2]
    c = se.cache(B, cfg.n_q_heads, H, D, Dv, cap, cfg.dtype, cfg.latent)
    K, V = gen.cache_kv(cfg, 5, cap, length=cap)
    ncp = (cap + P - 1) // P
    st = {}
    for tag in ("fused", "separate"):
        k = dev(K, dt)
        v = None if cfg.latent else dev(V, dt)
        kmin = torch.zeros((B, H, ncp, D), dtype=dt, device="cuda")
        kmax = torch.zeros_like(kmin)
        seq = torch.tensor(lens0, dtype=torch.int32, device="cuda")
        se.se_page_meta_update(c, k, kmin, kmax, seq, P, 0)
        st[tag] = (k, v, kmin, kmax, seq)
    for step in range(5):          # crosses a page boundary and runs into the full cache
        kn, vn = gen.decode_kv_new(cfg, 5, step)
        knd = dev(kn, dt)
        vnd = None if cfg.latent else dev(vn, dt)
        k, v, kmin, kmax, seq = st["fused"]
        se.se_kv_append_meta(c, k, v, knd, vnd, None, seq, kmin, kmax, P)
        k, v, kmin, kmax, seq = st["separate"]
        se.se_kv_append(c, k, v, knd, vnd, None, seq)
        se.se_page_meta_update(c, k, kmin, kmax, seq, P, -1)
        torch.cuda.synchronize()
        a, b = st["fused"], st["separate"]
        np.testing.assert_array_equal(host(a[4]), host(b[4]))
        np.testing.assert_array_equal(host(a[0]), host(b[0]))
        if not cfg.latent:
            np.testing.assert_array_equal(host(a[1]), host(b[1]))
        lens = host(a[4])
        for bb in range(B):
            npv = (int(lens[bb]) + P - 1) // P
            np.testing.assert_array_equal(host(a[2])[bb, :, :npv], host(b[2])[bb, :, :npv])
            np.testing.assert_array_equal(host(a[3])[bb, :, :npv], host(b[3])[bb, :, :npv])
    assert list(host(st["fused"][4])) == [min(l + 5, cap) for l in lens0]


def test_append_meta_into_freed_slot(se):
    """With a slot per unit (a slot freed by eviction), the page holding that slot is
    rebuilt over the valid slots and seq_len is unchanged."""
    cfg = APPEND_CFGS["bf16_d128_g8"]
    banner("append+meta into a slot")
    B, H, D, P = cfg.batch, cfg.n_kv_heads, cfg.d_k, cfg.page_size
    cap = 5 * P
    c = se.cache(B, cfg.n_q_heads, H, D, D, cap, "bf16")
    K, V = gen.cache_kv(cfg, 6, cap, length=cap)
    ncp = cap // P
    k, v = dev(K, torch.bfloat16), dev(V, torch.bfloat16)
    kmin = torch.zeros((B, H, ncp, D), dtype=torch.bfloat16, device="cuda")
    kmax = torch.zeros_like(kmin)
    seq = torch.full((B,), cap, dtype=torch.int32, device="cuda")
    se.se_page_meta_update(c, k, kmin, kmax, seq, P, 0)
    slots = np.array([[3, 40], [17, 79], [0, 64]], np.int32)
    kn, vn = gen.decode_kv_new(cfg, 6, 0)
    se.se_kv_append_meta(c, k, v, dev(kn, torch.bfloat16), dev(vn, torch.bfloat16), dev(slots, torch.int32), seq,
                         kmin, kmax, P)
    torch.cuda.synchronize()
    assert np.all(host(seq) == cap)
    Kx = K.copy()
    for bb in range(B):
        for h in range(H):
            Kx[bb, h, slots[bb, h]] = kn[bb, h]
    np.testing.assert_array_equal(host(k), Kx)
    mn, mx = oquest.page_meta(Kx, [cap] * B, P)
    np.testing.assert_array_equal(host(kmin), mn)
    np.testing.assert_array_equal(host(kmax), mx)
