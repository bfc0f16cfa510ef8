"""se_quest_decode_step_fp8 (a whole Quest decode step over FP8 rows: the new rows
quantized, the appended page's min / max from the stored values, page scores, page
selection and attention) against se_kv_append_fp8, se_quest_select and
se_sparse_decode_attn_fp8, bit for bit, over consecutive steps: codes, scale bytes,
page metadata, seq_len, page scores, views, outputs and lse.  Shapes that run the
fused launches (d_k 128 and 64, ragged and fresh pages, a full cache, page counts
across the selection's key-per-thread variants, new rows that exercise the encoder:
zero, huge and tiny rows, values on a code boundary) and a shape that runs the
separate calls' kernels (more pages than the in-launch selection holds); a page size
the FP8 attention does not support is rejected before anything is written.  The
step call against the oracle at full size is in test_gpu_fp8.py."""
import numpy as np
import pytest
import torch

from tests.gpu_util import banner, dev
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
    "ncp_above_selection": (get_config(0, dtype="bf16", batch=1, n_q_heads=8, n_kv_heads=1, d_k=64, d_v=64,
                                       context=70000, top_pages=40), 2),
    # other page sizes: slot quads split across view entries (2) and within one (4, 32)
    "page2_d64": (get_config(0, dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2, context=150, page_size=2,
                             top_pages=20), 5),
    "page4": (get_config(0, dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2, d_k=128, d_v=128, context=201,
                         page_size=4, top_pages=10), 6),
    "page32": (get_config(0, dtype="bf16", batch=2, n_q_heads=16, n_kv_heads=2, d_k=128, d_v=128, context=700,
                          page_size=32, top_pages=5), 4),
}


def same_bits(x, y):
    return torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8))


def new_rows(cfg, step):
    """The step's new K / V rows, with encoder edge cases planted in some steps."""
    kn, vn = gen.decode_kv_new(cfg, 70, step)
    if step % 4 == 1:
        kn[0, 0] = 0.0                                  # a zero row: exponent 0, all codes 0
        vn[-1, -1] *= 2.0 ** -40                        # tiny values: the exponent's floor region
    if step % 4 == 2:
        kn[-1, 0] *= 1e6                                # huge values
        kn[0, -1, :] = 0.0
        kn[0, -1, 5] = 448.0                            # the largest code exactly
        kn[0, -1, 6] = -0.0
    return kn, vn


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_step_matches_separate_calls(se, name):
    cfg, steps = CASES[name]
    banner(f"fp8 quest decode step vs separate calls: {name}")
    B, H, Hq, D, P, k = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.page_size, cfg.top_pages
    cap = cfg.context + (steps if name != "d128_full_cache" else 2)
    c = se.cache(B, Hq, H, D, D, cap, "bf16")
    K, V = gen.cache_kv(cfg, 70, cap)
    ncp = (cap + P - 1) // P
    side = {}
    for tag in ("step", "separate"):
        st = dict(kq=torch.full((B, H, cap, D), 0x55, dtype=torch.uint8, device="cuda"),
                  ks=torch.full((B, H, cap), 0x55, dtype=torch.uint8, device="cuda"),
                  seq=torch.full((B,), cfg.context, dtype=torch.int32, device="cuda"),
                  kmin=torch.zeros((B, H, ncp, D), dtype=torch.bfloat16, device="cuda"),
                  view=torch.full((B, H, k), -7, dtype=torch.int32, device="cuda"),
                  vlen=torch.full((B, H), -7, dtype=torch.int32, device="cuda"),
                  score=torch.zeros((B, H, ncp), device="cuda"),
                  out=torch.zeros((B, Hq, D), device="cuda"), lse=torch.zeros((B, Hq), device="cuda"))
        st["vq"], st["vs"], st["kmax"] = torch.full_like(st["kq"], 0x55), torch.full_like(st["ks"], 0x55), \
            torch.zeros_like(st["kmin"])
        se.se_kv_quantize_fp8(c, dev(K, torch.bfloat16), dev(V, torch.bfloat16), st["seq"], st["kq"], st["vq"],
                              st["ks"], st["vs"], st["kmin"], st["kmax"], P)
        side[tag] = st
    ws_step = se.workspace(se.SE_OP_QUEST_STEP, c, P, k)
    ws_q = se.workspace(se.SE_OP_QUEST, c, P, k)
    ws_a = se.workspace(se.SE_OP_ATTN, c, k * P, 0)
    for step in range(steps):
        q = dev(gen.decode_query(cfg, 70, step), torch.bfloat16)
        kn, vn = new_rows(cfg, step)
        knd, vnd = dev(kn, torch.bfloat16), dev(vn, torch.bfloat16)
        a = side["step"]
        se.se_quest_decode_step_fp8(c, q, a["kq"], a["vq"], a["ks"], a["vs"], knd, vnd, a["seq"], a["kmin"],
                                    a["kmax"], P, k, cfg.softmax_scale, a["out"], a["lse"], a["view"], a["vlen"],
                                    a["score"], ws_step)
        b = side["separate"]
        se.se_kv_append_fp8(c, b["kq"], b["vq"], b["ks"], b["vs"], knd, vnd, b["seq"], b["kmin"], b["kmax"], P)
        se.se_quest_select(c, q, b["kmin"], b["kmax"], b["seq"], P, k, b["view"], b["vlen"], b["score"], ws_q)
        se.se_sparse_decode_attn_fp8(c, q, b["kq"], b["vq"], b["ks"], b["vs"], b["seq"], b["view"], b["vlen"], k, P,
                                     cfg.softmax_scale, b["out"], b["lse"], ws=ws_a)
        torch.cuda.synchronize()
        for n in ("kq", "vq", "ks", "vs", "seq", "kmin", "kmax", "score", "view", "vlen", "out", "lse"):
            assert same_bits(a[n], b[n]), f"step {step}: {n} differs"
    lens = side["step"]["seq"].cpu().numpy()
    assert np.all(lens == min(cfg.context + steps, cap))


def test_fp8_step_without_view_outputs(se):
    """The view and scores are optional outputs: the same out / lse without them."""
    cfg, _ = CASES["d128_g8_ragged"]
    banner("fp8 quest decode step without view outputs")
    B, H, Hq, D, P, k = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.page_size, cfg.top_pages
    cap = cfg.context + 1
    c = se.cache(B, Hq, H, D, D, cap, "bf16")
    K, V = gen.cache_kv(cfg, 71, cap)
    res = []
    for with_view in (True, False):
        kq = torch.zeros((B, H, cap, D), dtype=torch.uint8, device="cuda")
        vq = torch.zeros_like(kq)
        ks = torch.zeros((B, H, cap), dtype=torch.uint8, device="cuda")
        vs = torch.zeros_like(ks)
        seq = torch.full((B,), cfg.context, dtype=torch.int32, device="cuda")
        ncp = (cap + P - 1) // P
        kmin = torch.zeros((B, H, ncp, D), dtype=torch.bfloat16, device="cuda")
        kmax = torch.zeros_like(kmin)
        se.se_kv_quantize_fp8(c, dev(K, torch.bfloat16), dev(V, torch.bfloat16), seq, kq, vq, ks, vs, kmin, kmax, P)
        out, lse = torch.zeros((B, Hq, D), device="cuda"), torch.zeros((B, Hq), device="cuda")
        view = torch.zeros((B, H, k), dtype=torch.int32, device="cuda") if with_view else None
        vlen = torch.zeros((B, H), dtype=torch.int32, device="cuda") if with_view else None
        kn, vn = gen.decode_kv_new(cfg, 71, 0)
        se.se_quest_decode_step_fp8(c, dev(gen.decode_query(cfg, 71, 0), torch.bfloat16), kq, vq, ks, vs,
                                    dev(kn, torch.bfloat16), dev(vn, torch.bfloat16), seq, kmin, kmax, P, k,
                                    cfg.softmax_scale, out, lse, view, vlen, None,
                                    se.workspace(se.SE_OP_QUEST_STEP, c, P, k))
        torch.cuda.synchronize()
        res.append((out, lse, seq, kq, ks))
    for x, y in zip(res[0], res[1]):
        assert same_bits(x, y)


def test_fp8_step_rejects_unsupported_page_size(se):
    """A non-power-of-two page size: the FP8 attention rejects it, and so does the step,
    before it writes anything (codes, metadata and seq_len unchanged)."""
    cfg = get_config(0, dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2, d_k=128, d_v=128, context=300,
                     page_size=12, top_pages=6)
    B, H, Hq, D, P, k = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.page_size, cfg.top_pages
    cap = cfg.context + 2
    c = se.cache(B, Hq, H, D, D, cap, "bf16")
    kq = torch.zeros((B, H, cap, D), dtype=torch.uint8, device="cuda")
    vq = torch.zeros_like(kq)
    ks = torch.zeros((B, H, cap), dtype=torch.uint8, device="cuda")
    vs = torch.zeros_like(ks)
    seq = torch.full((B,), cfg.context, dtype=torch.int32, device="cuda")
    ncp = (cap + P - 1) // P
    kmin = torch.zeros((B, H, ncp, D), dtype=torch.bfloat16, device="cuda")
    kmax = torch.zeros_like(kmin)
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    kn = torch.ones((B, H, D), dtype=torch.bfloat16, device="cuda")
    out, lse = torch.zeros((B, Hq, D), device="cuda"), torch.zeros((B, Hq), device="cuda")
    with pytest.raises(se.SeError) as e:
        se.se_quest_decode_step_fp8(c, q, kq, vq, ks, vs, kn, kn, seq, kmin, kmax, P, k, cfg.softmax_scale, out, lse,
                                    ws=se.workspace(se.SE_OP_QUEST_STEP, c, P, k))
    assert se.STATUS[e.value.status] == "SE_ERR_UNSUPPORTED"
    torch.cuda.synchronize()
    assert torch.all(seq == cfg.context) and int(kq.sum()) == 0 and int(ks.sum()) == 0
