"""se_h2o_decode_step (a whole H2O decode step: append into the freed slot,
attention over every slot, accumulate, evict) against se_kv_append,
se_sparse_decode_attn with logits and se_h2o_accumulate_evict, bit for bit, over
consecutive steps: cache rows, seq_len, slot positions, scores, outputs, lse and
the evicted slots.  Shapes that run the one-launch step (bf16, d_k 128 and 64,
the 16K workload's 64 x 4 units) and shapes that run the three calls' kernels
(fp32, a capacity past the LDS logits).  The step call's results against the
oracle are checked at full size in test_gpu_h2o_omnikv.py."""
import numpy as np
import pytest
import torch

from tests.gpu_util import banner, dev, tdtype
from workloads import generator as gen
from workloads import get_config

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_d128_g4": (get_config(3, batch=2, n_q_heads=8, n_kv_heads=2, context=96, h2o_heavy=12, h2o_recent=6), 24),
    "d64_g8": (get_config(3, batch=3, n_q_heads=16, n_kv_heads=2, d_k=64, d_v=64, context=500, h2o_heavy=100,
                          h2o_recent=40), 12),
    "g16_cap768": (get_config(3, batch=2, n_q_heads=32, n_kv_heads=2, context=3000, h2o_heavy=600, h2o_recent=167),
                   6),
    "full_16k": (get_config(3), 6),
    "f32_fallback": (get_config(3, dtype="f32", batch=2, n_q_heads=8, n_kv_heads=2, context=300, h2o_heavy=40,
                                h2o_recent=20), 10),
    "cap_fallback": (get_config(3, batch=1, n_q_heads=8, n_kv_heads=2, context=9000, h2o_heavy=2000, h2o_recent=500),
                     4),
}


def same_bits(x, y):
    return torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8))


def start_state(cfg):
    B, H, D = cfg.batch, cfg.n_kv_heads, cfg.d_k
    cap = cfg.h2o_heavy + cfg.h2o_recent + 1
    K = np.zeros((B, H, cap, D), np.float32)
    V = np.zeros_like(K)
    pos = np.zeros((B, H, cap), np.int32)
    acc = np.zeros((B, H, cap), np.float32)
    for u in range(B * H):
        b, h = divmod(u, H)
        K[b, h] = gen.unit_rows(cfg, 0, gen.T_K, u, cap, D)
        V[b, h] = gen.unit_rows(cfg, 0, gen.T_V, u, cap, D)
        pos[b, h], acc[b, h] = gen.h2o_initial_state(cfg, 0, u)
    return K, V, pos, acc


@pytest.mark.parametrize("name", list(CASES))
def test_step_matches_separate_calls(se, name):
    cfg, steps = CASES[name]
    banner(f"h2o decode step vs separate calls: {name}")
    dt = tdtype(cfg)
    B, H, Hq, D = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k
    cap = cfg.h2o_heavy + cfg.h2o_recent + 1
    c = se.cache(B, Hq, H, D, D, cap, cfg.dtype)
    K, V, pos, acc = start_state(cfg)
    side = {}
    for tag in ("step", "separate"):
        side[tag] = dict(k=dev(K, dt), v=dev(V, dt), pos=dev(pos, torch.int32), acc=dev(acc),
                         seq=torch.full((B,), cap, dtype=torch.int32, device="cuda"),
                         out=torch.zeros((B, Hq, D), device="cuda"), lse=torch.zeros((B, Hq), device="cuda"))
    ev = [torch.full((B, H), cap - 1, dtype=torch.int32, device="cuda"),
          torch.full((B, H), -7, dtype=torch.int32, device="cuda")]
    ev_sep = torch.full((B, H), cap - 1, dtype=torch.int32, device="cuda")
    logits = torch.zeros((B, Hq, cap), device="cuda")
    ws_step = se.workspace(se.SE_OP_H2O_STEP, c, 0, 0)
    ws_att = se.workspace(se.SE_OP_ATTN, c, cap, 1)
    for t in range(steps):
        q = dev(gen.decode_query(cfg, 0, t), dt)
        kn, vn = gen.decode_kv_new(cfg, 0, t)
        knd, vnd = dev(kn, dt), dev(vn, dt)
        a = side["step"]
        se.se_h2o_decode_step(c, q, a["k"], a["v"], knd, vnd, ev[t % 2], a["seq"], a["pos"], a["acc"],
                              cfg.context + t, cfg.h2o_heavy, cfg.h2o_recent, cfg.softmax_scale, a["out"], a["lse"],
                              ev[(t + 1) % 2], ws_step)
        b = side["separate"]
        se.se_kv_append(c, b["k"], b["v"], knd, vnd, ev_sep, b["seq"])
        se.se_sparse_decode_attn(c, q, b["k"], b["v"], b["seq"], None, None, 0, 1, cfg.softmax_scale, b["out"],
                                 b["lse"], logits, cap, 1, ws_att)
        se.se_h2o_accumulate_evict(c, logits, b["lse"], cap, b["seq"], b["pos"], b["acc"], cfg.context + t,
                                   cfg.h2o_heavy, cfg.h2o_recent, ev_sep)
        torch.cuda.synchronize()
        for n in ("k", "v", "seq", "pos", "acc", "out", "lse"):
            assert same_bits(a[n], b[n]), f"step {t}: {n} differs"
        assert torch.equal(ev[(t + 1) % 2], ev_sep), f"step {t}: evicted slots differ"
        assert int((ev_sep >= 0).sum()) == B * H    # over budget every step: one eviction per unit


def test_step_rejects_aliased_slot_arrays(se):
    cfg, _ = CASES["tiny_d128_g4"]
    B, H, Hq, D = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k
    cap = cfg.h2o_heavy + cfg.h2o_recent + 1
    c = se.cache(B, Hq, H, D, D, cap, "bf16")
    t = torch.zeros(B * H * cap * D, dtype=torch.bfloat16, device="cuda")
    ev = torch.zeros((B, H), dtype=torch.int32, device="cuda")
    f = torch.zeros(B * Hq * D, device="cuda")
    with pytest.raises(se.SeError) as e:
        se.se_h2o_decode_step(c, t, t, t, t, t, ev, ev, ev, f, 5, cfg.h2o_heavy, cfg.h2o_recent, 0.1, f, None, ev,
                              se.workspace(se.SE_OP_H2O_STEP, c, 0, 0))
    assert e.value.status == -2
