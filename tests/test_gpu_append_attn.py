"""GPU parity of se_kv_append_decode_attn (a decode step's append and attention
in one launch) against se_kv_append followed by se_sparse_decode_attn, bit for
bit: the K / V caches, seq_len, out, lse and logits, over identity, page and
token views, appends at seq_len (bumping it, or dropped at a full cache) and
into given slots (seq_len unchanged), several split factors, consecutive steps,
and the fp32 shape that runs the two calls' kernels."""
import numpy as np
import pytest
import torch

from tests.gpu_util import banner, dev, tdtype
from workloads import generator as gen
from workloads import get_config

pytestmark = pytest.mark.gpu

CFGS = {
    "bf16_d128_g8": get_config(0, dtype="bf16", batch=3, n_q_heads=16, n_kv_heads=2, d_k=128, d_v=128),
    "bf16_d64_g4": get_config(0, dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2),
    "f32_d64": get_config(0, batch=2, n_q_heads=4, n_kv_heads=2),
}


def same_bits(x, y):
    dt = torch.int16 if x.element_size() == 2 else torch.int32
    return torch.equal(x.contiguous().view(dt), y.contiguous().view(dt))


class Side:
    def __init__(self, se, cfg, cap, lens, seed):
        dt = tdtype(cfg)
        B, H = cfg.batch, cfg.n_kv_heads
        self.c = se.cache(B, cfg.n_q_heads, H, cfg.d_k, cfg.d_v, cap, cfg.dtype)
        K, V = gen.cache_kv(cfg, seed, cap, length=cap)
        self.k, self.v = dev(K, dt), dev(V, dt)
        self.seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
        self.out = torch.full((B, cfg.n_q_heads, cfg.d_v), 7.0, device="cuda")
        self.lse = torch.full((B, cfg.n_q_heads), 7.0, device="cuda")

    def state(self):
        return [self.k, self.v, self.seq, self.out, self.lse]


def run_case(se, cfg, cap, lens, steps, seed, view=None, gran=1, slots=None, splits=0, logit_cap=0):
    """view: None (identity) or (view_idx [B][H][vc] int32 numpy, view_len [B][H]); slots: None or a
    function step -> int32 [B][H] numpy."""
    dt = tdtype(cfg)
    B, H = cfg.batch, cfg.n_kv_heads
    fused, sep = Side(se, cfg, cap, lens, seed), Side(se, cfg, cap, lens, seed)
    vi = vl = None
    vc = 0
    if view is not None:
        vi, vl = dev(view[0], torch.int32), dev(view[1], torch.int32)
        vc = view[0].shape[-1]
    n_slots = vc * gran if view is not None else cap
    ws_f = se.workspace(se.SE_OP_APPEND_ATTN, fused.c, n_slots, splits)
    ws_s = se.workspace(se.SE_OP_ATTN, sep.c, n_slots, splits)
    lg = {t: (torch.full((B, cfg.n_q_heads, logit_cap), 7.0, device="cuda") if logit_cap else None)
          for t in ("fused", "sep")}
    for step in range(steps):
        q = dev(gen.decode_query(cfg, seed, step), dt)
        kn, vn = gen.decode_kv_new(cfg, seed, step)
        knd, vnd = dev(kn, dt), dev(vn, dt)
        sl = dev(slots(step), torch.int32) if slots is not None else None
        se.se_kv_append_decode_attn(fused.c, q, fused.k, fused.v, knd, vnd, sl, fused.seq, vi, vl, vc, gran,
                                    cfg.softmax_scale, fused.out, fused.lse, lg["fused"], logit_cap, splits, ws_f)
        se.se_kv_append(sep.c, sep.k, sep.v, knd, vnd, sl, sep.seq)
        se.se_sparse_decode_attn(sep.c, q, sep.k, sep.v, sep.seq, vi, vl, vc, gran, cfg.softmax_scale, sep.out,
                                 sep.lse, lg["sep"], logit_cap, splits, ws_s)
        torch.cuda.synchronize()
        for x, y, what in zip(fused.state(), sep.state(), ("k", "v", "seq_len", "out", "lse")):
            assert same_bits(x, y), f"step {step}: {what} differ"
        if logit_cap:
            assert same_bits(lg["fused"], lg["sep"]), f"step {step}: logits differ"
    return fused


@pytest.mark.parametrize("name", list(CFGS))
@pytest.mark.parametrize("splits", [0, 1, 3, 20])   # 20: partials merged by the combine kernel
def test_identity_append_at_seq_len(se, name, splits):
    """Appends at seq_len: ragged lengths, one batch row reaching the capacity (its
    later appends are dropped), logits on."""
    cfg = CFGS[name]
    banner(f"append+attn identity {name} splits={splits}")
    cap = 150
    lens = [37, cap - 2, 100][:cfg.batch]
    run_case(se, cfg, cap, lens, steps=4, seed=3, splits=splits, logit_cap=cap)


@pytest.mark.parametrize("name", ["bf16_d128_g8", "f32_d64"])
def test_identity_append_into_slots(se, name):
    """H2O's flow: rows go into given slots (seq_len unchanged) for some batch rows,
    at seq_len for a row whose head-0 slot is negative; a slot at the capacity is
    dropped."""
    cfg = CFGS[name]
    banner(f"append+attn slots {name}")
    B, H = cfg.batch, cfg.n_kv_heads
    cap = 129
    lens = [cap, cap, 60][:B]

    def slots(step):
        s = np.zeros((B, H), np.int32)
        s[0] = [(7 * step + 3) % cap, (5 * step + 11) % cap]
        s[1] = [cap, 40 + step]                   # head 0 dropped (at the capacity), head 1 into slot 40 + step
        if B > 2:
            s[2] = [-1, -1]                      # append at seq_len, seq_len grows
        return s
    run_case(se, cfg, cap, lens, steps=5, seed=4, slots=slots, splits=0, logit_cap=cap)


@pytest.mark.parametrize("gran", [16, 1])
def test_page_and_token_views(se, gran):
    """Views that hold the page / token receiving the new row, and views that do not."""
    cfg = CFGS["bf16_d128_g8"]
    banner(f"append+attn view g={gran}")
    B, H = cfg.batch, cfg.n_kv_heads
    cap = 16 * 20
    lens = [16 * 7 + 5, 16 * 12, 16 * 3 + 15]
    rng = np.random.default_rng(gran)
    vc = 6 if gran == 16 else 90
    idx = np.full((B, H, vc), -1, np.int32)
    vlen = np.zeros((B, H), np.int32)
    for b in range(B):
        n_ent = (lens[b] + 1 + gran - 1) // gran         # entries that exist after the append
        for h in range(H):
            pick = np.sort(rng.choice(n_ent, size=min(vc - 1, n_ent), replace=False))
            if h == 0 and (lens[b] // gran) not in pick:   # head 0 always sees the new token
                pick = np.sort(np.append(pick[1:], lens[b] // gran))
            idx[b, h, :pick.size] = pick
            vlen[b, h] = pick.size
    run_case(se, cfg, cap, lens, steps=1, seed=5, view=(idx, vlen), gran=gran, splits=0, logit_cap=vc * gran)
