"""GPU parity of the MFMA latent-attention kernel (576-wide rows, V = first 512
columns) over head-group sizes, view kinds, ragged and empty views, logits and
split-K variations, against the CPU oracle through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import TOL, banner, dev, host, zeros
from workloads import generator as gen
from workloads import get_config

pytestmark = pytest.mark.gpu


def setup(se, heads, batch, cap, lens, layer=0):
    cfg = get_config(4, batch=batch, n_q_heads=heads, context=cap)
    C, _ = gen.cache_kv(cfg, layer, cap, length=cap)
    q = gen.decode_query(cfg, layer, 0)
    c = se.cache(batch, heads, 1, 576, 512, cap, "bf16", latent=True)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    return cfg, c, C, q, dev(C, torch.bfloat16), dev(q, torch.bfloat16), seq


def run(se, c, qd, cd, seq, view=None, vlen=None, view_cap=0, gran=1, scale=0.07, logit_cap=0, splits=0):
    B, Hq = c.batch, c.n_q_heads
    out, lse = zeros((B, Hq, 512)), zeros((B, Hq))
    logits = torch.full((B, Hq, logit_cap), 7.0, device="cuda") if logit_cap else None
    slots = view_cap * gran if view is not None else c.capacity
    ws = se.workspace(se.SE_OP_ATTN, c, slots, splits)
    se.se_sparse_decode_attn(c, qd, cd, None, seq, view, vlen, view_cap, gran, scale, out, lse, logits, logit_cap,
                             splits, ws)
    torch.cuda.synchronize()
    return host(out), host(lse), (host(logits) if logit_cap else None)


def check(got, ref, lens_or_counts, logit_cap):
    out, lse, lg = got
    ro, rl, rlg = ref
    tol = TOL["bf16"]
    np.testing.assert_allclose(out, ro, rtol=0, atol=tol)
    fin = np.isfinite(rl)
    np.testing.assert_allclose(lse[fin], rl[fin], rtol=0, atol=tol)
    assert np.all(np.isneginf(lse[~fin])) and np.all(out[~fin] == 0)
    if logit_cap:
        for b, n in enumerate(lens_or_counts):
            n = min(n, logit_cap)
            np.testing.assert_allclose(lg[b, :, :n], rlg[b, :, :n], rtol=0, atol=tol)


@pytest.mark.parametrize("heads", [16, 17, 24, 32, 48, 64])   # 17, 24: partial second head block of a group
@pytest.mark.parametrize("splits", [0, 1, 2, 3])
def test_mla_identity_view_head_groups(se, heads, splits):
    banner(f"mla mfma identity heads={heads} splits={splits}")
    cap = 777
    lens = [777, 650, 129]
    cfg, c, C, q, cd, qd, seq = setup(se, heads, 3, cap, lens)
    got = run(se, c, qd, cd, seq, scale=cfg.softmax_scale, logit_cap=cap + 3, splits=splits)
    ref = oracle.decode_attention(q, C, None, lens, cfg.softmax_scale, latent_dv=512, logit_cap=cap + 3)
    check(got, ref, lens, cap + 3)
    for b, L in enumerate(lens):
        assert np.all(got[2][b, :, L:] == 7.0)   # slots past the view: not written


@pytest.mark.parametrize("splits", [0, 2, 64])
def test_mla_page_view_ragged(se, splits):
    """64-token pages: views shorter than their capacity, pages past seq_len, an empty view."""
    banner(f"mla mfma page view splits={splits}")
    P, vc = 64, 12
    cap = 1600
    lens = [1600, 1000, 777, 64]
    cfg, c, C, q, cd, qd, seq = setup(se, 32, 4, cap, lens)
    rng = np.random.default_rng(11)
    view = np.full((4, 1, vc), -1, np.int32)
    vlen = np.zeros((4, 1), np.int32)
    for b in range(4):
        n = [vc, 9, 13, 0][b]
        n = min(n, vc)
        pages = np.sort(rng.choice(cap // P, n, replace=False))   # may lie past seq_len
        view[b, 0, :n] = pages
        vlen[b, 0] = n
    got = run(se, c, qd, cd, seq, dev(view, torch.int32), dev(vlen, torch.int32), vc, P, cfg.softmax_scale,
              logit_cap=vc * P, splits=splits)
    ref = oracle.decode_attention(q, C, None, lens, cfg.softmax_scale, view, vlen, P, latent_dv=512,
                                  logit_cap=vc * P)
    check(got, ref, [int(n) * P for n in vlen[:, 0]], vc * P)
    assert np.all(got[0][3] == 0) and np.all(np.isneginf(got[1][3]))


def test_mla_token_view_scattered(se):
    banner("mla mfma token view")
    cap, vc = 900, 301
    lens = [900, 611]
    cfg, c, C, q, cd, qd, seq = setup(se, 32, 2, cap, lens)
    rng = np.random.default_rng(5)
    view = np.full((2, 1, vc), -1, np.int32)
    vlen = np.zeros((2, 1), np.int32)
    for b, n in enumerate((vc, 150)):
        view[b, 0, :n] = np.sort(rng.choice(lens[b], n, replace=False))
        vlen[b, 0] = n
    got = run(se, c, qd, cd, seq, dev(view, torch.int32), dev(vlen, torch.int32), vc, 1, cfg.softmax_scale,
              logit_cap=200)
    ref = oracle.decode_attention(q, C, None, lens, cfg.softmax_scale, view, vlen, 1, latent_dv=512, logit_cap=200)
    check(got, ref, [int(n) for n in vlen[:, 0]], 200)


def test_mla_large_logits_force_rescaling(se):
    """A scale large enough that the running maximum has to move many times."""
    banner("mla mfma rescaling")
    cap = 1500
    lens = [1500, 1499]
    cfg, c, C, q, cd, qd, seq = setup(se, 32, 2, cap, lens, layer=3)
    got = run(se, c, qd, cd, seq, scale=0.9, splits=1)
    ref = oracle.decode_attention(q, C, None, lens, 0.9, latent_dv=512)
    check(got, ref, lens, 0)
