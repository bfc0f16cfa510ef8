"""The workspace-free attention (se_sparse_decode_attn_noalloc) against
se_sparse_decode_attn with a caller workspace, through the C ABI: bit-identical
outputs on consecutive calls that share the library's static scratch (a large
call, then a smaller one, then one with logits over an identity view), each also
within the bf16 tolerance of the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quest as oquest
from tests.gpu_util import TOL, banner, dev, host, zeros
from workloads import generator as gen
from workloads import get_config

pytestmark = pytest.mark.gpu

CASES = (
    # Quest page views, split factor chosen by the library, then a smaller cache with 3 splits
    dict(shape=dict(batch=4, n_q_heads=32, n_kv_heads=4, context=3000, top_pages=32), splits=0, view="pages"),
    dict(shape=dict(batch=2, n_q_heads=16, n_kv_heads=2, context=700, top_pages=8), splits=3, view="pages"),
    # every slot, with logits (the H2O / OmniKV filter form)
    dict(shape=dict(batch=3, n_q_heads=8, n_kv_heads=1, context=1281, top_pages=1), splits=0, view="identity"),
)


def run_case(se, case, seed):
    cfg = get_config(0, dtype="bf16", d_k=128, d_v=128, page_size=16, **case["shape"])
    B, H, Hq, D, P, top = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.page_size, cfg.top_pages
    L = cfg.context
    K, V = gen.cache_kv(cfg, seed, L)
    q = gen.decode_query(cfg, seed, 0)
    c = se.cache(B, Hq, H, D, D, L, "bf16")
    k, v, qd = dev(K, torch.bfloat16), dev(V, torch.bfloat16), dev(q, torch.bfloat16)
    seq = torch.full((B,), L, dtype=torch.int32, device="cuda")
    if case["view"] == "pages":
        kmin, kmax = oquest.page_meta(K, [L] * B, P)
        view_h, vlen_h, _ = oquest.quest_select(q, kmin, kmax, [L] * B, P, top)
        view, vlen, cap, g, logit_cap = dev(view_h, torch.int32), dev(vlen_h, torch.int32), top, P, 0
    else:
        view_h = vlen_h = view = vlen = None
        cap, g, logit_cap = 0, 1, L
    res = {}
    for tag in ("workspace", "noalloc"):
        out, lse = zeros((B, Hq, D)), zeros((B, Hq))
        logits = zeros((B, Hq, logit_cap)) if logit_cap else None
        if tag == "workspace":
            ws = se.workspace(se.SE_OP_ATTN, c, cap * g if view is not None else L, case["splits"])
            se.se_sparse_decode_attn(c, qd, k, v, seq, view, vlen, cap, g, cfg.softmax_scale, out, lse, logits,
                                     logit_cap, case["splits"], ws)
        else:
            se.se_sparse_decode_attn_noalloc(c, qd, k, v, seq, view, vlen, cap, g, cfg.softmax_scale, out, lse,
                                             logits, logit_cap, case["splits"])
        torch.cuda.synchronize()
        res[tag] = (host(out), host(lse), None if logits is None else host(logits))
    a, b = res["workspace"], res["noalloc"]
    np.testing.assert_array_equal(b[0], a[0])
    np.testing.assert_array_equal(b[1], a[1])
    if a[2] is not None:
        np.testing.assert_array_equal(b[2], a[2])
    ref_out, ref_lse, ref_logits = oracle.decode_attention(q, K, V, [L] * B, cfg.softmax_scale, view_h, vlen_h, g,
                                                           logit_cap=logit_cap)
    np.testing.assert_allclose(b[0], ref_out, rtol=0, atol=TOL["bf16"])
    np.testing.assert_allclose(b[1], ref_lse, rtol=0, atol=TOL["bf16"])
    if ref_logits is not None:
        np.testing.assert_allclose(b[2], ref_logits, rtol=0, atol=TOL["bf16"])


def test_noalloc_attention_matches_workspace_call(se):
    for i, case in enumerate(CASES):
        banner(f"noalloc attention call {i}: {case}")
        run_case(se, case, 40 + i)


def test_noalloc_attention_rejects_oversized_request(se):
    """A request past the fixed scratch is refused before anything is enqueued."""
    c = se.cache(64, 32, 4, 128, 128, 16384, "bf16")
    dummy = torch.zeros(16, dtype=torch.float32, device="cuda")
    with pytest.raises(se.SeError) as e:
        se.se_sparse_decode_attn_noalloc(c, dummy, dummy, dummy, dummy, None, None, 0, 1, 0.1, dummy, None, None, 0,
                                         256)
    assert e.value.status == -6
