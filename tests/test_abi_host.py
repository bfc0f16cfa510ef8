"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before launching."""
import ctypes
import os
import re

import pytest

import sparse_attention_kv_quest_amd as se

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "se.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(se.LIB_PATH):
        pytest.fail("libse.so is not built (run __graft_entry__.build())")
    return se.load()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:se_status|size_t|const char\*|int32_t)\s+(se_\w+)\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_symbols()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(se.EXPORTS) == set(names)


def test_version_and_strings(lib):
    assert se.se_abi_version() == 4
    assert se.se_status_string(0) == "ok"
    assert se.se_status_string(-6) == "workspace too small"
    assert se.se_status_string(123) == "unknown status"


def test_workspace_sizes(lib):
    c = se.cache(16, 32, 4, 128, 128, 32832, "bf16")
    assert se.se_workspace_bytes(se.SE_OP_QUEST, c, 16, 128) == 16 * 4 * 2052 * 4
    # fused append + select: 16 batch-row tickets (rounded up to 256 bytes), then the scores
    assert se.se_workspace_bytes(se.SE_OP_QUEST_APPEND, c, 16, 0) == 256 + 16 * 4 * 2052 * 4
    n = se.se_workspace_bytes(se.SE_OP_ATTN, c, 2048, 8)
    counters = 512          # 64 units x 2 head groups x int32, rounded up to 256 bytes
    assert n == counters + 16 * 4 * 8 * 8 * (128 + 2) * 4
    assert se.se_workspace_bytes(se.SE_OP_ATTN, c, 2048, 0) > 0
    bad = se.cache(16, 30, 4, 128, 128, 32832, "bf16")
    assert se.se_workspace_bytes(se.SE_OP_ATTN, bad, 2048, 8) == 0


def test_workspace_init_validation(lib):
    assert lib.se_workspace_init(None, 0, None) == 0                  # nothing to do, nothing launched
    assert lib.se_workspace_init(None, 256, None) == -1               # SE_ERR_NULL
    assert lib.se_workspace_init(0x10008, 256, None) == -4            # SE_ERR_ALIGN


FAKE = 0x10000     # an aligned, never dereferenced address: validation fails before any launch
MIS = 0x10008      # 8-byte aligned only


def call_attn(lib, c, q=FAKE, k=FAKE, v=FAKE, seq=FAKE, view=None, vlen=None, cap=0, g=1, scale=0.1, out=FAKE,
              logits=None, logit_cap=0, splits=0, ws=None, ws_bytes=0):
    return lib.se_sparse_decode_attn(ctypes.byref(c), q, k, v, seq, view, vlen, cap, g, scale, out, None, logits,
                                     logit_cap, splits, ws, ws_bytes, None)


def test_attention_argument_errors(lib):
    c = se.cache(2, 8, 2, 128, 128, 1024, "bf16")
    assert call_attn(lib, c, q=None) == -1
    assert call_attn(lib, c, q=MIS) == -4
    assert call_attn(lib, c, view=FAKE, vlen=None, cap=4, g=16) == -1
    assert call_attn(lib, c, view=FAKE, vlen=FAKE, cap=0, g=16) == -2
    assert call_attn(lib, c, logits=FAKE, logit_cap=0) == -2
    assert call_attn(lib, c, logits=FAKE, logit_cap=(1 << 31) // 4 + 1) == -2   # G * logit_cap past 2^31 - 1
    assert call_attn(lib, c, scale=0.0) == -2
    assert call_attn(lib, c, ws=None) == -6
    assert call_attn(lib, c, ws=FAKE, ws_bytes=16) == -6
    assert call_attn(lib, se.cache(2, 8, 3, 128, 128, 1024, "bf16")) == -2     # Hq % Hkv
    assert call_attn(lib, se.cache(2, 8, 2, 96, 96, 1024, "bf16")) == -2      # head width
    assert call_attn(lib, se.se_cache(2, 8, 2, 128, 128, 1024, 7, 0)) == -3   # dtype
    assert call_attn(lib, se.cache(2, 8, 2, 128, 64, 1024, "bf16")) == -2     # d_v != d_k without latent
    assert call_attn(lib, se.cache(2, 32, 2, 576, 512, 1024, "bf16", latent=True)) == -2  # latent needs Hkv 1


def test_other_entry_points_reject_bad_arguments(lib):
    c = se.cache(2, 8, 2, 128, 128, 1024, "bf16")
    cr = ctypes.byref(c)
    assert lib.se_kv_append(cr, FAKE, FAKE, None, FAKE, None, FAKE, None) == -1
    assert lib.se_kv_append(cr, FAKE, FAKE, MIS, FAKE, None, FAKE, None) == -4
    assert lib.se_page_meta_update(cr, FAKE, FAKE, FAKE, FAKE, 0, -1, None) == -2
    assert lib.se_page_meta_update(cr, FAKE, FAKE, FAKE, FAKE, 16, -2, None) == -2
    assert lib.se_quest_select(cr, FAKE, FAKE, FAKE, FAKE, 16, 0, FAKE, FAKE, None, FAKE, 1 << 20, None) == -5
    assert lib.se_quest_select(cr, FAKE, FAKE, FAKE, FAKE, 16, 8, FAKE, FAKE, None, FAKE, 4, None) == -6
    qa = lambda k_new=FAKE, P=16, top=8, ws=FAKE, ws_bytes=1 << 20: lib.se_quest_append_select(
        cr, FAKE, FAKE, FAKE, k_new, FAKE, FAKE, FAKE, FAKE, P, top, FAKE, FAKE, None, ws, ws_bytes, None)
    assert qa(k_new=None) == -1
    assert qa(k_new=MIS) == -4
    assert qa(P=0) == -2
    assert qa(top=0) == -5
    assert qa(ws=None) == -1                   # the fused call always needs its ticket counters
    assert qa(ws_bytes=64) == -6
    oc = se.cache(2, 8, 2, 128, 128, 64, "bf16")
    ocr = ctypes.byref(oc)
    snap = lambda L, W, pool, budget, out=ocr: lib.se_snapkv_score_compact(
        cr, FAKE, FAKE, FAKE, L, W, pool, budget, 0.1, out, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 30, None)
    assert snap(512, 0, 7, 64) == -5           # window must be >= 1
    assert snap(512, 512, 7, 64) == -5         # window < prompt_len
    assert snap(512, 16, 6, 64) == -5          # even pool kernel
    assert snap(512, 16, 7, 8) == -5           # budget < window
    assert snap(512, 16, 7, 128) == -5         # output capacity < budget
    assert snap(2048, 16, 7, 64) == -2         # prompt longer than the cache
    bad_out = se.cache(2, 8, 1, 128, 128, 64, "bf16")
    assert snap(512, 16, 7, 64, ctypes.byref(bad_out)) == -2
    h2o = lambda heavy, recent, cap=1024: lib.se_h2o_accumulate_evict(
        cr, FAKE, FAKE, cap, FAKE, FAKE, FAKE, 5000, heavy, recent, FAKE, None)
    assert h2o(1000, 24) == -5                 # heavy + recent + 1 > capacity
    assert h2o(-1, 4) == -5
    assert h2o(10, 4, cap=100) == -2           # logits narrower than the cache
    assert lib.se_omnikv_topk(cr, FAKE, FAKE, 1024, FAKE, 0, FAKE, FAKE, None, FAKE, 1 << 20, None) == -5
    assert lib.se_omnikv_topk(cr, FAKE, FAKE, 1024, FAKE, 2048, FAKE, FAKE, None, FAKE, 1 << 20, None) == -5
    assert lib.se_omnikv_topk(cr, None, FAKE, 1024, FAKE, 16, FAKE, FAKE, None, FAKE, 1 << 20, None) == -1


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "sparse_attention_kv_quest_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f), errors="ignore").read()
                assert "oracle" not in text.lower(), f


def call_attn_noalloc(lib, c, q=FAKE, k=FAKE, v=FAKE, seq=FAKE, view=None, vlen=None, cap=0, g=1, scale=0.1,
                      out=FAKE, logits=None, logit_cap=0, splits=0):
    return lib.se_sparse_decode_attn_noalloc(ctypes.byref(c), q, k, v, seq, view, vlen, cap, g, scale, out, None,
                                             logits, logit_cap, splits, None)


def test_noalloc_attention_argument_errors(lib):
    """The workspace-free attention checks its arguments as se_sparse_decode_attn does and
    rejects calls whose workspace would not fit its fixed scratch, before any HIP call."""
    c = se.cache(2, 8, 2, 128, 128, 1024, "bf16")
    assert call_attn_noalloc(lib, c, q=None) == -1
    assert call_attn_noalloc(lib, c, out=MIS) == -4
    assert call_attn_noalloc(lib, c, view=FAKE, vlen=None, cap=4, g=16) == -1
    assert call_attn_noalloc(lib, c, scale=float("nan")) == -2
    assert call_attn_noalloc(lib, c, splits=300) == -2
    assert call_attn_noalloc(lib, se.cache(2, 8, 3, 128, 128, 1024, "bf16")) == -2
    big = se.cache(64, 32, 4, 128, 128, 16384, "bf16")
    assert se.se_workspace_bytes(se.SE_OP_ATTN, big, 16384, 256) > (32 << 20)
    assert call_attn_noalloc(lib, big, splits=256) == -6
    # the headline shape fits
    quest = se.cache(16, 32, 4, 128, 128, 32832, "bf16")
    assert se.se_workspace_bytes(se.SE_OP_ATTN, quest, 2048, 0) <= (32 << 20)
