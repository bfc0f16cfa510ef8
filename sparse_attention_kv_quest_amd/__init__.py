"""Python binding of libse (the MI355X sparse-decode library).

Argument marshalling only: every call forwards device pointers of torch
tensors, sizes and the current HIP stream to the C ABI declared in
include/se.h; all computation runs in the library's HIP kernels.  The
functions carry the C names.  A nonzero status raises SeError.  If libse.so
is missing, `load()` raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libse.so")

SE_F32, SE_BF16 = 0, 1
SE_OP_QUEST, SE_OP_ATTN, SE_OP_SNAPKV, SE_OP_OMNIKV, SE_OP_QUEST_APPEND, SE_OP_H2O_PREFILL, SE_OP_APPEND_ATTN = \
    1, 2, 3, 4, 5, 6, 7
SE_OP_QUEST_STEP, SE_OP_H2O_STEP = 8, 9
STATUS = {0: "SE_OK", -1: "SE_ERR_NULL", -2: "SE_ERR_SHAPE", -3: "SE_ERR_DTYPE", -4: "SE_ERR_ALIGN",
          -5: "SE_ERR_BUDGET", -6: "SE_ERR_WORKSPACE", -7: "SE_ERR_UNSUPPORTED", -8: "SE_ERR_HIP"}

EXPORTS = ("se_kv_append", "se_kv_append_meta", "se_page_meta_update", "se_quest_select", "se_quest_append_select",
           "se_quest_decode_step",
           "se_sparse_decode_attn", "se_sparse_decode_attn_noalloc", "se_kv_append_decode_attn", "se_streaming_view", "se_pyramid_budgets",
           "se_kv_quantize_fp8", "se_kv_append_fp8", "se_sparse_decode_attn_fp8", "se_quest_decode_step_fp8",
           "se_chain_match", "se_chain_remap", "se_chain_append_positions", "se_h2o_prefill_init", "se_h2o_decode_step",
           "se_snapkv_score_compact", "se_h2o_accumulate_evict", "se_omnikv_topk",
           "se_workspace_bytes", "se_workspace_init", "se_status_string", "se_abi_version")


class SeError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")
        self.status = status


class se_cache(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("latent", ctypes.c_int32)]


_lib = None
_P, _I32, _F32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_C = ctypes.POINTER(se_cache)
_SIGS = {
    "se_kv_append": [_C, _P, _P, _P, _P, _P, _P, _P],
    "se_page_meta_update": [_C, _P, _P, _P, _P, _I32, _I32, _P],
    "se_kv_append_meta": [_C, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P],
    "se_quest_select": [_C, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _P, _SZ, _P],
    "se_quest_append_select": [_C, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _P, _SZ, _P],
    "se_quest_decode_step": [_C, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _F32, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "se_sparse_decode_attn": [_C, _P, _P, _P, _P, _P, _P, _I32, _I32, _F32, _P, _P, _P, _I32, _I32, _P, _SZ, _P],
    "se_sparse_decode_attn_noalloc": [_C, _P, _P, _P, _P, _P, _P, _I32, _I32, _F32, _P, _P, _P, _I32, _I32, _P],
    "se_kv_append_decode_attn": [_C, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _F32, _P, _P, _P, _I32, _I32, _P,
                                 _SZ, _P],
    "se_streaming_view": [_C, _P, _I32, _I32, _P, _P, _I32, _I32, _P],
    "se_kv_quantize_fp8": [_C, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P],
    "se_kv_append_fp8": [_C, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P],
    "se_quest_decode_step_fp8": [_C, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _F32, _P, _P, _P, _P, _P, _P,
                                 _SZ, _P],
    "se_sparse_decode_attn_fp8": [_C, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _F32, _P, _P, _P, _I32, _I32, _P, _SZ,
                                  _P],
    "se_pyramid_budgets": [_I32, _I32, _I32, _P],
    "se_chain_match": [_P, _I32, _P, _P, _I32, _P, _P],
    "se_chain_remap": [_C, _P, _I32, _P, _I32, _P, _P, _P],
    "se_chain_append_positions": [_C, _P, _P, _P, _I32, _P],
    "se_h2o_prefill_init": [_C, _P, _P, _P, _I32, _I32, _I32, _F32, _C, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "se_snapkv_score_compact": [_C, _P, _P, _P, _I32, _I32, _I32, _I32, _F32, _C, _P, _P, _P, _P, _P, _P, _SZ,
                                _P],
    "se_h2o_decode_step": [_C, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _F32, _P, _P, _P, _P, _SZ, _P],
    "se_h2o_accumulate_evict": [_C, _P, _P, _I32, _P, _P, _P, _I32, _I32, _I32, _P, _P],
    "se_omnikv_topk": [_C, _P, _P, _I32, _P, _I32, _P, _P, _P, _P, _SZ, _P],
}


def load(path: str = LIB_PATH):
    """Load libse.so (built by `python -m sparse_attention_kv_quest_amd.build`)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m sparse_attention_kv_quest_amd.build`")
    lib = ctypes.CDLL(path)
    for name, args in _SIGS.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int32
    lib.se_workspace_init.argtypes = [_P, _SZ, _P]
    lib.se_workspace_init.restype = ctypes.c_int32
    lib.se_workspace_bytes.argtypes = [_I32, _C, _I32, _I32]
    lib.se_workspace_bytes.restype = _SZ
    lib.se_status_string.argtypes = [_I32]
    lib.se_status_string.restype = ctypes.c_char_p
    lib.se_abi_version.argtypes = []
    lib.se_abi_version.restype = _I32
    _lib = lib
    return lib


def cache(batch, n_q_heads, n_kv_heads, d_k, d_v, capacity, dtype="bf16", latent=False) -> se_cache:
    dt = {"f32": SE_F32, "float32": SE_F32, "bf16": SE_BF16, "bfloat16": SE_BF16}[str(dtype).replace("torch.", "")]
    return se_cache(batch, n_q_heads, n_kv_heads, d_k, d_v, capacity, dt, int(bool(latent)))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("libse takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libse takes contiguous tensors")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _check(name, st):
    if st != 0:
        raise SeError(name, st, load().se_status_string(st).decode())


def se_abi_version() -> int:
    return load().se_abi_version()


def se_status_string(st: int) -> str:
    return load().se_status_string(st).decode()


def se_workspace_bytes(op: int, c: se_cache, a0: int, a1: int) -> int:
    return load().se_workspace_bytes(op, ctypes.byref(c), a0, a1)


def workspace(op: int, c: se_cache, a0: int, a1: int, device="cuda"):
    """A zero-filled device byte buffer of se_workspace_bytes(op, c, a0, a1) bytes (at
    least 256): workspaces start zero-filled and every call leaves their counters zero."""
    import torch
    n = max(256, se_workspace_bytes(op, c, a0, a1))
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    se_workspace_init(ws)
    return ws


def se_workspace_init(ws, nbytes=None, stream=None):
    n = _nbytes(ws) if nbytes is None else int(nbytes)
    _check("se_workspace_init", load().se_workspace_init(_ptr(ws), n, _stream(stream)))


def se_kv_append(c, k, v, k_new, v_new, slot, seq_len, stream=None):
    _check("se_kv_append", load().se_kv_append(ctypes.byref(c), _ptr(k), _ptr(v), _ptr(k_new), _ptr(v_new),
                                               _ptr(slot), _ptr(seq_len), _stream(stream)))


def se_kv_append_meta(c, k, v, k_new, v_new, slot, seq_len, kmin, kmax, page_size, stream=None):
    _check("se_kv_append_meta", load().se_kv_append_meta(
        ctypes.byref(c), _ptr(k), _ptr(v), _ptr(k_new), _ptr(v_new), _ptr(slot), _ptr(seq_len), _ptr(kmin),
        _ptr(kmax), page_size, _stream(stream)))


def se_page_meta_update(c, k, kmin, kmax, seq_len, page_size, first_page=-1, stream=None):
    _check("se_page_meta_update", load().se_page_meta_update(ctypes.byref(c), _ptr(k), _ptr(kmin), _ptr(kmax),
                                                             _ptr(seq_len), page_size, first_page, _stream(stream)))


def se_quest_select(c, q, kmin, kmax, seq_len, page_size, top_pages, view_idx, view_len, page_score=None,
                    ws=None, stream=None):
    _check("se_quest_select", load().se_quest_select(
        ctypes.byref(c), _ptr(q), _ptr(kmin), _ptr(kmax), _ptr(seq_len), page_size, top_pages, _ptr(view_idx),
        _ptr(view_len), _ptr(page_score), _ptr(ws), _nbytes(ws), _stream(stream)))


def se_quest_append_select(c, q, k, v, k_new, v_new, seq_len, kmin, kmax, page_size, top_pages, view_idx, view_len,
                           page_score=None, ws=None, stream=None):
    _check("se_quest_append_select", load().se_quest_append_select(
        ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(k_new), _ptr(v_new), _ptr(seq_len), _ptr(kmin), _ptr(kmax),
        page_size, top_pages, _ptr(view_idx), _ptr(view_len), _ptr(page_score), _ptr(ws), _nbytes(ws),
        _stream(stream)))


def se_quest_decode_step(c, q, k, v, k_new, v_new, seq_len, kmin, kmax, page_size, top_pages, scale, out, lse=None,
                         view_idx=None, view_len=None, page_score=None, ws=None, stream=None):
    _check("se_quest_decode_step", load().se_quest_decode_step(
        ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(k_new), _ptr(v_new), _ptr(seq_len), _ptr(kmin), _ptr(kmax),
        page_size, top_pages, scale, _ptr(out), _ptr(lse), _ptr(view_idx), _ptr(view_len), _ptr(page_score), _ptr(ws),
        _nbytes(ws), _stream(stream)))


def se_quest_decode_step_fp8(c, q, k_q, v_q, k_scale, v_scale, k_new, v_new, seq_len, kmin, kmax, page_size, top_pages,
                             scale, out, lse=None, view_idx=None, view_len=None, page_score=None, ws=None, stream=None):
    _check("se_quest_decode_step_fp8", load().se_quest_decode_step_fp8(
        ctypes.byref(c), _ptr(q), _ptr(k_q), _ptr(v_q), _ptr(k_scale), _ptr(v_scale), _ptr(k_new), _ptr(v_new),
        _ptr(seq_len), _ptr(kmin), _ptr(kmax), page_size, top_pages, scale, _ptr(out), _ptr(lse), _ptr(view_idx),
        _ptr(view_len), _ptr(page_score), _ptr(ws), _nbytes(ws), _stream(stream)))


def se_kv_quantize_fp8(c, k, v, seq_len, k_q, v_q, k_scale, v_scale, kmin=None, kmax=None, page_size=0,
                       stream=None):
    _check("se_kv_quantize_fp8", load().se_kv_quantize_fp8(
        ctypes.byref(c), _ptr(k), _ptr(v), _ptr(seq_len), _ptr(k_q), _ptr(v_q), _ptr(k_scale), _ptr(v_scale),
        _ptr(kmin), _ptr(kmax), page_size, _stream(stream)))


def se_kv_append_fp8(c, k_q, v_q, k_scale, v_scale, k_new, v_new, seq_len, kmin=None, kmax=None, page_size=1,
                     stream=None):
    _check("se_kv_append_fp8", load().se_kv_append_fp8(
        ctypes.byref(c), _ptr(k_q), _ptr(v_q), _ptr(k_scale), _ptr(v_scale), _ptr(k_new), _ptr(v_new), _ptr(seq_len),
        _ptr(kmin), _ptr(kmax), page_size, _stream(stream)))


def se_sparse_decode_attn_fp8(c, q, k_q, v_q, k_scale, v_scale, seq_len, view_idx, view_len, view_cap, granularity,
                              scale, out, lse=None, logits=None, logit_cap=0, num_splits=0, ws=None, stream=None):
    _check("se_sparse_decode_attn_fp8", load().se_sparse_decode_attn_fp8(
        ctypes.byref(c), _ptr(q), _ptr(k_q), _ptr(v_q), _ptr(k_scale), _ptr(v_scale), _ptr(seq_len), _ptr(view_idx),
        _ptr(view_len), view_cap, granularity, scale, _ptr(out), _ptr(lse), _ptr(logits), logit_cap, num_splits,
        _ptr(ws), _nbytes(ws), _stream(stream)))


def se_streaming_view(c, seq_len, sink, recent, view_idx, view_len, pending=0, stream=None):
    _check("se_streaming_view", load().se_streaming_view(ctypes.byref(c), _ptr(seq_len), sink, recent, _ptr(view_idx),
                                                         _ptr(view_len), view_idx.shape[-1], pending, _stream(stream)))


def se_h2o_prefill_init(c, q_prompt, k, v, prompt_len, heavy, recent, scale, slots, k_slots, v_slots, slot_pos, acc,
                        scores=None, ws=None, stream=None):
    _check("se_h2o_prefill_init", load().se_h2o_prefill_init(
        ctypes.byref(c), _ptr(q_prompt), _ptr(k), _ptr(v), prompt_len, heavy, recent, scale, ctypes.byref(slots),
        _ptr(k_slots), _ptr(v_slots), _ptr(slot_pos), _ptr(acc), _ptr(scores), _ptr(ws), _nbytes(ws), _stream(stream)))


def se_chain_match(tokens, prefixes):
    """(session index or -1, matched length) for host token lists; host computation."""
    arrs = [(ctypes.c_int32 * max(1, len(p)))(*p) for p in prefixes]
    ptrs = (ctypes.c_void_p * max(1, len(arrs)))(*[ctypes.cast(a, ctypes.c_void_p) for a in arrs])
    lens = (ctypes.c_int32 * max(1, len(prefixes)))(*[len(p) for p in prefixes])
    toks = (ctypes.c_int32 * max(1, len(tokens)))(*tokens)
    sess, n = ctypes.c_int32(), ctypes.c_int32()
    _check("se_chain_match", load().se_chain_match(toks, len(tokens), ptrs, lens, len(prefixes), ctypes.byref(sess),
                                                   ctypes.byref(n)))
    return sess.value, n.value


def se_chain_remap(c_out, map_in, kept, kept_len, map_out, stream=None):
    _check("se_chain_remap", load().se_chain_remap(
        ctypes.byref(c_out), _ptr(map_in), 0 if map_in is None else map_in.shape[-1], _ptr(kept), kept.shape[-1],
        _ptr(kept_len), _ptr(map_out), _stream(stream)))


def se_chain_append_positions(c, pos_map, seq_len, logical_len, n_new, stream=None):
    _check("se_chain_append_positions", load().se_chain_append_positions(
        ctypes.byref(c), _ptr(pos_map), _ptr(seq_len), _ptr(logical_len), n_new, _stream(stream)))


def se_pyramid_budgets(n_layers, avg_budget, min_budget):
    """Per-layer budgets (list of ints, layer 0 first); host computation."""
    out = (ctypes.c_int32 * max(1, n_layers))()
    _check("se_pyramid_budgets", load().se_pyramid_budgets(n_layers, avg_budget, min_budget, out))
    return list(out)[:n_layers]


def se_sparse_decode_attn(c, q, k, v, seq_len, view_idx, view_len, view_cap, granularity, scale, out, lse=None,
                          logits=None, logit_cap=0, num_splits=0, ws=None, stream=None):
    _check("se_sparse_decode_attn", load().se_sparse_decode_attn(
        ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(seq_len), _ptr(view_idx), _ptr(view_len), view_cap,
        granularity, scale, _ptr(out), _ptr(lse), _ptr(logits), logit_cap, num_splits, _ptr(ws), _nbytes(ws),
        _stream(stream)))


def se_sparse_decode_attn_noalloc(c, q, k, v, seq_len, view_idx, view_len, view_cap, granularity, scale, out,
                                  lse=None, logits=None, logit_cap=0, num_splits=0, stream=None):
    _check("se_sparse_decode_attn_noalloc", load().se_sparse_decode_attn_noalloc(
        ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(seq_len), _ptr(view_idx), _ptr(view_len), view_cap,
        granularity, scale, _ptr(out), _ptr(lse), _ptr(logits), logit_cap, num_splits, _stream(stream)))


def se_kv_append_decode_attn(c, q, k, v, k_new, v_new, slot, seq_len, view_idx, view_len, view_cap, granularity,
                             scale, out, lse=None, logits=None, logit_cap=0, num_splits=0, ws=None, stream=None):
    _check("se_kv_append_decode_attn", load().se_kv_append_decode_attn(
        ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(k_new), _ptr(v_new), _ptr(slot), _ptr(seq_len),
        _ptr(view_idx), _ptr(view_len), view_cap, granularity, scale, _ptr(out), _ptr(lse), _ptr(logits), logit_cap,
        num_splits, _ptr(ws), _nbytes(ws), _stream(stream)))



def se_snapkv_score_compact(c, q_obs, k, v, prompt_len, window, pool_kernel, budget, scale, out_c, k_out, v_out,
                            kept_pos, votes=None, out_seq_len=None, ws=None, stream=None):
    _check("se_snapkv_score_compact", load().se_snapkv_score_compact(
        ctypes.byref(c), _ptr(q_obs), _ptr(k), _ptr(v), prompt_len, window, pool_kernel, budget, scale,
        ctypes.byref(out_c), _ptr(k_out), _ptr(v_out), _ptr(kept_pos), _ptr(votes), _ptr(out_seq_len), _ptr(ws),
        _nbytes(ws), _stream(stream)))


def se_h2o_accumulate_evict(c, logits, lse, logit_cap, seq_len, slot_pos, acc, cur_pos, heavy_budget,
                            recent_window, evict_slot, stream=None):
    _check("se_h2o_accumulate_evict", load().se_h2o_accumulate_evict(
        ctypes.byref(c), _ptr(logits), _ptr(lse), logit_cap, _ptr(seq_len), _ptr(slot_pos), _ptr(acc), cur_pos,
        heavy_budget, recent_window, _ptr(evict_slot), _stream(stream)))


def se_h2o_decode_step(c, q, k, v, k_new, v_new, slot_in, seq_len, slot_pos, acc, cur_pos, heavy_budget, recent_window,
                       scale, out, lse, evict_out, ws=None, stream=None):
    _check("se_h2o_decode_step", load().se_h2o_decode_step(
        ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(k_new), _ptr(v_new), _ptr(slot_in), _ptr(seq_len),
        _ptr(slot_pos), _ptr(acc), cur_pos, heavy_budget, recent_window, scale, _ptr(out), _ptr(lse), _ptr(evict_out),
        _ptr(ws), _nbytes(ws), _stream(stream)))


def se_omnikv_topk(c, logits, lse, logit_cap, seq_len, top_k, view_idx, view_len, scores=None, ws=None,
                   stream=None):
    _check("se_omnikv_topk", load().se_omnikv_topk(
        ctypes.byref(c), _ptr(logits), _ptr(lse), logit_cap, _ptr(seq_len), top_k, _ptr(view_idx), _ptr(view_len),
        _ptr(scores), _ptr(ws), _nbytes(ws), _stream(stream)))
