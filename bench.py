"""Decode-step throughput of the sparse-decode path on one MI355X.

Headline: the Quest path on the 32K workload (16 x 32q/4kv x d128, pages of 16,
top-128 pages).  A step is one decode token for every batch row through one
layer, one se_quest_decode_step call: a first launch appends the new K/V row,
folds it into the last page's min/max and scores every page; a second launch
selects each unit's top pages and runs split-K decode attention over them.
The roofline is that of the sparse decode attention kernel, timed alone over
the step's views (se_sparse_decode_attn).  Steps rotate over
--layers distinct layer caches so that each step's working set has left the
256 MB Infinity Cache before it is read again.  Inputs are resident in HBM
before timing starts; steps are replayed from HIP graphs.

The other workloads are timed the same way and reported under "workloads":
  snapkv_128k  prefill-end SnapKV eviction of a 131072-token prompt to 8192
               tokens (timed per call), then decode steps over the compacted
               cache (append + attention);
  h2o_16k      H2O decode steps (append into the freed slot, attention with
               logits, accumulate + evict) over 1024 heavy + 256 recent slots,
               and the prefill-end initialisation (scores of every prompt key
               over the full causal prefill, heavy + recent kept slots);
  omnikv_16k   48-layer OmniKV sweeps (dense layers 0-1, filter layers 2/8/16
               with top-2048 selection, 43 layers over the reused views);
  streaming_32k StreamingLLM decode steps on the Quest 32K shape: append, the
               sink + recent token view (4 + 2044 positions, the same 2048-token
               budget as the Quest view), attention over it;
  quest_32k_fp8 the Quest 32K step over FP8 KV rows (E4M3 codes, one power-of-two
               scale per row): FP8 append + last-page metadata, page scores and
               top-k, attention over the stored values;
  mla_128k     MLA latent Quest steps at 131072 tokens (576-wide latent rows,
               pages of 64, top-64 pages, 32 heads): se_quest_append_select,
               then the latent attention on MFMA.

Prints one JSON line: tokens/s per layer-step of the headline, achieved HBM
GB/s of its attention call against the 8 TB/s peak, per-workload figures, and
the CPU oracle timed on a bounded sample of the headline step as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
ALL_WORKLOADS = ("quest_32k", "snapkv_128k", "h2o_16k", "omnikv_16k", "mla_128k", "streaming_32k", "quest_32k_fp8")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--layers", type=int, default=8, help="distinct layer caches rotated through")
    ap.add_argument("--attn-reps", type=int, default=20, help="graph replays for the attention-call timing")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--splits", type=int, default=0, help="split-K factor of the attention (0 = library choice)")
    ap.add_argument("--workloads", default=",".join(ALL_WORKLOADS),
                    help="comma-separated subset of " + ",".join(ALL_WORKLOADS))
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- timing helpers

class Timer:
    """Captures a list of launches into one HIP graph (or replays them eagerly) and
    times replays with events on the stream the launches run on."""

    def __init__(self, torch, fn, use_graph):
        self.torch, self.fn, self.use_graph = torch, fn, use_graph
        self.stream = torch.cuda.Stream()
        if use_graph:
            self.graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(self.graph, stream=self.stream):
                fn()
            torch.cuda.synchronize()

    def ms_per_replay(self, reps):
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            e0.record(self.stream)
            for _ in range(reps):
                if self.use_graph:
                    self.graph.replay()
                else:
                    self.fn()
            e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps


def dev_grid(torch, shape, seed, dtype):
    """Seeded grid values on the device: round(32 x) / 32 clipped to +-255/32 with
    x ~ N(0, 1), the distribution of the host generator (torch's Philox stream)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
    x.mul_(32.0).round_().clamp_(-255.0, 255.0).div_(32.0)
    return x.to(dtype)


def free(torch):
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def sha16(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counter_traffic(summary, kernels, source):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None when
    the kernel source has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", summary)
    src = os.path.join(ROOT, "sparse_attention_kv_quest_amd", "csrc", source)
    if not (os.path.exists(path) and os.path.exists(src)):
        return None
    text = open(path).read()
    m = re.search(r"sha256\[:16\] at measurement: " + re.escape(source) + r" ([0-9a-f]{16})", text)
    if not m or m.group(1) != sha16(src):
        return None
    total = 0.0
    for k in kernels:
        m = re.search(re.escape(k) + r": scaled HBM traffic per launch = ([0-9.]+) MiB read \+ ([0-9.]+) MiB written",
                      text)
        if not m:
            return None
        total += (float(m.group(1)) + float(m.group(2))) * (1 << 20)
    return int(total)


# ---------------------------------------------------------------- headline: Quest 32K

class QuestLayer:
    """Device buffers of one layer: K, V, page metadata, view, outputs."""

    def __init__(self, se, cfg, c, K0, V0, shift, torch):
        B, H, Hq, D, P = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.page_size
        self.k = torch.roll(K0, shifts=shift, dims=2).contiguous() if shift else K0.clone()
        self.v = torch.roll(V0, shifts=shift, dims=2).contiguous() if shift else V0.clone()
        self.seq = torch.full((B,), cfg.context, dtype=torch.int32, device="cuda")
        ncp = (c.capacity + P - 1) // P
        self.kmin = torch.empty((B, H, ncp, D), dtype=K0.dtype, device="cuda")
        self.kmax = torch.empty_like(self.kmin)
        self.view = torch.empty((B, H, cfg.top_pages), dtype=torch.int32, device="cuda")
        self.vlen = torch.empty((B, H), dtype=torch.int32, device="cuda")
        self.out = torch.empty((B, Hq, D), device="cuda")
        se.se_page_meta_update(c, self.k, self.kmin, self.kmax, self.seq, P, 0)


def run_quest(se, torch, args):
    from workloads import generator as gen
    from workloads import get_config

    cfg = get_config(1)
    B, H, Hq, D, P, k = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.page_size, cfg.top_pages
    nL = args.layers
    # appends per layer: warm-up and timed steps, the append + select stage timing, slack
    steps_per_layer = -(-(args.warmup + args.steps) // nL) + 3 * args.attn_reps + 4
    cap = cfg.context + steps_per_layer
    c = se.cache(B, Hq, H, D, D, cap, "bf16")
    log(f"quest_32k: B={B} Hq={Hq} Hkv={H} D={D} ctx={cfg.context} P={P} top={k} cap={cap} layers={nL}")
    t0 = time.time()
    K, V = gen.cache_kv(cfg, 0, cap)
    K0 = torch.from_numpy(K).to("cuda", torch.bfloat16)
    V0 = torch.from_numpy(V).to("cuda", torch.bfloat16)
    del K, V
    q = torch.from_numpy(gen.decode_query(cfg, 0, 0)).to("cuda", torch.bfloat16)
    kn, vn = gen.decode_kv_new(cfg, 0, 0)
    kn = torch.from_numpy(kn).to("cuda", torch.bfloat16)
    vn = torch.from_numpy(vn).to("cuda", torch.bfloat16)
    layers = [QuestLayer(se, cfg, c, K0, V0, 977 * i, torch) for i in range(nL)]
    del K0, V0
    ws_q = se.workspace(se.SE_OP_QUEST_APPEND, c, P, 0)
    ws_a = se.workspace(se.SE_OP_ATTN, c, k * P, args.splits)
    ws_s = se.workspace(se.SE_OP_QUEST_STEP, c, P, k)
    lse = torch.empty((B, Hq), device="cuda")
    torch.cuda.synchronize()
    log(f"quest_32k: caches ready in {time.time() - t0:.1f}s")

    def step(L, view=False):
        """One decode step: se_quest_decode_step (launch 1: the new rows, the appended
        page's min / max, every page's score; launch 2: per unit the top pages and the
        attention over them).  view: also write the step's view (for the timings below)."""
        se.se_quest_decode_step(c, q, L.k, L.v, kn, vn, L.seq, L.kmin, L.kmax, P, k, cfg.softmax_scale, L.out, lse,
                                L.view if view else None, L.vlen if view else None, None, ws_s)

    def append_select(L):
        se.se_quest_append_select(c, q, L.k, L.v, kn, vn, L.seq, L.kmin, L.kmax, P, k, L.view, L.vlen, None, ws_q)

    def attn_only(L):
        se.se_sparse_decode_attn(c, q, L.k, L.v, L.seq, L.view, L.vlen, k, P, cfg.softmax_scale, L.out, lse,
                                 num_splits=args.splits, ws=ws_a)

    def two_calls(L):   # the same step as the separate calls: append + selection, then attention
        append_select(L)
        attn_only(L)

    use_graph = not args.no_graph
    for i in range(args.warmup):
        step(layers[i % nL], view=True)
    torch.cuda.synchronize()
    # one replay = exactly --steps decode steps, rotating over the layer caches
    n_steps = max(1, args.steps)
    t_step = Timer(torch, lambda: [step(layers[i % nL]) for i in range(n_steps)], use_graph)
    ms_step = t_step.ms_per_replay(1) / n_steps
    # the sparse decode attention alone over each layer's current view
    for L in layers:
        step(L, view=True)
    t_attn = Timer(torch, lambda: [attn_only(L) for L in layers], use_graph)
    us_attn = t_attn.ms_per_replay(args.attn_reps) * 1e3 / nL
    # for reference: the append + selection call alone, and the step as the two separate calls
    t_sel = Timer(torch, lambda: [append_select(L) for L in layers], use_graph)
    us_sel = t_sel.ms_per_replay(args.attn_reps) * 1e3 / nL
    t_two = Timer(torch, lambda: [two_calls(L) for L in layers], use_graph)
    us_two = t_two.ms_per_replay(max(1, args.attn_reps // 2)) * 1e3 / nL

    # algorithmic bytes of one attention call: K and V rows of the selected tokens,
    # plus q, the views and the fp32 outputs
    seq_h = layers[0].seq.cpu().numpy()
    vlen_h = layers[0].vlen.cpu().numpy()
    view_h = layers[0].view.cpu().numpy()
    toks = 0
    for b in range(B):
        for h in range(H):
            pages = view_h[b, h, :vlen_h[b, h]]
            toks += int(np.minimum(P, np.maximum(0, seq_h[b] - pages * P)).sum())
    attn_bytes = toks * D * 2 * 2 + B * Hq * D * 2 + B * H * k * 4 + B * Hq * (D + 1) * 4
    achieved = attn_bytes / (us_attn * 1e-6) / 1e9
    traffic = counter_traffic("quest_32k_hbm_counters.txt", ("attn_mfma_kernel",), "attn_mfma.hip")
    del layers
    free(torch)
    return cfg, {
        "tokens_per_s": B / (ms_step * 1e-3), "ms_per_step": ms_step, "steps": n_steps,
        "stages_us": {"step": round(ms_step * 1e3, 3), "attention": round(us_attn, 3),
                      "append_select": round(us_sel, 3), "two_call_step": round(us_two, 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "attn_mfma_kernel (se_sparse_decode_attn: split-K, splits merged in-kernel)", "us_per_launch": round(us_attn, 3),
                     "bytes_per_launch": attn_bytes},
    }


# ---------------------------------------------------------------- SnapKV 128K

def run_snapkv(se, torch, args):
    from workloads import get_config

    cfg = get_config(2)
    B, H, Hq, D = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k
    L, W, pool, budget = cfg.context, cfg.snap_window, cfg.snap_pool, cfg.snap_budget
    nL = args.layers
    steps = max(nL, args.steps // 2 // nL * nL)
    cap_out = budget + (steps // nL + 4)
    log(f"snapkv_128k: B={B} Hq={Hq} Hkv={H} D={D} prompt={L} W={W} pool={pool} budget={budget}")
    c = se.cache(B, Hq, H, D, D, L, "bf16")
    oc = se.cache(B, Hq, H, D, D, cap_out, "bf16")
    K = dev_grid(torch, (B, H, L, D), 21, torch.bfloat16)
    V = dev_grid(torch, (B, H, L, D), 22, torch.bfloat16)
    qo = dev_grid(torch, (B, Hq, W, D), 23, torch.bfloat16)
    k_out = torch.zeros((B, H, cap_out, D), dtype=torch.bfloat16, device="cuda")
    v_out = torch.zeros_like(k_out)
    kept = torch.empty((B, H, budget), dtype=torch.int32, device="cuda")
    olen = torch.empty((B,), dtype=torch.int32, device="cuda")
    ws = se.workspace(se.SE_OP_SNAPKV, c, L, W)

    def compact():
        se.se_snapkv_score_compact(c, qo, K, V, L, W, pool, budget, cfg.softmax_scale, oc, k_out, v_out, kept,
                                   None, olen, ws)

    compact()
    torch.cuda.synchronize()
    t_c = Timer(torch, compact, not args.no_graph)
    ms_compact = t_c.ms_per_replay(3)
    # algorithmic bytes: two passes over the prompt's keys, the kept rows read and written
    compact_bytes = 2 * B * H * L * D * 2 + 2 * 2 * B * H * budget * D * 2
    compact_flops = 2 * 2 * B * Hq * W * L * D   # q.k in both passes
    del K, V, t_c
    free(torch)

    # decode over the compacted cache: nL copies (identity view over seq_len rows)
    lay = []
    for i in range(nL):
        lay.append(dict(k=torch.roll(k_out, shifts=i, dims=2).contiguous(),
                        v=torch.roll(v_out, shifts=i, dims=2).contiguous(), seq=olen.clone(),
                        out=torch.empty((B, Hq, D), device="cuda")))
    q = dev_grid(torch, (B, Hq, D), 24, torch.bfloat16)
    kn = dev_grid(torch, (B, H, D), 25, torch.bfloat16)
    vn = dev_grid(torch, (B, H, D), 26, torch.bfloat16)
    lse = torch.empty((B, Hq), device="cuda")
    ws_a = se.workspace(se.SE_OP_ATTN, oc, cap_out, 0)
    ws_aa = se.workspace(se.SE_OP_APPEND_ATTN, oc, cap_out, 0)

    def step(Ly):   # append + attention over the compacted cache, one launch
        se.se_kv_append_decode_attn(oc, q, Ly["k"], Ly["v"], kn, vn, None, Ly["seq"], None, None, 0, 1,
                                    cfg.softmax_scale, Ly["out"], lse, ws=ws_aa)

    def attn(Ly):
        se.se_sparse_decode_attn(oc, q, Ly["k"], Ly["v"], Ly["seq"], None, None, 0, 1, cfg.softmax_scale,
                                 Ly["out"], lse, ws=ws_a)

    step(lay[0])
    t_s = Timer(torch, lambda: [step(Ly) for Ly in lay], not args.no_graph)
    t_a = Timer(torch, lambda: [attn(Ly) for Ly in lay], not args.no_graph)
    ms_step = t_s.ms_per_replay(steps // nL) / nL
    us_attn = t_a.ms_per_replay(4) * 1e3 / nL
    toks = int(lay[0]["seq"].sum().item()) * H
    attn_bytes = toks * D * 2 * 2 + B * Hq * D * 2 + B * Hq * (D + 1) * 4
    del lay, k_out, v_out, t_s, t_a
    free(torch)
    return {
        "workload": "snapkv_128k", "batch": B, "prompt": L, "budget": budget, "window": W, "pool": pool,
        "compaction": {"ms_per_call": round(ms_compact, 4),
                       "prompt_tokens_per_s": round(B * L / (ms_compact * 1e-3), 1),
                       "algorithmic_GBps": round(compact_bytes / (ms_compact * 1e-3) / 1e9, 1),
                       "score_TFLOPs": round(compact_flops / (ms_compact * 1e-3) / 1e12, 1)},
        "decode": {"tokens_per_s": round(B / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 5), "steps": steps,
                   "attn_us": round(us_attn, 3), "attn_GBps": round(attn_bytes / (us_attn * 1e-6) / 1e9, 1),
                   "attn_frac_of_peak": round(attn_bytes / (us_attn * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
    }


# ---------------------------------------------------------------- H2O 16K

def run_h2o(se, torch, args):
    from workloads import generator as gen
    from workloads import get_config

    cfg = get_config(3)
    B, H, Hq, D, G = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.group
    heavy, recent = cfg.h2o_heavy, cfg.h2o_recent
    cap = heavy + recent + 1
    nL = args.layers
    steps = max(nL, args.steps // nL * nL)
    log(f"h2o_16k: B={B} Hq={Hq} Hkv={H} D={D} ctx={cfg.context} heavy={heavy} recent={recent}")
    c = se.cache(B, Hq, H, D, D, cap, "bf16")
    pos = np.empty((B, H, cap), np.int32)
    acc = np.empty((B, H, cap), np.float32)
    for u in range(B * H):
        pos[u // H, u % H], acc[u // H, u % H] = gen.h2o_initial_state(cfg, 0, u)
    pos_d = torch.from_numpy(pos).cuda()
    acc_d = torch.from_numpy(acc).cuda()
    lay = []
    for i in range(nL):
        lay.append(dict(k=dev_grid(torch, (B, H, cap, D), 31 + 2 * i, torch.bfloat16),
                        v=dev_grid(torch, (B, H, cap, D), 32 + 2 * i, torch.bfloat16),
                        pos=pos_d.clone(), acc=acc_d.clone(),
                        seq=torch.full((B,), cap, dtype=torch.int32, device="cuda"),
                        ev=(torch.full((B, H), cap - 1, dtype=torch.int32, device="cuda"),
                            torch.full((B, H), -1, dtype=torch.int32, device="cuda")),
                        out=torch.empty((B, Hq, D), device="cuda"), cur=cfg.context + 2 * i))
    q = dev_grid(torch, (B, Hq, D), 30, torch.bfloat16)
    kn = dev_grid(torch, (B, H, D), 29, torch.bfloat16)
    vn = dev_grid(torch, (B, H, D), 28, torch.bfloat16)
    lse = torch.empty((B, Hq), device="cuda")
    ws_h = se.workspace(se.SE_OP_H2O_STEP, c, 0, 0)

    # one H2O decode step, se_h2o_decode_step: the new row into the slot the previous
    # step freed, attention over every slot, accumulate + evict, in one launch; a layer's
    # two steps alternate the slot arrays, so replays continue the eviction sequence
    def step(Ly, t):
        se.se_h2o_decode_step(c, q, Ly["k"], Ly["v"], kn, vn, Ly["ev"][t], Ly["seq"], Ly["pos"], Ly["acc"],
                              Ly["cur"] + t, heavy, recent, cfg.softmax_scale, Ly["out"], lse, Ly["ev"][1 - t], ws_h)

    for Ly in lay:
        step(Ly, 0)
        step(Ly, 1)
    t_s = Timer(torch, lambda: [step(Ly, t) for Ly in lay for t in (0, 1)], not args.no_graph)
    ms_step = t_s.ms_per_replay(max(1, steps // (2 * nL))) / (2 * nL)
    steps = max(1, steps // (2 * nL)) * 2 * nL
    # K and V rows of every slot, the slot's score (read, written) and position, q and out
    step_bytes = B * H * cap * (2 * D * 2 + 4 * 3) + B * Hq * D * (2 + 4)
    del lay, t_s
    free(torch)
    pre = h2o_prefill_timing(se, torch, cfg, c)
    return {"workload": "h2o_16k", "batch": B, "heavy": heavy, "recent": recent,
            "tokens_per_s": round(B / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 5), "steps": steps,
            "step_algorithmic_GBps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1), "prefill_init": pre}


def h2o_prefill_timing(se, torch, cfg, slots):
    """se_h2o_prefill_init on the full prompt (every prompt query of every head): its
    time, prompt tokens/s and the MFMA rate of its two causal passes."""
    B, H, Hq, D, L = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.context
    heavy, recent = cfg.h2o_heavy, cfg.h2o_recent
    c = se.cache(B, Hq, H, D, D, L, "bf16")
    qp = dev_grid(torch, (B, Hq, L, D), 33, torch.bfloat16)
    kp = dev_grid(torch, (B, H, L, D), 34, torch.bfloat16)
    vp = dev_grid(torch, (B, H, L, D), 35, torch.bfloat16)
    cap = slots.capacity
    k_s = torch.empty((B, H, cap, D), dtype=torch.bfloat16, device="cuda")
    v_s = torch.empty_like(k_s)
    pos = torch.empty((B, H, cap), dtype=torch.int32, device="cuda")
    acc = torch.empty((B, H, cap), device="cuda")
    ws = se.workspace(se.SE_OP_H2O_PREFILL, c, L, recent)

    def call():
        se.se_h2o_prefill_init(c, qp, kp, vp, L, heavy, recent, cfg.softmax_scale, slots, k_s, v_s, pos, acc, None, ws)

    call()
    torch.cuda.synchronize()
    t = Timer(torch, call, False)
    ms = t.ms_per_replay(2)
    flops = 2 * 2 * B * Hq * (L * (L + 1) / 2) * D        # q.k over the causal half, in each of the two passes
    del qp, kp, vp, k_s, v_s, ws, t
    free(torch)
    return {"ms_per_call": round(ms, 3), "prompt_tokens_per_s": round(B * L / (ms * 1e-3), 1),
            "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac_of_mfma_peak": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


# ---------------------------------------------------------------- OmniKV 16K, 48 layers

def omni_plan(n_layers, filters):
    """(mode, source filter layer) per layer: dense before the first filter layer,
    'filter' at a filter layer, else 'sparse' over the nearest filter layer below."""
    plan = []
    for layer in range(n_layers):
        if layer in filters:
            plan.append(("filter", layer))
        else:
            below = [f for f in filters if f < layer]
            plan.append(("sparse", max(below)) if below else ("dense", -1))
    return plan


def run_omnikv(se, torch, args):
    from workloads import get_config

    cfg = get_config(3)
    B, H, Hq, D = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k
    NL, filters, top = cfg.omni_layers, cfg.omni_filters, cfg.omni_top_k
    sweeps = max(4, args.steps // 8)
    cap = cfg.context + sweeps + 8
    log(f"omnikv_16k: B={B} Hq={Hq} Hkv={H} D={D} ctx={cfg.context} layers={NL} filters={filters} top={top}")
    c = se.cache(B, Hq, H, D, D, cap, "bf16")
    plan = omni_plan(NL, filters)
    ks, vs, seqs = [], [], []
    for layer in range(NL):
        ks.append(dev_grid(torch, (B, H, cap, D), 1000 + 2 * layer, torch.bfloat16))
        vs.append(dev_grid(torch, (B, H, cap, D), 1001 + 2 * layer, torch.bfloat16))
        seqs.append(torch.full((B,), cfg.context, dtype=torch.int32, device="cuda"))
    views = {f: torch.empty((B, H, top), dtype=torch.int32, device="cuda") for f in filters}
    vlens = {f: torch.empty((B, H), dtype=torch.int32, device="cuda") for f in filters}
    qs = [dev_grid(torch, (B, Hq, D), 2000 + layer, torch.bfloat16) for layer in range(NL)]
    kn = dev_grid(torch, (B, H, D), 2100, torch.bfloat16)
    vn = dev_grid(torch, (B, H, D), 2101, torch.bfloat16)
    out = torch.empty((B, Hq, D), device="cuda")
    lse = torch.empty((B, Hq), device="cuda")
    logits = torch.empty((B, Hq, cap), device="cuda")
    ws_dense = se.workspace(se.SE_OP_APPEND_ATTN, c, cap, 0)
    ws_sparse = se.workspace(se.SE_OP_APPEND_ATTN, c, top, 0)
    ws_topk = se.workspace(se.SE_OP_OMNIKV, c, cap, top)

    def sweep():   # every layer: the append and its attention in one launch
        for layer, (mode, src) in enumerate(plan):
            if mode == "sparse":
                se.se_kv_append_decode_attn(c, qs[layer], ks[layer], vs[layer], kn, vn, None, seqs[layer], views[src],
                                            vlens[src], top, 1, cfg.softmax_scale, out, lse, ws=ws_sparse)
            elif mode == "dense":
                se.se_kv_append_decode_attn(c, qs[layer], ks[layer], vs[layer], kn, vn, None, seqs[layer], None, None,
                                            0, 1, cfg.softmax_scale, out, lse, ws=ws_dense)
            else:
                se.se_kv_append_decode_attn(c, qs[layer], ks[layer], vs[layer], kn, vn, None, seqs[layer], None, None,
                                            0, 1, cfg.softmax_scale, out, lse, logits, cap, 0, ws_dense)
                se.se_omnikv_topk(c, logits, lse, cap, seqs[layer], top, views[layer], vlens[layer], None, ws_topk)

    sweep()
    t_s = Timer(torch, sweep, not args.no_graph)
    ms_sweep = t_s.ms_per_replay(sweeps - 2)
    n = cfg.context + sweeps
    n_dense = sum(1 for m, _ in plan if m != "sparse")
    n_sparse = NL - n_dense
    sweep_bytes = B * H * (n_dense * n * D * 4 + n_sparse * top * D * 4) + len(filters) * B * Hq * n * 4 * 2
    del ks, vs, t_s, logits
    free(torch)
    return {"workload": "omnikv_16k", "batch": B, "layers": NL, "filters": list(filters), "top_k": top,
            "tokens_per_s_per_48_layer_step": round(B / (ms_sweep * 1e-3), 1),
            "ms_per_48_layer_step": round(ms_sweep, 4), "ms_per_layer": round(ms_sweep / NL, 5),
            "sweeps": sweeps - 2, "sweep_algorithmic_GBps": round(sweep_bytes / (ms_sweep * 1e-3) / 1e9, 1)}


# ---------------------------------------------------------------- MLA 128K

def run_mla(se, torch, args):
    from workloads import get_config

    cfg = get_config(4)
    B, Hq, D, Dv, P, k = cfg.batch, cfg.n_q_heads, cfg.d_k, cfg.d_v, cfg.page_size, cfg.top_pages
    nL = args.layers
    steps = max(nL, args.steps // 2 // nL * nL)
    cap = cfg.context + steps // nL + 4
    log(f"mla_128k: B={B} heads={Hq} latent={D} (V {Dv}) ctx={cfg.context} P={P} top={k} layers={nL}")
    c = se.cache(B, Hq, 1, D, Dv, cap, "bf16", latent=True)
    ncp = (cap + P - 1) // P
    lay = []
    for i in range(nL):
        Ly = dict(c=torch.empty((B, 1, cap, D), dtype=torch.bfloat16, device="cuda"),
                  seq=torch.full((B,), cfg.context, dtype=torch.int32, device="cuda"),
                  kmin=torch.empty((B, 1, ncp, D), dtype=torch.bfloat16, device="cuda"),
                  view=torch.empty((B, 1, k), dtype=torch.int32, device="cuda"),
                  vlen=torch.empty((B, 1), dtype=torch.int32, device="cuda"),
                  out=torch.empty((B, Hq, Dv), device="cuda"))
        Ly["kmax"] = torch.empty_like(Ly["kmin"])
        for b in range(B):
            Ly["c"][b] = dev_grid(torch, (1, cap, D), 3000 + 64 * i + b, torch.bfloat16)
        se.se_page_meta_update(c, Ly["c"], Ly["kmin"], Ly["kmax"], Ly["seq"], P, 0)
        lay.append(Ly)
    q = dev_grid(torch, (B, Hq, D), 3900, torch.bfloat16)
    kn = dev_grid(torch, (B, 1, D), 3901, torch.bfloat16)
    lse = torch.empty((B, Hq), device="cuda")
    ws_s = se.workspace(se.SE_OP_QUEST_STEP, c, P, k)
    ws_a = se.workspace(se.SE_OP_ATTN, c, k * P, 0)

    def step(Ly):
        """One decode step (se_quest_decode_step: launch 1 appends the latent row, folds it
        into its page's min / max and scores every page; launch 2 selects each row's top
        pages and attends over them; the split combine).  The view is written for the
        attention-alone timing below."""
        se.se_quest_decode_step(c, q, Ly["c"], None, kn, None, Ly["seq"], Ly["kmin"], Ly["kmax"], P, k,
                                cfg.softmax_scale, Ly["out"], lse, Ly["view"], Ly["vlen"], None, ws_s)

    def attn(Ly):
        se.se_sparse_decode_attn(c, q, Ly["c"], None, Ly["seq"], Ly["view"], Ly["vlen"], k, P, cfg.softmax_scale,
                                 Ly["out"], lse, ws=ws_a)

    step(lay[0])
    t_s = Timer(torch, lambda: [step(Ly) for Ly in lay], not args.no_graph)
    t_a = Timer(torch, lambda: [attn(Ly) for Ly in lay], not args.no_graph)
    ms_step = t_s.ms_per_replay(steps // nL) / nL
    us_attn = t_a.ms_per_replay(4) * 1e3 / nL
    seq_h = lay[0]["seq"].cpu().numpy()
    vlen_h, view_h = lay[0]["vlen"].cpu().numpy(), lay[0]["view"].cpu().numpy()
    toks = 0
    for b in range(B):
        pages = view_h[b, 0, :vlen_h[b, 0]]
        toks += int(np.minimum(P, np.maximum(0, seq_h[b] - pages * P)).sum())
    attn_bytes = toks * D * 2 + B * Hq * D * 2 + B * k * 4 + B * Hq * (Dv + 1) * 4
    attn_flops = 2 * Hq * toks * (D + Dv)
    del lay, t_s, t_a
    free(torch)
    gbps = attn_bytes / (us_attn * 1e-6) / 1e9
    tfl = attn_flops / (us_attn * 1e-6) / 1e12
    return {"workload": "mla_128k", "batch": B, "heads": Hq, "latent": D, "d_v": Dv, "context": cfg.context,
            "page_size": P, "top_pages": k,
            "tokens_per_s": round(B / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 5), "steps": steps,
            "attn_us": round(us_attn, 3), "attn_GBps": round(gbps, 1), "attn_frac_of_hbm_peak": round(gbps / HBM_PEAK_GBS, 4),
            "attn_TFLOPs": round(tfl, 1), "attn_frac_of_mfma_peak": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4)}


# ---------------------------------------------------------------- StreamingLLM 32K

def run_streaming(se, torch, args):
    from workloads import get_config

    cfg = get_config(1)
    B, H, Hq, D = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k
    sink, recent = 4, cfg.top_pages * cfg.page_size - 4
    nL = args.layers
    steps = max(nL, args.steps // nL * nL)
    cap = cfg.context + steps // nL + args.attn_reps + 8
    log(f"streaming_32k: B={B} Hq={Hq} Hkv={H} D={D} ctx={cfg.context} sink={sink} recent={recent} layers={nL}")
    c = se.cache(B, Hq, H, D, D, cap, "bf16")
    vc = sink + recent
    lay = []
    for i in range(nL):
        lay.append(dict(k=dev_grid(torch, (B, H, cap, D), 4000 + 2 * i, torch.bfloat16),
                        v=dev_grid(torch, (B, H, cap, D), 4001 + 2 * i, torch.bfloat16),
                        seq=torch.full((B,), cfg.context, dtype=torch.int32, device="cuda"),
                        view=torch.empty((B, H, vc), dtype=torch.int32, device="cuda"),
                        vlen=torch.empty((B, H), dtype=torch.int32, device="cuda"),
                        out=torch.empty((B, Hq, D), device="cuda")))
    q = dev_grid(torch, (B, Hq, D), 4100, torch.bfloat16)
    kn = dev_grid(torch, (B, H, D), 4101, torch.bfloat16)
    vn = dev_grid(torch, (B, H, D), 4102, torch.bfloat16)
    lse = torch.empty((B, Hq), device="cuda")
    ws_a = se.workspace(se.SE_OP_ATTN, c, vc, 0)

    def attn(Ly):
        se.se_sparse_decode_attn(c, q, Ly["k"], Ly["v"], Ly["seq"], Ly["view"], Ly["vlen"], vc, 1, cfg.softmax_scale,
                                 Ly["out"], lse, ws=ws_a)

    ws_aa = se.workspace(se.SE_OP_APPEND_ATTN, c, vc, 0)

    def step(Ly):   # the view one append ahead, then the append and the attention in one launch
        se.se_streaming_view(c, Ly["seq"], sink, recent, Ly["view"], Ly["vlen"], 1)
        se.se_kv_append_decode_attn(c, q, Ly["k"], Ly["v"], kn, vn, None, Ly["seq"], Ly["view"], Ly["vlen"], vc, 1,
                                    cfg.softmax_scale, Ly["out"], lse, ws=ws_aa)

    for Ly in lay:
        step(Ly)
    t_s = Timer(torch, lambda: [step(Ly) for Ly in lay], not args.no_graph)
    t_a = Timer(torch, lambda: [attn(Ly) for Ly in lay], not args.no_graph)
    ms_step = t_s.ms_per_replay(steps // nL) / nL
    us_attn = t_a.ms_per_replay(args.attn_reps) * 1e3 / nL
    toks = int(lay[0]["vlen"].sum().item())
    attn_bytes = toks * D * 2 * 2 + B * Hq * D * 2 + B * H * vc * 4 + B * Hq * (D + 1) * 4
    gbps = attn_bytes / (us_attn * 1e-6) / 1e9
    del lay, t_s, t_a
    free(torch)
    return {"workload": "streaming_32k", "batch": B, "context": cfg.context, "sink": sink, "recent": recent,
            "tokens_per_s": round(B / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 5), "steps": steps,
            "attn_us": round(us_attn, 3), "attn_GBps": round(gbps, 1), "attn_frac_of_hbm_peak": round(gbps / HBM_PEAK_GBS, 4)}


# ---------------------------------------------------------------- Quest 32K over FP8 rows

def run_quest_fp8(se, torch, args):
    from workloads import get_config

    cfg = get_config(1)
    B, H, Hq, D, P, k = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.page_size, cfg.top_pages
    nL = args.layers
    steps = max(nL, args.steps // nL * nL)
    cap = cfg.context + steps // nL + args.attn_reps + 8
    log(f"quest_32k_fp8: B={B} Hq={Hq} Hkv={H} D={D} ctx={cfg.context} P={P} top={k} layers={nL}")
    c = se.cache(B, Hq, H, D, D, cap, "bf16")
    ncp = (cap + P - 1) // P
    lay = []
    for i in range(nL):
        Ly = dict(kq=torch.empty((B, H, cap, D), dtype=torch.uint8, device="cuda"),
                  ks=torch.empty((B, H, cap), dtype=torch.uint8, device="cuda"),
                  seq=torch.full((B,), cfg.context, dtype=torch.int32, device="cuda"),
                  kmin=torch.empty((B, H, ncp, D), dtype=torch.bfloat16, device="cuda"),
                  view=torch.empty((B, H, k), dtype=torch.int32, device="cuda"),
                  vlen=torch.empty((B, H), dtype=torch.int32, device="cuda"),
                  out=torch.empty((B, Hq, D), device="cuda"))
        Ly["vq"], Ly["vs"], Ly["kmax"] = torch.empty_like(Ly["kq"]), torch.empty_like(Ly["ks"]), torch.empty_like(Ly["kmin"])
        kb = dev_grid(torch, (B, H, cap, D), 5000 + 2 * i, torch.bfloat16)
        vb = dev_grid(torch, (B, H, cap, D), 5001 + 2 * i, torch.bfloat16)
        se.se_kv_quantize_fp8(c, kb, vb, Ly["seq"], Ly["kq"], Ly["vq"], Ly["ks"], Ly["vs"], Ly["kmin"], Ly["kmax"], P)
        del kb, vb
        lay.append(Ly)
    free(torch)
    q = dev_grid(torch, (B, Hq, D), 5100, torch.bfloat16)
    kn = dev_grid(torch, (B, H, D), 5101, torch.bfloat16)
    vn = dev_grid(torch, (B, H, D), 5102, torch.bfloat16)
    lse = torch.empty((B, Hq), device="cuda")
    ws_s = se.workspace(se.SE_OP_QUEST_STEP, c, P, k)
    ws_a = se.workspace(se.SE_OP_ATTN, c, k * P, args.splits)

    def attn(Ly):
        se.se_sparse_decode_attn_fp8(c, q, Ly["kq"], Ly["vq"], Ly["ks"], Ly["vs"], Ly["seq"], Ly["view"], Ly["vlen"], k,
                                     P, cfg.softmax_scale, Ly["out"], lse, num_splits=args.splits, ws=ws_a)

    def step(Ly):
        """One decode step over FP8 rows (se_quest_decode_step_fp8: launch 1 quantizes the
        new rows, folds their stored K values into the page's min / max and scores every
        page; launch 2 selects the pages and attends over the FP8 rows).  The view is
        written for the attention-alone timing."""
        se.se_quest_decode_step_fp8(c, q, Ly["kq"], Ly["vq"], Ly["ks"], Ly["vs"], kn, vn, Ly["seq"], Ly["kmin"],
                                    Ly["kmax"], P, k, cfg.softmax_scale, Ly["out"], lse, Ly["view"], Ly["vlen"], None,
                                    ws_s)

    for Ly in lay:
        step(Ly)
    t_s = Timer(torch, lambda: [step(Ly) for Ly in lay], not args.no_graph)
    t_a = Timer(torch, lambda: [attn(Ly) for Ly in lay], not args.no_graph)
    ms_step = t_s.ms_per_replay(steps // nL) / nL
    us_attn = t_a.ms_per_replay(args.attn_reps) * 1e3 / nL
    seq_h, vlen_h, view_h = lay[0]["seq"].cpu().numpy(), lay[0]["vlen"].cpu().numpy(), lay[0]["view"].cpu().numpy()
    toks = 0
    for b in range(B):
        for h in range(H):
            pages = view_h[b, h, :vlen_h[b, h]]
            toks += int(np.minimum(P, np.maximum(0, seq_h[b] - pages * P)).sum())
    # codes and scale bytes of the selected K and V rows, q, views, outputs
    attn_bytes = toks * (D + 1) * 2 + B * Hq * D * 2 + B * H * k * 4 + B * Hq * (D + 1) * 4
    gbps = attn_bytes / (us_attn * 1e-6) / 1e9
    del lay, t_s, t_a
    free(torch)
    return {"workload": "quest_32k_fp8", "batch": B, "context": cfg.context, "page_size": P, "top_pages": k,
            "kv_format": "E4M3 + one E8M0 scale per row",
            "tokens_per_s": round(B / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 5), "steps": steps,
            "attn_us": round(us_attn, 3), "attn_GBps": round(gbps, 1), "attn_frac_of_hbm_peak": round(gbps / HBM_PEAK_GBS, 4)}


# ---------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the path has no multi-GPU mode; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    wanted = [w.strip() for w in args.workloads.split(",") if w.strip()]
    bad = [w for w in wanted if w not in ALL_WORKLOADS]
    if bad:
        print(f"unknown workloads {bad}; choose from {ALL_WORKLOADS}", file=sys.stderr)
        sys.exit(2)
    if "quest_32k" in wanted and not args.no_cpu_baseline:
        # the CPU baseline's process pool forks from a forkserver started before the GPU is used
        import multiprocessing as mp
        import multiprocessing.forkserver as mpfs
        mp.get_context("forkserver").set_forkserver_preload(["numpy"])
        mpfs.ensure_running()
    import torch
    import sparse_attention_kv_quest_amd as se

    se.load()
    # the run's first device copy: a plain 256 MiB clone of known size, by which the
    # rocprofv3 FETCH_SIZE / WRITE_SIZE counts of the kernels are scaled to bytes
    calib = torch.zeros(128 << 20, dtype=torch.bfloat16, device="cuda")
    calib_copy = calib.clone()
    torch.cuda.synchronize()
    del calib, calib_copy
    result = {
        "metric": "sparse decode tokens/s per layer-step (Quest, 32K ctx) + achieved HBM GB/s of the attention kernel",
        "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": 0, "warmup": args.warmup, "ms_per_step": None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded grid-quantised N(0,1); Quest: 8 planted pages per KV head)",
    }
    extra = {}
    if "quest_32k" in wanted:
        cfg, r = run_quest(se, torch, args)
        result.update({"value": round(r["tokens_per_s"], 1), "steps": r["steps"],
                       "ms_per_step": round(r["ms_per_step"], 5)})
        result["config"] = {"workload": "quest_32k", "batch": cfg.batch, "q_heads": cfg.n_q_heads,
                            "kv_heads": cfg.n_kv_heads, "head_dim": cfg.d_k, "context": cfg.context,
                            "page_size": cfg.page_size, "top_pages": cfg.top_pages, "layers_rotated": args.layers,
                            "graph": not args.no_graph, "attn_splits": args.splits}
        result["roofline"] = r["roofline"]
        result["stages_us"] = r["stages_us"]
        log(f"quest_32k: {r['ms_per_step'] * 1e3:.2f} us/step; stages alone (us): {r['stages_us']}")
    else:
        result["config"] = {"workload": "none (headline skipped)"}
    runners = {"snapkv_128k": run_snapkv, "h2o_16k": run_h2o, "omnikv_16k": run_omnikv, "mla_128k": run_mla,
               "streaming_32k": run_streaming, "quest_32k_fp8": run_quest_fp8}
    for w in wanted:
        if w in runners:
            extra[w] = runners[w](se, torch, args)
            log(f"{w}: {json.dumps(extra[w])}")
    if extra:
        result["workloads"] = extra
    if "quest_32k" in wanted and not args.no_cpu_baseline:
        log("cpu baseline: the oracle over the host cores")
        result["cpu_baseline"] = cpu_baseline()
        log(f"cpu baseline: {json.dumps(result['cpu_baseline'])}")
    print(json.dumps(result), flush=True)


# ---------------------------------------------------------------- CPU oracle baseline
#
# The oracle as it stands (plain single-threaded NumPy per unit), run over the
# host's cores in a process pool: every job rebuilds one unit's inputs from the
# seeded generator (untimed), then times the same per-step work the GPU path
# does -- for Quest / MLA the appended row, the last page's min / max (the other
# pages' metadata carried over), page scores, top-k and attention; for H2O one
# full step; for OmniKV one 48-layer sweep -- and returns the timed seconds.

CPU_MAX_WORKERS = 16


def _cpu_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def _cpu_quest_unit(job):
    """Quest decode steps of one unit (GQA or latent): seconds spent in the steps."""
    cfg_id, unit, steps = job
    from oracle import attention as oatt
    from oracle import quest as oquest
    from workloads import generator as gen
    from workloads import get_config
    cfg = get_config(cfg_id)
    P, k, L = cfg.page_size, cfg.top_pages, cfg.context
    K0, V0 = gen.unit_kv(cfg, 0, unit, L)
    K = np.zeros((L + steps, cfg.d_k), np.float32)
    K[:L] = K0
    V = None
    if V0 is not None:
        V = np.zeros((L + steps, cfg.d_v), np.float32)
        V[:L] = V0
    kmin, kmax = oquest.page_meta(K[None, None], [L], P)
    b, h = divmod(unit, cfg.n_kv_heads)
    spent = 0.0
    for s in range(steps):
        qg = gen.unit_query(cfg, 0, s, unit)[None]
        kn, vn = gen.decode_kv_new(cfg, 0, s)
        t0 = time.perf_counter()
        K[L] = kn[b, h]
        if V is not None:
            V[L] = vn[b, h]
        L += 1
        p0 = (L - 1) // P * P
        mn, mx = oquest.page_meta(K[None, None, p0:L], [L - p0], P)
        kmin[0, 0, p0 // P], kmax[0, 0, p0 // P] = mn[0, 0, 0], mx[0, 0, 0]
        view, vlen, _ = oquest.quest_select(qg, kmin, kmax, [L], P, k)
        oatt.decode_attention(qg, K[None, None], None if V is None else V[None, None], [L], cfg.softmax_scale, view,
                              vlen, P, latent_dv=cfg.d_v if V is None else None)
        spent += time.perf_counter() - t0
    return spent


def _cpu_snap_unit(job):
    """SnapKV on one unit: (seconds of the eviction -- votes, pool, keep, compaction --,
    seconds of the decode steps over the compacted cache)."""
    unit, steps = job
    import oracle
    from oracle import snapkv as osnap
    from workloads import generator as gen
    from workloads import get_config
    cfg = get_config(2)
    L, W = cfg.context, cfg.snap_window
    K, V = gen.unit_kv(cfg, 0, unit, L)
    qo = gen.unit_obs_queries(cfg, 0, unit)
    t0 = time.perf_counter()
    pooled = osnap.snapkv_pool(osnap.unit_votes(qo, K, L, W, cfg.softmax_scale), cfg.snap_pool)
    kept = osnap.snapkv_keep(pooled, L, W, cfg.snap_budget)
    Kc, Vc = osnap.snapkv_compact(K, kept), osnap.snapkv_compact(V, kept)
    t_compact = time.perf_counter() - t0
    b, h = divmod(unit, cfg.n_kv_heads)
    t_dec = 0.0
    for s in range(steps):
        qg = gen.unit_query(cfg, 0, s, unit)
        kn, vn = gen.decode_kv_new(cfg, 0, s)
        t0 = time.perf_counter()
        Kc, Vc = np.concatenate([Kc, kn[b, h][None]]), np.concatenate([Vc, vn[b, h][None]])
        oracle.unit_attention(qg, Kc, Vc, cfg.softmax_scale)
        t_dec += time.perf_counter() - t0
    return t_compact, t_dec


def _cpu_h2o_unit(job):
    """H2O decode steps of one unit from its post-prefill state."""
    unit, steps = job
    from oracle import h2o as oh2o
    from workloads import generator as gen
    from workloads import get_config
    cfg = get_config(3)
    cap = cfg.h2o_heavy + cfg.h2o_recent + 1
    k = gen.unit_rows(cfg, 0, gen.T_K, unit, cap, cfg.d_k)
    v = gen.unit_rows(cfg, 0, gen.T_V, unit, cap, cfg.d_v)
    pos, acc = gen.h2o_initial_state(cfg, 0, unit)
    acc = acc.astype(np.float64)
    n, free = cap, cap - 1
    b, h = divmod(unit, cfg.n_kv_heads)
    spent = 0.0
    for t in range(steps):
        qg = gen.unit_query(cfg, 0, t, unit)
        kn, vn = gen.decode_kv_new(cfg, 0, t)
        t0 = time.perf_counter()
        _, _, pos, acc, n, free = oh2o.h2o_step(k, v, pos, acc, n, free, qg, kn[b, h], vn[b, h], cfg.context + t,
                                                cfg.h2o_heavy, cfg.h2o_recent, cfg.softmax_scale)
        spent += time.perf_counter() - t0
    return spent


def _cpu_omni_unit(job):
    """OmniKV 48-layer sweeps of one unit (appends, dense / filter / reused-view layers)."""
    unit, steps = job
    from oracle import omnikv as oomni
    from workloads import generator as gen
    from workloads import get_config
    cfg = get_config(3)
    b, h = divmod(unit, cfg.n_kv_heads)
    cap = cfg.context + steps
    Ks, Vs = [], []
    for layer in range(cfg.omni_layers):
        kk, vv = gen.unit_kv(cfg, layer, unit, cfg.context)
        Kl, Vl = np.zeros((cap, cfg.d_k), np.float32), np.zeros((cap, cfg.d_v), np.float32)
        Kl[:cfg.context], Vl[:cfg.context] = kk, vv
        Ks.append(Kl)
        Vs.append(Vl)
    spent = 0.0
    for s in range(steps):
        qs = [gen.unit_query(cfg, layer, s, unit) for layer in range(cfg.omni_layers)]
        new = [gen.decode_kv_new(cfg, layer, s) for layer in range(cfg.omni_layers)]
        t0 = time.perf_counter()
        for layer in range(cfg.omni_layers):
            Ks[layer][cfg.context + s], Vs[layer][cfg.context + s] = new[layer][0][b, h], new[layer][1][b, h]
        oomni.unit_sweep(qs, Ks, Vs, cfg.context + s + 1, cfg.omni_filters, cfg.omni_top_k, cfg.softmax_scale)
        spent += time.perf_counter() - t0
    return spent


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(steps=2, omni_units=32):
    """Decode tokens/s of the CPU oracle on every workload, from the seeded inputs of the
    same shapes: per workload, the timed seconds of every unit's steps are summed and
    divided by the worker count (units are independent, one per worker at a time)."""
    import concurrent.futures as cf
    import multiprocessing as mp
    from workloads import get_config

    n = max(1, min(CPU_MAX_WORKERS, len(os.sched_getaffinity(0))))
    ex = cf.ProcessPoolExecutor(n, mp_context=mp.get_context("forkserver"), initializer=_cpu_init)
    t_wall = time.time()
    q1, q4, c2, c3 = get_config(1), get_config(4), get_config(2), get_config(3)
    quest = list(ex.map(_cpu_quest_unit, [(1, u, steps) for u in range(q1.units)]))
    mla = list(ex.map(_cpu_quest_unit, [(4, u, steps) for u in range(q4.units)]))
    snap = list(ex.map(_cpu_snap_unit, [(u, steps) for u in range(c2.units)]))
    h2o = list(ex.map(_cpu_h2o_unit, [(u, steps) for u in range(c3.units)]))
    omni_sample = list(range(0, c3.units, c3.units // omni_units))[:omni_units]
    omni = list(ex.map(_cpu_omni_unit, [(u, steps) for u in omni_sample]))
    ex.shutdown()

    def tok_s(batch, secs, scale=1.0):
        step_wall = sum(secs) * scale / steps / n
        return round(batch / step_wall, 3)

    per = {
        "quest_32k": {"tokens_per_s": tok_s(q1.batch, quest)},
        "mla_128k": {"tokens_per_s": tok_s(q4.batch, mla)},
        "snapkv_128k": {"compaction_ms_per_call": round(sum(t for t, _ in snap) / n * 1e3, 1),
                        "decode_tokens_per_s": tok_s(c2.batch, [d for _, d in snap])},
        "h2o_16k": {"tokens_per_s": tok_s(c3.batch, h2o)},
        "omnikv_16k": {"tokens_per_s_per_48_layer_step": tok_s(c3.batch, omni, c3.units / len(omni_sample)),
                       "units_sampled": len(omni_sample)},
    }
    return {"value": per["quest_32k"]["tokens_per_s"], "unit": "tokens/s", "cores": n, "kind": "oracle",
            "sample": f"{steps} decode steps of every unit of quest_32k (the headline), with the same work per step "
                      f"as the GPU path (append, last-page min/max, page scores, top-k, attention); "
                      f"per-unit step seconds summed over units and divided by the {n} worker processes",
            "cpu_model": cpu_model(), "threads_per_worker": 1, "workloads": per,
            "wall_s": round(time.time() - t_wall, 1)}


if __name__ == "__main__":
    main()
