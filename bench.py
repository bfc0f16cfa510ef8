"""Decode-step throughput of the sparse-decode path on one MI355X.

A step is one decode token for every batch row through one layer of the
Quest path on the 32K workload (16 x 32q/4kv x d128, pages of 16, top-128
pages): append the new K/V row, rebuild the last page's min/max, score and
select pages, and run split-K decode attention over the selected pages.
Steps rotate over --layers distinct layer caches so that each step's working
set has left the 256 MB Infinity Cache before it is read again.  Inputs are
resident in HBM before timing starts.

Prints one JSON line (tokens/s per layer-step, achieved HBM GB/s of the
attention kernel against the 8 TB/s peak, and the CPU oracle timed on a
bounded sample of the same step as a baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--layers", type=int, default=8, help="distinct layer caches rotated through")
    ap.add_argument("--attn-reps", type=int, default=20, help="graph replays for the attention-kernel timing")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    ap.add_argument("--splits", type=int, default=0, help="split-K factor of the attention (0 = library choice)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Layer:
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


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the path has no multi-GPU mode; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import sparse_attention_kv_quest_amd as se
    from workloads import generator as gen
    from workloads import get_config

    se.load()
    cfg = get_config(1)
    B, H, Hq, D, P, k = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.d_k, cfg.page_size, cfg.top_pages
    steps_per_layer = -(-(args.warmup + args.steps) // args.layers) + 2
    cap = cfg.context + steps_per_layer
    c = se.cache(B, Hq, H, D, D, cap, "bf16")
    log(f"workload quest_32k: B={B} Hq={Hq} Hkv={H} D={D} ctx={cfg.context} P={P} top={k} cap={cap} "
        f"layers={args.layers}")
    t0 = time.time()
    K, V = gen.cache_kv(cfg, 0, cap)
    K0 = torch.from_numpy(K).to("cuda", torch.bfloat16)
    V0 = torch.from_numpy(V).to("cuda", torch.bfloat16)
    del K, V
    q = torch.from_numpy(gen.decode_query(cfg, 0, 0)).to("cuda", torch.bfloat16)
    kn, vn = gen.decode_kv_new(cfg, 0, 0)
    kn = torch.from_numpy(kn).to("cuda", torch.bfloat16)
    vn = torch.from_numpy(vn).to("cuda", torch.bfloat16)
    layers = [Layer(se, cfg, c, K0, V0, 977 * i, torch) for i in range(args.layers)]
    del K0, V0
    ws_q = se.workspace(se.SE_OP_QUEST, c, P, k)
    ws_a = se.workspace(se.SE_OP_ATTN, c, k * P, args.splits)
    lse = torch.empty((B, Hq), device="cuda")
    torch.cuda.synchronize()
    log(f"caches ready in {time.time() - t0:.1f}s")
    # a plain 256 MiB device copy of known size: counter-based traffic figures are
    # scaled by what the counters report for it
    calib = torch.empty(128 << 20, dtype=torch.bfloat16, device="cuda")
    calib_copy = calib.clone()
    del calib, calib_copy
    torch.cuda.synchronize()

    def step(L):
        se.se_kv_append(c, L.k, L.v, kn, vn, None, L.seq)
        se.se_page_meta_update(c, L.k, L.kmin, L.kmax, L.seq, P, -1)
        se.se_quest_select(c, q, L.kmin, L.kmax, L.seq, P, k, L.view, L.vlen, None, ws_q)
        se.se_sparse_decode_attn(c, q, L.k, L.v, L.seq, L.view, L.vlen, k, P, cfg.softmax_scale, L.out, lse,
                                 num_splits=args.splits, ws=ws_a)

    def attn_only(L):
        se.se_sparse_decode_attn(c, q, L.k, L.v, L.seq, L.view, L.vlen, k, P, cfg.softmax_scale, L.out, lse,
                                 num_splits=args.splits, ws=ws_a)

    nL = args.layers
    use_graph = not args.no_graph
    # warm-up (eager), also compiles nothing: the kernels are prebuilt
    for i in range(args.warmup):
        step(layers[i % nL])
    torch.cuda.synchronize()

    if use_graph:
        s = torch.cuda.Stream()
        g_step = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_step, stream=s):
            for L in layers:
                step(L)
        g_attn = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_attn, stream=s):
            for L in layers:
                attn_only(L)
        torch.cuda.synchronize()

    # ---- timed whole steps
    reps = max(1, args.steps // nL) if use_graph else args.steps
    n_steps = reps * nL if use_graph else args.steps
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if use_graph:
        with torch.cuda.stream(s):
            e0.record(s)
            for _ in range(reps):
                g_step.replay()
            e1.record(s)
    else:
        e0.record()
        for i in range(n_steps):
            step(layers[i % nL])
        e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / n_steps

    # ---- attention kernel alone (same views), for the roofline
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if use_graph:
        with torch.cuda.stream(s):
            a0.record(s)
            for _ in range(args.attn_reps):
                g_attn.replay()
            a1.record(s)
        n_attn = args.attn_reps * nL
    else:
        a0.record()
        for i in range(args.attn_reps * nL):
            attn_only(layers[i % nL])
        a1.record()
        n_attn = args.attn_reps * nL
    torch.cuda.synchronize()
    us_attn = a0.elapsed_time(a1) * 1e3 / n_attn

    # algorithmic bytes of one attention launch: K and V rows of the selected tokens,
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

    tok_s = B / (ms_step * 1e-3)
    result = {
        "metric": "sparse decode tokens/s per layer-step (Quest, 32K ctx) + achieved HBM GB/s of the attention kernel",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": n_steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded grid-quantised N(0,1), 8 planted pages per KV head)",
        "config": {"workload": "quest_32k", "batch": B, "q_heads": Hq, "kv_heads": H, "head_dim": D,
                   "context": cfg.context, "page_size": P, "top_pages": k, "layers_rotated": nL,
                   "graph": use_graph, "attn_splits": args.splits},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "se_sparse_decode_attn (split-K main + combine)", "us_per_launch": round(us_attn, 3),
                     "bytes_per_launch": attn_bytes},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline(cfg, budget_s):
    """The CPU oracle, single-threaded, on a bounded sample of the same decode step:
    per unit, page metadata, the Quest page view and the attention over it."""
    from threadpoolctl import threadpool_limits
    import oracle
    from oracle import quest as oquest
    from workloads import generator as gen

    P, k, G = cfg.page_size, cfg.top_pages, cfg.group
    L = cfg.context + 1
    q = gen.decode_query(cfg, 0, 0)
    done, spent = 0, 0.0
    with threadpool_limits(1):
        for unit in range(cfg.units):
            Ku, Vu = gen.unit_kv(cfg, 0, unit, L)
            b, h = divmod(unit, cfg.n_kv_heads)
            qu = q[b:b + 1, h * G:(h + 1) * G]
            t0 = time.perf_counter()
            kmin, kmax = oquest.page_meta(Ku[None, None], [L], P)
            view, vlen, _ = oquest.quest_select(qu, kmin, kmax, [L], P, k)
            oracle.decode_attention(qu, Ku[None, None], Vu[None, None], [L], cfg.softmax_scale, view, vlen, P)
            spent += time.perf_counter() - t0
            done += 1
            if spent >= budget_s and done >= 4:
                break
    step_s = spent / done * cfg.units
    return {"value": round(cfg.batch / step_s, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {cfg.units} KV-head units of one quest_32k decode step "
                      f"(page metadata + page view + attention), scaled to the full step"}


if __name__ == "__main__":
    main()
