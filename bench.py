#!/usr/bin/env python3
"""Benchmark of one SALS decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one call of sals_decode_step on one attention layer: latent query, latent scoring of
every cached token, top-k + window selection, gather + rebuild + RoPE + attention over the
selected tokens, split merge. The headline workload is the 4K-context Llama-2-7B-shaped layer
(B=8, H=32, d=128, ctx=4096, r=512, k=512, w=64, bf16 cache); the 32K-context Llama-3.1-8B-shaped
GQA layer (B=4, 32/8 heads, ctx=32768, r=256, k=2048, w=128) is reported beside it.

Inputs are resident in HBM before timing starts. Several independent copies of each input set
are rotated so that consecutive steps never find their inputs in the 256 MB Infinity Cache. W
untimed eager steps run first (their per-step time is reported as eager_us_per_step), then the K
steps are captured once as a HIP graph, replayed once untimed (upload), and exactly K steps are
timed as one replay between two device synchronisations. Per-kernel durations come from a
second captured pass of K steps through sals_decode_step_traced, which records HIP events
between the kernels on the launch stream. One JSON line goes to stdout; progress to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20
STAGES = ["latent_query", "latent_score", "topk_window", "select_attend", "combine"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(cfg, ctx):
    """Compulsory bytes/flops of one step (the method's own traffic, not the implementation's)."""
    s = 4 if cfg.dtype == "f32" else 2
    B, G, r, d, D = cfg.B, cfg.G, cfg.r, cfg.d, cfg.H_kv * cfg.d
    Tc = max(0, ctx - cfg.w)
    n_sel = min(cfg.k, Tc) + (ctx - Tc)
    lk_read = B * Tc * r * s
    sel_rows = 2 * B * G * n_sel * r * s
    p_bytes = 2 * D * r * s
    return dict(
        lk_read=lk_read, sel_rows=sel_rows, p_bytes=p_bytes, compulsory=lk_read + sel_rows + p_bytes,
        recon_flops=4 * B * cfg.H_kv * n_sel * r * d, score_flops=2 * B * G * Tc * r,
        attn_flops=4 * B * cfg.H_q * n_sel * d, n_sel=n_sel, Tc=Tc,
        stage_bytes={"latent_query": D * r * s + B * cfg.H_q * d * s, "latent_score": lk_read,
                     "topk_window": B * G * Tc * 4, "select_attend": sel_rows + p_bytes,
                     "combine": 0},
    )


def run_workload(cfg, steps, warmup, label):
    import numpy as np  # noqa: F401
    import torch

    import kv_cache_compression_sals_amd as sals
    from kv_cache_compression_sals_amd._lib import lib
    from workloads import decode_case

    t0 = time.time()
    case = decode_case(cfg)
    log(f"[{label}] generated inputs in {time.time() - t0:.1f}s")
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def dev(a):
        import numpy as np
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if cfg.dtype == "bf16" else torch.from_numpy(a)
        return t.cuda()

    base = {n: dev(case[n]) for n in ("q", "Lk", "Lv", "Pk", "Pv")}
    per_copy = sum(t.numel() * t.element_size() for t in base.values())
    n_copies = max(2, -(-2 * MALL_BYTES // per_copy))
    copies = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(n_copies - 1)]
    ctx = case["ctx"]
    ws_bytes = sals.sals_decode_workspace_bytes(base["q"], base["Pk"], ctx=ctx, k=cfg.k, w=cfg.w, G=cfg.G)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.B, cfg.H_q, cfg.d), dtype=torch.float32, device="cuda")
    log(f"[{label}] {n_copies} input copies of {per_copy / 1e6:.1f} MB, workspace {ws_bytes / 1e6:.1f} MB")

    def step(i):
        c = copies[i % n_copies]
        sals.sals_decode_step(c["q"], c["Lk"], c["Lv"], c["Pk"], c["Pv"], ctx=ctx, k=cfg.k, w=cfg.w, G=cfg.G,
                              rope_base=cfg.base, out=out, workspace=ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - t_start) / steps * 1e6

    # Timed region: the K steps captured once as a HIP graph (as a serving loop would), so the
    # host's per-launch cost does not pace the GPU. One untimed replay uploads the graph.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    us_step = (time.perf_counter() - t_start) / steps * 1e6

    # Per-kernel durations: the traced entry point records HIP events between the kernels on the
    # launch stream; the traced steps are captured and replayed the same way.
    import ctypes
    from kv_cache_compression_sals_amd._lib import SalsSelect, SalsShape
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    for row in evs:  # materialise the underlying hipEvent_t handles
        for e in row:
            e.record()
    torch.cuda.synchronize()
    shape = SalsShape(cfg.B, cfg.H_q, cfg.H_kv, cfg.d, cfg.r, 1 if cfg.dtype == "bf16" else 0)
    sel = SalsSelect(cfg.k, cfg.w, cfg.G)
    L = lib()

    def traced(i, stream):
        c = copies[i % n_copies]
        handles = (ctypes.c_void_p * 6)(*[e.cuda_event for e in evs[i]])
        st = L.sals_decode_step_traced(ctypes.byref(shape), ctypes.byref(sel), ctypes.c_float(cfg.base),
                                       c["q"].data_ptr(), c["Lk"].data_ptr(), c["Lv"].data_ptr(),
                                       c["Pk"].data_ptr(), c["Pv"].data_ptr(), c["Lk"].shape[1], ctx,
                                       out.data_ptr(), None, ws.data_ptr(), ws_bytes, stream.cuda_stream,
                                       handles, 6)
        assert st == 0, st

    tgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(tgraph):
        cs = torch.cuda.current_stream()
        for i in range(steps):
            traced(i, cs)
    tgraph.replay()
    torch.cuda.synchronize()
    tgraph.replay()
    torch.cuda.synchronize()
    stage_us = {}
    for j, name in enumerate(STAGES):
        stage_us[name] = sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)) / steps * 1e3
    traced_step_us = sum(evs[i][0].elapsed_time(evs[i][5]) for i in range(steps)) / steps * 1e3
    del graph, tgraph
    del copies
    torch.cuda.empty_cache()
    return case, us_step, stage_us, traced_step_us, eager_us


def roofline_for(cfg, ctx, stage_us):
    alg = algorithmic(cfg, ctx)
    dom = max(stage_us, key=stage_us.get)
    t = stage_us[dom] * 1e-6
    if dom == "select_attend":
        achieved = alg["recon_flops"] / t / 1e12
        rl = dict(kernel=dom, bound="mfma", achieved=round(achieved, 2), peak=BF16_MFMA_PEAK_TFLOPS,
                  unit="TFLOP/s", frac=round(achieved / BF16_MFMA_PEAK_TFLOPS, 4), traffic=None)
    else:
        achieved = alg["stage_bytes"][dom] / t / 1e9
        rl = dict(kernel=dom, bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                  frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=None)
    return rl, alg


def cpu_baseline(case, budget_s=12.0):
    import numpy as np  # noqa: F401
    import oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = 1
    B = case["q"].shape[0]
    done, t0 = 0, time.perf_counter()
    while done < B:
        oracle.decode_step(case["q"], case["Lk"], case["Lv"], case["Pk"], case["Pv"], ctx=case["ctx"],
                           k=case["k"], w=case["w"], G=case["G"], H_kv=case["H_kv"], base=case["base"],
                           dtype=case["dtype"], batches=[done])
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    per_seq = (time.perf_counter() - t0) / done
    return dict(value=round(per_seq * B * 1e6, 1), unit="us/decode_step", cores=cores, kind="oracle",
                sample=f"oracle decode step on {done} of {B} sequences (all heads), scaled x{B}/{done}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures the single-GPU decode path only; --gpus must be 1 "
              "(the method is independent per sequence and shards by batch with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from workloads import CONFIGS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    results = {}
    for key, label in (("c2", "ctx4k"), ("c3", "ctx32k")):
        cfg = CONFIGS[key]
        case, us, stage_us, traced_us, eager_us = run_workload(cfg, args.steps, args.warmup, label)
        rl, alg = roofline_for(cfg, case["ctx"], stage_us)
        gbps = alg["compulsory"] / (us * 1e-6) / 1e9
        results[key] = dict(case=case, us=us, stage_us=stage_us, traced_us=traced_us, roofline=rl, alg=alg,
                            gbps=gbps, eager_us=eager_us)
        log(f"[{label}] {us:.1f} us/step (graph; eager {eager_us:.1f}, traced {traced_us:.1f}), {gbps:.0f} GB/s effective, stages "
            + ", ".join(f"{k}={v:.1f}" for k, v in stage_us.items()))

    c2, c3 = results["c2"], results["c3"]
    cfg2 = CONFIGS["c2"]
    line = {
        "metric": "us/decode step + effective KV GB/s (% HBM peak) at 4K and 32K ctx, 1 GPU",
        "value": round(c2["us"], 2),
        "unit": "us/decode_step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(c2["us"] / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg2.name}: B={cfg2.B} H={cfg2.H_q} d={cfg2.d} ctx={cfg2.ctx} r={cfg2.r} "
                        f"k={cfg2.k} w={cfg2.w} G={cfg2.G}, one layer",
            "global_batch": cfg2.B, "seq_len": cfg2.ctx, "parallelism": "none (1 GPU)",
        },
        "kv_gbps": round(c2["gbps"], 1),
        "hbm_frac": round(c2["gbps"] / HBM_PEAK_GBPS, 4),
        "stage_us": {k: round(v, 2) for k, v in c2["stage_us"].items()},
        "eager_us_per_step": round(c2["eager_us"], 2),
        "recon_tflops": round(c2["alg"]["recon_flops"] / (c2["stage_us"]["select_attend"] * 1e-6) / 1e12, 1),
        "roofline": c2["roofline"],
        "ctx32k": {
            "workload": f"{CONFIGS['c3'].name}: B=4 H_q=32 H_kv=8 d=128 ctx=32768 r=256 k=2048 w=128 G=8",
            "us_per_step": round(c3["us"], 2),
            "kv_gbps": round(c3["gbps"], 1),
            "hbm_frac": round(c3["gbps"] / HBM_PEAK_GBPS, 4),
            "stage_us": {k: round(v, 2) for k, v in c3["stage_us"].items()},
            "eager_us_per_step": round(c3["eager_us"], 2),
            "recon_tflops": round(c3["alg"]["recon_flops"] / (c3["stage_us"]["select_attend"] * 1e-6) / 1e12, 2),
            "roofline": c3["roofline"],
        },
    }
    if not args.no_cpu_baseline:
        log("[cpu] timing the oracle on a bounded sample of the 4K workload")
        line["cpu_baseline"] = cpu_baseline(c2["case"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
