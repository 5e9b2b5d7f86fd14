#!/usr/bin/env python3
"""Benchmark of one SALS decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--replays R] [--no-cpu-baseline]
                    [--no-hbm-probe] [--only c1,c2,c3,c4,c5] [--calib-copy-mib M]

A step is one call of the decode path on one attention layer: latent query, latent scoring of
every cached token, top-k + window selection, gather + rebuild + RoPE + attention over the
selected tokens, split merge. The headline workload is the 4K-context Llama-2-7B-shaped layer
(B=8, H=32, d=128, ctx=4096, r=512, k=512, w=64, bf16 cache); the 32K-context Llama-3.1-8B-shaped
GQA layer (B=4, 32/8 heads, ctx=32768, r=256, k=2048, w=128, G=8) is reported beside it.

Inputs are resident in HBM before timing starts. Several independent copies of each input set
are rotated so that consecutive steps never find their inputs in the 256 MB Infinity Cache.
W untimed eager steps run first, then untimed steps for about 0.3 s more (the first calls after an
upload run slower: see settle()). The K steps are then captured once as a HIP graph (as a serving
loop runs its decode step), replayed once untimed (upload), and the timed region is exactly one
replay of the K steps between two device synchronisations: that is the value. Right after it,
the same K steps are issued eagerly through sals_decode_step_traced, which records HIP events on
the launch stream at every stage boundary; the events give each stage's average duration
(stage_us), and the host clock around that pass gives eager_us_per_step. The attention stage
(select_attend, the dominant kernel) is bounded by events that the runtime records at its
kernel's own start and end, so its figure (the roofline's avg_launch_us) is the kernel's duration
without the launch gap before it; the other stages include that gap. At ctx4k the two-head key
tile kernel ranks the score rows itself (no top-k launch): there the topk_window stage is only the
gap before that kernel, and the attention stage includes the ranking; at 128K the top-k stage is
the slice kernel alone and the attention stage includes the merge of the slices' candidates.
Each step is also followed,
outside the timed replay, by the dense baselines (comparators): flash-decode over the whole KV
cache, and the full rebuild of the cache followed by it. One JSON line goes to stdout; progress
goes to stderr.

--calib-copy-mib M first copies an M MiB buffer with torch (a plain copy kernel of known size),
so that a counter run can scale FETCH_SIZE / WRITE_SIZE to bytes.

The default run also measures, as extra objects of the same JSON line (--only picks a subset):
  c1  the tiny fp32 layer (ctx 512): latency only;
  c4  post-prefill compaction of the 16K-context VLM-shaped cache (kv_compact and its stages, the
      dense decode over the compact cache, reuse of the importance, sparsity, the frequency-domain
      outlier importance, the mixed-precision cache and its decode, the importance budgets), each
      timed as K back-to-back calls between HIP events (K at most 10);
  c5  one decode step through 32 independent resident layers of the 128K-context GQA workload
      (one replay of K captured 32-layer steps), with per-stage times from a traced pass.
Before the workloads, an in-tree streaming read (sals_hbm_read) measures the HBM read bandwidth
that hbm_frac_measured is stated against, and an in-tree register-only MFMA loop (sals_mfma_peak)
the bf16 MFMA throughput; every roofline object also gives its fraction of the measured peak
(peak_measured, frac_measured) beside the one of the specification. Each decode workload also reports the median, p10 and
p90 of the per-step time over --replays further replays, a warm variant (every step on the same
input copy), the scoring + attention HBM fraction, and threshold selection on the same layer.
The cpu_baseline object adds the CPU model and one-thread oracle times.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20
STAGES = ["latent_query", "latent_score", "topk_window", "select_attend", "combine"]


def stages_of(cfg):
    """Stage names of one step, in launch order. When one selection serves four or more KV heads
    the attention stops after the softmax and the value side runs as its own two kernels
    ("value": weighted latent row sum + P_v product); otherwise the split partials are merged
    ("combine")."""
    return STAGES[:4] + (["value"] if shared_value(cfg) else ["combine"])


def shared_value(cfg):
    return cfg.H_kv // cfg.G >= 4


# rows of at most this many candidates are ranked inside the two-head key tile kernel (512
# threads, 8 keys each) when it serves the layer: that kernel then also does the top-k stage
RANK_IN_KEYS_MAX = 4096


def ranks_in_keys(cfg, ctx):
    return (shared_value(cfg) and cfg.dtype == "bf16" and cfg.d == 128 and (cfg.H_kv // cfg.G) % 2 == 0
            and cfg.H_q // cfg.H_kv <= 4 and cfg.r in (128, 256, 384, 512)
            and max(0, ctx - cfg.w) <= RANK_IN_KEYS_MAX)


KDIR = os.path.join(ROOT, "kv_cache_compression_sals_amd", "csrc")
# sources whose change invalidates a kernel's stored traffic counters
KERNEL_SOURCES = {
    "select_attend": ["kernels/select_attend.inc", "kernels/select_attend_bf16_d128.hip",
                      "kernels/select_shared.hip", "topk_rows.h", "common.h"],
    "latent_score": ["kernels/latent_score.hip", "common.h"],
    "topk_window": ["kernels/topk.hip", "topk_rows.h", "common.h"],
    "latent_query": ["kernels/latent_query.hip", "common.h"],
    "combine": ["kernels/select_attend.hip", "common.h"],
    "value": ["kernels/value.hip", "common.h"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


SETTLE_S = 0.3


def settle(fn, seconds=SETTLE_S):
    """Untimed calls of fn for about `seconds` before a workload is timed. Right after its inputs
    are uploaded (the GPU idle while the host generated them) the first calls run slower: the
    compaction took about 1300 us for its first few calls and 1135 us from about 20 calls on, on
    fresh and on reused buffers alike. The timed region then measures the steady state."""
    import torch

    t_end = time.time() + seconds
    while time.time() < t_end:
        fn()
        torch.cuda.synchronize()


def source_hash(stage):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[stage]:
        with open(os.path.join(KDIR, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(stage, label):
    """HBM bytes per launch from the committed counter summary of this kernel and workload, or
    None when there is none or the kernel's sources have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{stage}_{label}_traffic.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_h = re.search(r"^source_sha256:\s*(\S+)", txt, re.M)
    m_t = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", txt, re.M)
    if not m_h or not m_t or m_h.group(1) != source_hash(stage):
        return None
    return int(m_t.group(1))


def algorithmic(cfg, ctx):
    """The method's own bytes and flops for one step (not the implementation's traffic).

    Per stage: bytes = inputs read once + outputs written once; flops = the dense contractions
    (the MFMA work). The value side of the attention is computed as (p^T L_v,sel) P_v^T, so its
    flops are a weighted row sum plus one d x r product per query head, not a V rebuild."""
    s = 4 if cfg.dtype == "f32" else 2
    B, G, r, d, D, Hq, Hkv = cfg.B, cfg.G, cfg.r, cfg.d, cfg.H_kv * cfg.d, cfg.H_q, cfg.H_kv
    Tc = max(0, ctx - cfg.w)
    kp = min(cfg.k, Tc)
    n_sel = kp + (ctx - Tc)
    lk_read = B * Tc * r * s
    half_rows = B * G * n_sel * r * s  # the selected rows of one of L_k, L_v
    sel_rows = 2 * half_rows
    p_bytes = 2 * D * r * s
    scores = B * G * Tc * 4
    k_rebuild = 2 * B * Hkv * n_sel * r * d
    value_side = 2 * B * Hq * n_sel * r + 2 * B * Hq * d * r
    logits = 2 * B * Hq * n_sel * d
    sel_idx = B * G * n_sel * 4
    q_in, o_out = B * Hq * d * s, B * Hq * d * 4
    stage_bytes = {
        "latent_query": D * r * s + q_in + B * G * r * 4,
        "latent_score": lk_read + B * G * r * 4 + scores,
        "topk_window": scores + sel_idx,
    }
    stage_flops = {"latent_query": 2 * B * Hq * d * r, "latent_score": 2 * B * G * Tc * r, "topk_window": 0}
    if shared_value(cfg):
        # attention up to the softmax, probabilities out; then the value kernels read them back
        probs = B * Hq * n_sel * 4
        stage_bytes["select_attend"] = half_rows + D * r * s + sel_idx + q_in + probs
        if ranks_in_keys(cfg, ctx):
            # the key tile kernel ranks the score rows itself: the top-k stage is its launch gap
            stage_bytes["select_attend"] += scores
            stage_bytes["topk_window"] = 0
        stage_bytes["value"] = half_rows + D * r * s + sel_idx + probs + o_out
        stage_flops["select_attend"] = k_rebuild + logits
        stage_flops["value"] = value_side
    else:
        # the gather kernel ends with latent sums z = p^T L_v,sel per split; the split merge
        # applies P_v once per head and writes the output (the workloads here all have several
        # splits; with one split both would run in the gather kernel)
        stage_bytes["select_attend"] = sel_rows + D * r * s + sel_idx + q_in
        stage_bytes["combine"] = D * r * s + o_out
        stage_flops["select_attend"] = k_rebuild + 2 * B * Hq * n_sel * r + logits
        stage_flops["combine"] = 2 * B * Hq * d * r
    return dict(
        lk_read=lk_read, sel_rows=sel_rows, p_bytes=p_bytes, compulsory=lk_read + sel_rows + p_bytes,
        k_rebuild_flops=k_rebuild, n_sel=n_sel, Tc=Tc, stage_bytes=stage_bytes, stage_flops=stage_flops,
    )


def run_workload(cfg, steps, warmup, label, replays=10, comparators=True):
    import numpy as np
    import torch

    import kv_cache_compression_sals_amd as sals
    from kv_cache_compression_sals_amd._lib import SalsSelect, SalsShape, lib
    from workloads import decode_case

    t0 = time.time()
    case = decode_case(cfg)
    log(f"[{label}] generated inputs in {time.time() - t0:.1f}s")

    def dev(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if cfg.dtype == "bf16" else torch.from_numpy(a)
        return t.cuda()

    base = {n: dev(case[n]) for n in ("q", "Lk", "Lv", "Pk", "Pv")}
    per_copy = sum(t.numel() * t.element_size() for t in base.values())
    n_copies = max(2, -(-2 * MALL_BYTES // per_copy))
    copies = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(n_copies - 1)]
    ctx = case["ctx"]
    kw = dict(ctx=ctx, k=cfg.k, w=cfg.w, G=cfg.G, rope_base=cfg.base)
    ws_bytes = sals.sals_decode_workspace_bytes(base["q"], base["Pk"], ctx=ctx, k=cfg.k, w=cfg.w, G=cfg.G)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.B, cfg.H_q, cfg.d), dtype=torch.float32, device="cuda")
    log(f"[{label}] {n_copies} input copies of {per_copy / 1e6:.1f} MB, workspace {ws_bytes / 1e6:.1f} MB")

    def step(i):
        c = copies[i % n_copies]
        sals.sals_decode_step(c["q"], c["Lk"], c["Lv"], c["Pk"], c["Pv"], out=out, workspace=ws, **kw)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    for row in evs:  # each event is recorded once so that its HIP event exists
        for e in row:
            e.record()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    it = iter(range(1 << 30))
    settle(lambda: step(next(it)))

    # ---- timed region: the K steps captured once as a graph, replayed between two syncs ----
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
    # spread: further timed replays of the same graph (cold: rotated inputs), and a warm graph
    # whose steps all reuse one input copy (resident in the Infinity Cache when it fits)
    rep = replay_stats(graph, steps, replays)
    warm_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(warm_graph):
        for _ in range(steps):
            step(0)
    warm_graph.replay()
    torch.cuda.synchronize()
    warm = replay_stats(warm_graph, steps, replays)
    del warm_graph

    # ---- per-kernel durations: the same K steps, eagerly, with HIP events on the launch stream ----
    # The C entry point is called with argument lists marshalled beforehand, so the host issues
    # the steps faster than the GPU runs them.
    shape = SalsShape(cfg.B, cfg.H_q, cfg.H_kv, cfg.d, cfg.r, 1 if cfg.dtype == "bf16" else 0)
    selc = SalsSelect(cfg.k, cfg.w, cfg.G)
    stream = torch.cuda.current_stream().cuda_stream
    fn = lib().sals_decode_step_traced
    calls = []
    for i in range(steps):
        c = copies[i % n_copies]
        handles = (ctypes.c_void_p * 6)(*[e.cuda_event for e in evs[i]])
        calls.append((ctypes.byref(shape), ctypes.byref(selc), ctypes.c_float(cfg.base), c["q"].data_ptr(),
                      c["Lk"].data_ptr(), c["Lv"].data_ptr(), c["Pk"].data_ptr(), c["Pv"].data_ptr(),
                      c["Lk"].shape[1], ctx, out.data_ptr(), None, ws.data_ptr(), ws_bytes, stream, handles, 6))
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    status = [fn(*a) for a in calls]
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - t_start) / steps * 1e6
    if any(status):
        raise RuntimeError(f"sals_decode_step_traced returned {set(status)}")
    stage_us = {name: sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)) / steps * 1e3
                for j, name in enumerate(stages_of(cfg))}
    event_step_us = sum(evs[i][0].elapsed_time(evs[i][5]) for i in range(steps)) / steps * 1e3
    del graph, copies
    torch.cuda.empty_cache()
    comp = run_comparators(cfg, base, ctx, steps, warmup) if cfg.dtype == "bf16" and comparators else None
    thr = run_threshold(cfg, base, ctx, steps, warmup) if cfg.dtype == "bf16" and comparators else None
    return dict(case=case, us=us_step, stage_us=stage_us, event_step_us=event_step_us, eager_us=eager_us,
                comparators=comp, replays=rep, warm=warm, threshold=thr)


def replay_stats(graph, steps, replays):
    """Median, p10 and p90 of the per-step time over `replays` timed replays of a captured graph
    of `steps` steps (each replay between two device synchronisations)."""
    import numpy as np
    import torch

    per = []
    for _ in range(replays):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        per.append((time.perf_counter() - t0) / steps * 1e6)
    return dict(median=round(float(np.median(per)), 2), p10=round(float(np.percentile(per, 10)), 2),
                p90=round(float(np.percentile(per, 90)), 2), replays=replays)


def run_threshold(cfg, base, ctx, steps, warmup):
    """sals_decode_step_threshold on the same layer, with tau set (by bisection on the kernels' own
    per-row counts) so that the rows keep about half of the top-k capacity on average; timed as
    `steps` back-to-back calls between two HIP events."""
    import torch

    import kv_cache_compression_sals_amd as sals

    q, Lk, Lv, Pk, Pv = (base[n] for n in ("q", "Lk", "Lv", "Pk", "Pv"))
    kw = dict(ctx=ctx, k=cfg.k, w=cfg.w, G=cfg.G, rope_base=cfg.base)
    wc = min(cfg.w, ctx)
    out = torch.empty((cfg.B, cfg.H_q, cfg.d), dtype=torch.float32, device="cuda")
    cnt = torch.empty((cfg.B, cfg.G), dtype=torch.int32, device="cuda")
    ws = torch.empty(sals.sals_decode_workspace_bytes(q, Pk, ctx=ctx, k=cfg.k, w=cfg.w, G=cfg.G), dtype=torch.uint8,
                     device="cuda")

    def mean_kept(tau):
        sals.sals_decode_step_threshold(q, Lk, Lv, Pk, Pv, tau=tau, out=out, n_sel_out=cnt, workspace=ws, **kw)
        return float((cnt.float() - wc).mean().item())

    lo, hi = -1e4, 1e4
    for _ in range(40):
        mid = (lo + hi) / 2
        if mean_kept(mid) > cfg.k / 2:
            lo = mid
        else:
            hi = mid
    tau = (lo + hi) / 2
    kept = mean_kept(tau)
    call = lambda: sals.sals_decode_step_threshold(q, Lk, Lv, Pk, Pv, tau=tau, out=out, n_sel_out=cnt,  # noqa: E731
                                                   workspace=ws, **kw)
    for _ in range(warmup):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    return dict(us_per_step=round(e0.elapsed_time(e1) / steps * 1e3, 2), tau=round(tau, 4),
                mean_kept_candidates=round(kept, 1), capacity=cfg.k,
                note="threshold selection, eager calls between HIP events (not a captured graph)")


def run_comparators(cfg, base, ctx, steps, warmup):
    """The dense baselines on the same layer: (a) sals_dense_decode over the whole post-RoPE bf16
    KV cache (flash-decode, split over the context); (b) the full rebuild the selection avoids,
    sals_reconstruct_kv of every token (K rotated, V, the rotated query) followed by (a). Each is
    timed as `steps` back-to-back calls between two HIP events; the rebuilt cache (2 x 268 MB at
    these shapes) is larger than the MALL, so every call reads it from HBM."""
    import torch

    import kv_cache_compression_sals_amd as sals

    q, Lk, Lv, Pk, Pv = (base[n] for n in ("q", "Lk", "Lv", "Pk", "Pv"))
    B, H_q, d = q.shape
    H_kv, r = cfg.H_kv, cfg.r
    K = torch.empty((B, H_kv, ctx, d), dtype=q.dtype, device="cuda")
    V, q_rot = torch.empty_like(K), torch.empty_like(q)
    out = torch.empty((B, H_q, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(sals.sals_dense_decode_workspace_bytes(q_rot, K, n=ctx), dtype=torch.uint8, device="cuda")
    rebuild = lambda: sals.sals_reconstruct_kv(Lk, Pk, K, t0=0, T=ctx, d=d, rope_base=cfg.base, Lv=Lv, Pv=Pv,
                                               V=V, q=q, q_rot=q_rot, q_pos=ctx - 1)
    dense = lambda: sals.sals_dense_decode(q_rot, K, V, n=ctx, out=out, workspace=ws)

    def both():
        rebuild()
        dense()

    def timed(fn):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3

    rebuild_us, dense_us, naive_us = timed(rebuild), timed(dense), timed(both)
    kv_bytes = 2 * B * H_kv * ctx * d * 2
    rebuild_flops = 2 * 2 * B * ctx * r * H_kv * d
    del K, V, ws
    torch.cuda.empty_cache()
    return dict(dense_full_kv_us=round(dense_us, 2), dense_full_kv_gbps=round(kv_bytes / (dense_us * 1e-6) / 1e9, 1),
                full_rebuild_us=round(rebuild_us, 2),
                full_rebuild_tflops=round(rebuild_flops / (rebuild_us * 1e-6) / 1e12, 1),
                full_rebuild_then_dense_us=round(naive_us, 2), kv_bytes=kv_bytes, rebuild_flops=rebuild_flops)


def run_compact_workload(cfg, steps, warmup, label):
    """The post-prefill compaction workload (B=16, 32 heads, ctx 16384, w=64, 10% kept), each call
    timed as `steps` back-to-back calls between two HIP events:
      kv_compact (and its stages, through kv_compact_traced), the dense decode over the compact
      cache, kv_compact_from_importance (a higher layer reusing this layer's importance),
      kv_importance_sparsity, kv_outlier_importance (frequency-domain importance, 32 frequencies)
      and the compaction it drives, kv_quantize_mixed + sals_dense_decode_mixed (10% of the tokens
      at 8 bits, the rest at 4), kv_importance_budget, and the dense decode over the full cache."""
    import ctypes

    import numpy as np
    import torch

    import kv_cache_compression_sals_amd as sals
    from kv_cache_compression_sals_amd._lib import KvcShape, lib
    from workloads import compact_case

    t0 = time.time()
    case = compact_case(cfg, threads=16)
    log(f"[{label}] generated inputs in {time.time() - t0:.1f}s")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    K, V, Qobs, q = (dev(case[n]) for n in ("K", "V", "Qobs", "q"))
    del case
    B, H_kv, ctx_cap, d = K.shape
    H_q, w = Qobs.shape[1], Qobs.shape[2]
    ctx, kk = cfg.ctx, cfg.k_keep
    Kc = torch.empty((B, H_kv, kk, d), dtype=K.dtype, device="cuda")
    Vc, kept = torch.empty_like(Kc), torch.empty((B, H_kv, kk), dtype=torch.int32, device="cuda")
    out = torch.empty((B, H_q, d), dtype=torch.float32, device="cuda")
    ws_c = torch.empty(sals.kv_compact_workspace_bytes(K, Qobs, ctx=ctx, k_keep=kk), dtype=torch.uint8, device="cuda")
    ws_d = torch.empty(sals.sals_dense_decode_workspace_bytes(q, Kc, n=kk), dtype=torch.uint8, device="cuda")
    ws_f = torch.empty(sals.sals_dense_decode_workspace_bytes(q, K, n=ctx), dtype=torch.uint8, device="cuda")
    imp = torch.empty((B, H_kv, ctx), dtype=torch.float32, device="cuda")
    compact = lambda: sals.kv_compact(K, V, Qobs, ctx=ctx, k_keep=kk, Kc=Kc, Vc=Vc, kept=kept, importance=imp,  # noqa: E731
                                      workspace=ws_c)
    decode = lambda: sals.sals_dense_decode(q, Kc, Vc, n=kk, out=out, workspace=ws_d)  # noqa: E731
    full = lambda: sals.sals_dense_decode(q, K, V, n=ctx, out=out, workspace=ws_f)  # noqa: E731
    reuse = lambda: sals.kv_compact_from_importance(K, V, imp, k_keep=kk, Kc=Kc, Vc=Vc, kept=kept)  # noqa: E731
    spars = torch.empty((B, H_q), dtype=torch.float32, device="cuda")
    ws_s = torch.empty(sals.kv_importance_sparsity_workspace_bytes(K, Qobs, ctx=ctx), dtype=torch.uint8,
                       device="cuda")
    sparse = lambda: sals.kv_importance_sparsity(K, Qobs, ctx=ctx, p=1e-3, importance=imp, sparsity=spars,  # noqa: E731
                                                 workspace=ws_s)
    n_freq = 32
    oimp = torch.empty_like(imp)
    ws_o = torch.empty(sals.kv_outlier_importance_workspace_bytes(K, ctx=ctx, n_freq=n_freq), dtype=torch.uint8,
                       device="cuda")
    outlier = lambda: sals.kv_outlier_importance(K, V, ctx=ctx, n_freq=n_freq, importance=oimp, workspace=ws_o)  # noqa: E731
    outlier_keep = lambda: sals.kv_compact_from_importance(K, V, oimp, k_keep=kk, Kc=Kc, Vc=Vc, kept=kept)  # noqa: E731
    mixed = {}
    quantize = lambda: sals.kv_quantize_mixed(K, V, imp, n_hi=kk, out=mixed)  # noqa: E731
    budget = lambda: sals.kv_importance_budget(imp, mass=0.9)  # noqa: E731
    settle(compact)

    def timed(fn):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3

    c_us, d_us, r_us, s_us, f_us = timed(compact), timed(decode), timed(reuse), timed(sparse), timed(full)
    o_us, ok_us = timed(outlier), timed(outlier_keep)
    q_us = timed(quantize)
    ws_m = torch.empty(sals.sals_dense_decode_mixed_workspace_bytes(q, H_kv, n_hi=kk, n_lo=ctx - kk), dtype=torch.uint8,
                       device="cuda")
    md_us = timed(lambda: sals.sals_dense_decode_mixed(q, mixed, out=out, workspace=ws_m))
    b_us = timed(budget)

    # the stages of kv_compact, from HIP events on its stream
    c = KvcShape(B, H_q, H_kv, d, 1)
    stream = torch.cuda.current_stream().cuda_stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for i in range(steps):
        handles = (ctypes.c_void_p * 5)(*[e.cuda_event for e in evs[i]])
        st = lib().kv_compact_traced(ctypes.byref(c), K.data_ptr(), V.data_ptr(), Qobs.data_ptr(), w, ctx_cap, ctx,
                                     kk, Kc.data_ptr(), Vc.data_ptr(), kept.data_ptr(), imp.data_ptr(), ws_c.data_ptr(),
                                     ws_c.numel(), stream, handles, 5)
        if st:
            raise RuntimeError(f"kv_compact_traced returned {st}")
    torch.cuda.synchronize()
    names = ["importance_stats", "importance_accum", "topk", "gather"]
    stage_us = {n: sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)) / steps * 1e3
                for j, n in enumerate(names)}
    s = 2
    k_bytes = B * H_kv * ctx * d * s
    q_bytes = Qobs.numel() * s
    stage_bytes = {"importance_stats": k_bytes + q_bytes, "importance_accum": k_bytes + q_bytes + B * H_kv * ctx * 4,
                   "topk": B * H_kv * ctx * 4 + B * H_kv * kk * 4, "gather": 4 * B * H_kv * kk * d * s}
    dom = max(stage_us, key=stage_us.get)
    achieved = stage_bytes[dom] / (stage_us[dom] * 1e-6) / 1e9
    roofline = dict(kernel=dom, bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=None, algorithmic_per_launch=stage_bytes[dom],
                    avg_launch_us=round(stage_us[dom], 2),
                    flops_per_launch=2 * B * H_q * w * ctx * d)
    # compaction: K once for the importance (its second pass is recomputation), the kept K and V
    # rows read and written once, the observation queries; decode: the compact cache once
    c_bytes = k_bytes + 4 * B * H_kv * kk * d * s + q_bytes
    d_bytes = 2 * B * H_kv * kk * d * s
    f_bytes = 2 * k_bytes
    r_bytes = B * H_kv * ctx * 4 + 4 * B * H_kv * kk * d * s
    o_bytes = 2 * k_bytes + B * H_kv * ctx * 4  # K and V once, the importance out
    n_lo = ctx - kk
    m_bytes = 2 * B * H_kv * (kk * (d + d // 32 * 8) + n_lo * (d // 2 + d // 32 * 8))  # both sets, codes + params
    qz_bytes = 2 * k_bytes + B * H_kv * ctx * 4 + m_bytes
    gbps = lambda nbytes, us: round(nbytes / (us * 1e-6) / 1e9, 1)  # noqa: E731
    del K, V, Qobs, Kc, Vc, ws_c, ws_d, ws_f, imp, ws_s, oimp, ws_o, mixed, ws_m
    torch.cuda.empty_cache()
    return dict(workload=f"{label}: B={B} H_q={H_q} H_kv={H_kv} d={d} ctx={ctx} w={w} k_keep={kk}, bf16",
                compact_us=round(c_us, 1), compact_gbps=gbps(c_bytes, c_us),
                stage_us={k: round(v, 2) for k, v in stage_us.items()}, roofline=roofline,
                decode_us=round(d_us, 2), decode_gbps=gbps(d_bytes, d_us),
                full_cache_decode_us=round(f_us, 2), full_cache_decode_gbps=gbps(f_bytes, f_us),
                from_importance_us=round(r_us, 2), from_importance_gbps=gbps(r_bytes, r_us),
                importance_sparsity_us=round(s_us, 1),
                outlier_importance_us=round(o_us, 1), outlier_importance_gbps=gbps(o_bytes, o_us),
                outlier_compact_us=round(o_us + ok_us, 1), n_freq=n_freq,
                quantize_mixed_us=round(q_us, 1), quantize_mixed_gbps=gbps(qz_bytes, q_us),
                mixed_decode_us=round(md_us, 2), mixed_decode_gbps=gbps(m_bytes, md_us),
                mixed_cache_bytes=m_bytes, bf16_cache_bytes=f_bytes,
                importance_budget_us=round(b_us, 2),
                compact_bytes=c_bytes, decode_bytes=d_bytes, from_importance_bytes=r_bytes)


def _layer_inputs(layer):
    """One layer of the 128K-context workload (NumPy releases the GIL in its bulk work, so the
    layers are generated by threads of this process: no child process ever exists)."""
    from workloads import CONFIGS, decode_case

    c = decode_case(CONFIGS["c5"], layer=layer)
    return layer, {n: c[n] for n in ("q", "Lk", "Lv", "Pk", "Pv")}


def run_layers_workload(cfg, steps, warmup, label, n_layers=32):
    """One decode step through n_layers independent layers (all resident): `steps` steps captured
    as one HIP graph, one upload replay, then one timed replay."""
    from concurrent.futures import ThreadPoolExecutor, as_completed

    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import kv_cache_compression_sals_amd as sals

    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    t0 = time.time()
    layers = [None] * n_layers
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        futs = [ex.submit(_layer_inputs, l) for l in range(n_layers)]
        for i, fut in enumerate(as_completed(futs)):
            l, arrs = fut.result()
            layers[l] = {n: dev(a) for n, a in arrs.items()}
            log(f"[{label}] layer {l} resident ({i + 1}/{n_layers}, {time.time() - t0:.0f}s)")
    log(f"[{label}] generated and uploaded {n_layers} layers in {time.time() - t0:.1f}s")
    ctx = cfg.ctx
    kw = dict(ctx=ctx, k=cfg.k, w=cfg.w, G=cfg.G, rope_base=cfg.base)
    ws = torch.empty(sals.sals_decode_workspace_bytes(layers[0]["q"], layers[0]["Pk"], ctx=ctx, k=cfg.k, w=cfg.w,
                                                      G=cfg.G), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((cfg.B, cfg.H_q, cfg.d), dtype=torch.float32, device="cuda") for _ in range(n_layers)]

    def step():
        for l, t in enumerate(layers):
            sals.sals_decode_step(t["q"], t["Lk"], t["Lv"], t["Pk"], t["Pv"], out=outs[l], workspace=ws, **kw)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    settle(step)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            step()
    graph.replay()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t_start) / steps * 1e6
    rep = replay_stats(graph, steps, 3)
    alg = algorithmic(cfg, ctx)
    del graph
    # per-stage durations: one eager pass through the layers with HIP events at the stage boundaries
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(n_layers)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for l, t in enumerate(layers):
        sals.sals_decode_step_traced(t["q"], t["Lk"], t["Lv"], t["Pk"], t["Pv"], evs[l], out=outs[l], workspace=ws,
                                     **kw)
    torch.cuda.synchronize()
    stage_us = {name: sum(evs[l][j].elapsed_time(evs[l][j + 1]) for l in range(n_layers)) / n_layers * 1e3
                for j, name in enumerate(stages_of(cfg))}
    rl, _ = roofline_for(cfg, ctx, stage_us, label)
    del layers, ws
    torch.cuda.empty_cache()
    return dict(workload=f"{label}: {n_layers} layers, B={cfg.B} H_q={cfg.H_q} H_kv={cfg.H_kv} d={cfg.d} "
                         f"ctx={ctx} r={cfg.r} k={cfg.k} w={cfg.w} G={cfg.G}",
                us_per_step=round(us, 1), us_per_layer=round(us / n_layers, 2), us_per_step_stats=rep,
                kv_gbps=round(n_layers * alg["compulsory"] / (us * 1e-6) / 1e9, 1),
                hbm_frac=round(n_layers * alg["compulsory"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                compulsory_bytes_per_step=n_layers * alg["compulsory"],
                stage_us_per_layer={k: round(v, 2) for k, v in stage_us.items()}, roofline=rl)


def measure_hbm(gib=2):
    """HBM read bandwidth of the in-tree streaming kernel (sals_hbm_read) over a buffer of `gib`
    GiB, for 2048, 4096 and 8192 workgroups: the best of five timed reads each."""
    import torch

    from kv_cache_compression_sals_amd._lib import lib

    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(7)
    sink = torch.empty(8192, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    best = 0.0
    for blocks in (2048, 4096, 8192):
        for _ in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            st = lib().sals_hbm_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, stream)
            e1.record()
            torch.cuda.synchronize()
            if st:
                raise RuntimeError(f"sals_hbm_read returned {st}")
            best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf
    torch.cuda.empty_cache()
    return round(best, 1)


def measure_mfma():
    """bf16 MFMA throughput of the in-tree register-only MFMA loop (sals_mfma_peak): 1024, 2048 and
    4096 workgroups of 4 waves, each wave 4 independent 32x32x16 accumulators over 1500 steps; the
    best of five timed launches each, in TFLOP/s."""
    import torch

    from kv_cache_compression_sals_amd._lib import lib

    iters = 1500
    sink = torch.empty(4096, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    best = 0.0
    for blocks in (1024, 2048, 4096):
        for _ in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            st = lib().sals_mfma_peak(blocks, iters, sink.data_ptr(), stream)
            e1.record()
            torch.cuda.synchronize()
            if st:
                raise RuntimeError(f"sals_mfma_peak returned {st}")
            flops = blocks * 4 * iters * 4 * 32768
            best = max(best, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return round(best, 1)


def with_measured(rl, hbm_measured=None, mfma_measured=None):
    """The roofline object with its fraction of the peak measured on this machine (frac_measured)."""
    peak = mfma_measured if rl["bound"] == "mfma" else hbm_measured
    if peak:
        rl = dict(rl, peak_measured=peak, frac_measured=round(rl["achieved"] / peak, 4))
    return rl


def roofline_for(cfg, ctx, stage_us, label):
    """Roofline of the kernel that takes the most time: bound by HBM or by bf16 MFMA, whichever
    peak gives the longer time for its algorithmic bytes / flops."""
    alg = algorithmic(cfg, ctx)
    dom = max(stage_us, key=stage_us.get)
    t = stage_us[dom] * 1e-6
    nbytes, nflops = alg["stage_bytes"][dom], alg["stage_flops"][dom]
    t_hbm = nbytes / (HBM_PEAK_GBPS * 1e9)
    t_mfma = nflops / (BF16_MFMA_PEAK_TFLOPS * 1e12)
    traffic = stored_traffic(dom, label)
    if t_mfma > t_hbm:
        achieved = nflops / t / 1e12
        rl = dict(kernel=dom, bound="mfma", achieved=round(achieved, 2), peak=BF16_MFMA_PEAK_TFLOPS,
                  unit="TFLOP/s", frac=round(achieved / BF16_MFMA_PEAK_TFLOPS, 4), traffic=traffic,
                  algorithmic_per_launch=nflops, avg_launch_us=round(stage_us[dom], 2))
    else:
        achieved = nbytes / t / 1e9
        rl = dict(kernel=dom, bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                  frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=traffic,
                  algorithmic_per_launch=nbytes, avg_launch_us=round(stage_us[dom], 2))
    return rl, alg


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_step(case):
    import oracle

    oracle.decode_step(case["q"], case["Lk"], case["Lv"], case["Pk"], case["Pv"], ctx=case["ctx"], k=case["k"],
                       w=case["w"], G=case["G"], H_kv=case["H_kv"], base=case["base"], dtype=case["dtype"])


def cpu_baseline(case, budget_s=10.0, tiny=None):
    """The oracle (fp64 NumPy, as it stands) on the same stored inputs: whole decode steps of the
    workload (all sequences, all heads), repeated until about budget_s of CPU time has passed;
    the mean step time is reported, with every BLAS thread of the process. Beside it: one step
    with a single thread, and the tiny fp32 workload's step (median of 5) with all threads and
    with one."""
    from threadpoolctl import threadpool_info, threadpool_limits

    try:
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = 1
    n, t0 = 0, time.perf_counter()
    while n == 0 or time.perf_counter() - t0 < budget_s:
        _oracle_step(case)
        n += 1
    per_step = (time.perf_counter() - t0) / n
    one = {}
    with threadpool_limits(1):
        t1 = time.perf_counter()
        _oracle_step(case)
        one["headline_us"] = round((time.perf_counter() - t1) * 1e6, 1)
    if tiny is not None:
        def med5():
            ts = []
            for _ in range(5):
                t1 = time.perf_counter()
                _oracle_step(tiny)
                ts.append(time.perf_counter() - t1)
            return round(sorted(ts)[2] * 1e6, 1)
        tiny_all = med5()
        with threadpool_limits(1):
            one["tiny_us"] = med5()
    out = dict(value=round(per_step * 1e6, 1), unit="us/decode_step", cores=cores, kind="oracle",
               sample=f"{n} whole oracle decode steps of the same workload (all {case['B']} sequences, "
                      f"all heads), mean, {n * per_step:.1f} s in total", cpu_model=cpu_model(),
               one_thread=one)
    if tiny is not None:
        out["tiny_us"] = tiny_all
    return out


def summary(cfg, r, label, hbm_measured=None, mfma_measured=None):
    rl, alg = roofline_for(cfg, r["case"]["ctx"], r["stage_us"], label)
    rl = with_measured(rl, hbm_measured, mfma_measured)
    gbps = alg["compulsory"] / (r["us"] * 1e-6) / 1e9
    # scoring + attention: the latent scan and the rebuild/attention stages (the value kernels, or
    # the split merge that applies P_v) over their summed time
    sa = ("latent_score", "select_attend") + (("value",) if "value" in r["stage_us"] else ("combine",))
    sa_bytes = sum(alg["stage_bytes"][k] for k in sa)
    sa_us = sum(r["stage_us"][k] for k in sa)
    return dict(
        us_per_step=round(r["us"], 2),
        us_per_step_stats=r["replays"],
        warm_us_per_step=r["warm"]["median"],
        kv_gbps=round(gbps, 1),
        hbm_frac=round(gbps / HBM_PEAK_GBPS, 4),
        hbm_frac_measured=round(gbps / hbm_measured, 4) if hbm_measured else None,
        scoring_attention_gbps=round(sa_bytes / (sa_us * 1e-6) / 1e9, 1),
        scoring_attention_hbm_frac=round(sa_bytes / (sa_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        eager_us_per_step=round(r["eager_us"], 2),
        event_us_per_step=round(r["event_step_us"], 2),
        stage_us={k: round(v, 2) for k, v in r["stage_us"].items()},
        k_rebuild_tflops=round(alg["k_rebuild_flops"] / (r["stage_us"]["select_attend"] * 1e-6) / 1e12, 1),
        compulsory_bytes=alg["compulsory"],
        roofline=rl,
    ) | ({} if not r.get("threshold") else dict(threshold=r["threshold"])) | (
        {} if not r.get("comparators") else dict(comparators=dict(
        r["comparators"],
        speedup_vs_dense_full_kv=round(r["comparators"]["dense_full_kv_us"] / r["us"], 2),
        speedup_vs_full_rebuild=round(r["comparators"]["full_rebuild_then_dense_us"] / r["us"], 2))))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--replays", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-hbm-probe", action="store_true")
    ap.add_argument("--only", default="c1,c2,c3,c4,c5")
    ap.add_argument("--calib-copy-mib", type=int, default=0)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures the single-GPU decode path only; --gpus must be 1. The method is "
              "independent per sequence and would shard by batch with no exchange.", file=sys.stderr)
        sys.exit(2)
    import torch

    from workloads import CONFIGS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calib_copy_mib > 0:
        a = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"[calib] copied {args.calib_copy_mib} MiB")
        del a, b
    hbm = mfma = None
    if not args.no_hbm_probe:
        hbm = measure_hbm()
        log(f"[hbm] streaming read {hbm:.0f} GB/s")
        mfma = measure_mfma()
        log(f"[mfma] bf16 MFMA loop {mfma:.0f} TFLOP/s")

    labels = {"c1": "ctx512_tiny", "c2": "ctx4k", "c3": "ctx32k", "c4": "compact_ctx16k", "c5": "ctx128k_32layers"}
    keys = [k for k in args.only.split(",") if k]
    extra = {}
    for key in [k for k in keys if k in ("c4", "c5")]:
        fn = run_compact_workload if key == "c4" else run_layers_workload
        extra[labels[key]] = fn(CONFIGS[key], min(args.steps, 10), min(args.warmup, 2), labels[key])
        extra[labels[key]]["roofline"] = with_measured(extra[labels[key]]["roofline"], hbm, mfma)
        log(f"[{labels[key]}] {extra[labels[key]]}")
    tiny = None
    if "c1" in keys:
        cfg = CONFIGS["c1"]
        r = run_workload(cfg, args.steps, args.warmup, labels["c1"], args.replays, comparators=False)
        sm = summary(cfg, r, labels["c1"], hbm, mfma)
        extra[labels["c1"]] = dict(workload=f"{labels['c1']} decode, one layer: B={cfg.B} H_q={cfg.H_q} "
                                            f"H_kv={cfg.H_kv} d={cfg.d} ctx={cfg.ctx} r={cfg.r} k={cfg.k} w={cfg.w} "
                                            f"G={cfg.G}, fp32 (latency-bound)",
                                   us_per_step=sm["us_per_step"], us_per_step_stats=sm["us_per_step_stats"],
                                   warm_us_per_step=sm["warm_us_per_step"], stage_us=sm["stage_us"])
        tiny = r["case"]
        log(f"[{labels['c1']}] {sm['us_per_step']:.1f} us/step")
    keys = [k for k in keys if k in ("c2", "c3")]
    if not keys:
        print("--only must name c2 or c3 (the step the JSON line's value reports)", file=sys.stderr)
        sys.exit(2)
    res = {}
    for key in keys:
        cfg = CONFIGS[key]
        r = run_workload(cfg, args.steps, args.warmup, labels[key], args.replays)
        res[key] = (cfg, r, summary(cfg, r, labels[key], hbm, mfma))
        sm = res[key][2]
        log(f"[{labels[key]}] {sm['us_per_step']:.1f} us/step (eager traced {sm['eager_us_per_step']:.1f}), "
            f"{sm['kv_gbps']:.0f} GB/s effective, stages "
            + ", ".join(f"{k}={v:.1f}" for k, v in sm["stage_us"].items()))

    head = keys[0]
    cfg, r, sm = res[head]
    line = {
        "metric": "us/decode step + effective KV GB/s (% HBM peak) at 4K and 32K ctx, 1 GPU",
        "value": sm["us_per_step"],
        "unit": "us/decode_step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sm["us_per_step"] / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{labels[head]} decode, one layer: B={cfg.B} H_q={cfg.H_q} H_kv={cfg.H_kv} d={cfg.d} "
                        f"ctx={cfg.ctx} r={cfg.r} k={cfg.k} w={cfg.w} G={cfg.G}",
        },
        "hbm_measured_gbps": hbm,
        "mfma_measured_tflops": mfma,
    }
    line.update({k: v for k, v in sm.items() if k != "us_per_step"})
    for key in keys[1:]:
        c, _, s = res[key]
        line[labels[key]] = dict(workload=f"{labels[key]} decode, one layer: B={c.B} H_q={c.H_q} "
                                          f"H_kv={c.H_kv} d={c.d} ctx={c.ctx} r={c.r} k={c.k} w={c.w} G={c.G}",
                                 **s)
    line.update(extra)
    if not args.no_cpu_baseline:
        log(f"[cpu] timing the oracle on a bounded sample of the {labels[head]} workload")
        line["cpu_baseline"] = cpu_baseline(r["case"], tiny=tiny)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
