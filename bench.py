#!/usr/bin/env python3
"""Throughput of observation-window KV selection on one MI355X.

One step = the whole selection path (window logits, causal row statistics,
votes, pooling, top-(C-W), window append, K/V gather) over one batch of the
workload; for the default workload that is 32 layer calls, each over the
layer's 32 heads at L = 32768, W = 32, C = 1024, D = 128, bf16, max pooling
of width 5, with 1% of prefix keys planted near the window queries' mean.
Inputs are resident in HBM before the timed region starts; every layer has
its own K and V, so consecutive calls stream fresh data.

Prints one JSON line.  value = prompt tokens scored per second
= L * layers * steps / elapsed (a token counts once per layer, over all of
that layer's heads).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prompt tokens scored/s and HBM GB/s (% of peak), 32 heads, L=32768, D=128"
HBM_PEAK_GBPS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_alg_bytes(name, w, nch, lse=False, group=1):
    """Algorithmic bytes one launch of a kernel moves for one layer call
    (lse: the row statistics are handed over, so only the prefix keys, Qwin
    and the W log-sum-exps per head are read for the votes; group: query
    heads per K/V head, whose K is read once for the whole group)."""
    e = 2 if w.dtype == "bf16" else 4
    H, L, W, C, D = w.heads, w.L, w.W, w.C, w.D
    P = L - W
    q = H * W * D * e
    if group > 1:
        Hkv = H // group
        if name == "window_stats":      # K of every K/V head once, Qwin, partials
            return Hkv * L * D * e + q + H * nch * W * 8
        if name == "window_votes":      # prefix K of every K/V head, Qwin, partials (or lse), votes out
            return Hkv * P * D * e + q + (H * W * 4 if lse else H * nch * W * 8) + H * P * 4
    if lse and name in ("window_fused", "window_votes"):
        return H * P * D * e + q + H * W * 4 + H * P * 4
    if name == "window_fused":      # K once, Qwin, votes out (partials are noise)
        return H * L * D * e + q + H * P * 4
    if name == "window_stats":      # K once, Qwin, partial (max, sum) per chunk
        return H * L * D * e + q + H * nch * W * 8
    if name == "window_votes":      # prefix K, Qwin, partials, votes out
        return H * P * D * e + q + H * nch * W * 8 + H * P * 4
    if name == "pool":              # votes in, pooled out
        return H * P * 8
    if name == "candidates":        # pooled scores read once (the histogram reads hit L2)
        return H * P * 4
    if name == "threshold":         # histograms, segment counts (the candidates: data-dependent, few)
        return H * 2048 * 4 + H * 2 * 512 * 4
    if name == "emit":              # pooled scores, kept K and V rows read and written, indices
        return H * P * 4 + 4 * H * C * D * e + H * C * 4
    if name == "select":            # votes read, indices written, kept K and V rows read and written
        return H * P * 4 + H * C * 4 + 4 * H * C * D * e
    return None                     # fill: workspace clearing, not the method's traffic


def path_alg_bytes(w, group=1):
    """Minimum bytes of the whole path per layer call: K of every K/V head
    once, Qwin, the kept K/V rows read and written, the indices."""
    e = 2 if w.dtype == "bf16" else 4
    return (w.heads // group) * w.L * w.D * e + w.heads * (w.W * w.D * e + 4 * w.C * w.D * e + 4 * w.C)


# Sources each kernel is compiled from: stored counter bytes stay valid while
# these files are unchanged.
KERNEL_SOURCES = {
    "window_fused": ("kvsel_fused.hip", "kvsel_internal.h"),
    "window_fused_lse": ("kvsel_fused.hip", "kvsel_internal.h"),
    "fill": ("kvsel_fused.hip", "kvsel_internal.h"),
    "window_stats": ("kvsel_score.hip", "kvsel_internal.h"),
    "window_votes": ("kvsel_score.hip", "kvsel_internal.h"),
    "pool": ("kvsel_select.hip", "kvsel_internal.h"),
    "candidates": ("kvsel_select.hip", "kvsel_internal.h"),
    "threshold": ("kvsel_select.hip", "kvsel_internal.h"),
    "emit": ("kvsel_select.hip", "kvsel_internal.h"),
    "gather": ("kvsel_select.hip", "kvsel_internal.h"),
    "select": ("kvsel_select.hip", "kvsel_internal.h"),
    "jacap_logits": ("kvsel_jacap.hip", "kvsel_jacap.h", "kvsel_internal.h"),
    "jacap_weights": ("kvsel_jacap.hip", "kvsel_jacap.h", "kvsel_internal.h"),
    "jacap_gram": ("kvsel_jacap.hip", "kvsel_jacap.h", "kvsel_internal.h"),
    "jacap_reduce": ("kvsel_jacap.hip", "kvsel_jacap.h", "kvsel_internal.h"),
    "jacap_factor": ("kvsel_jacap.hip", "kvsel_jacap.h", "kvsel_internal.h"),
    "jacap_leverage": ("kvsel_jacap.hip", "kvsel_jacap.h", "kvsel_internal.h"),
}


def source_digest(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "prompt_kv_selection_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel):
    """Counter-measured HBM bytes per launch, if the stored counters were
    taken on the kernel's current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get("kernels", {}).get(kernel)
    if not ent or kernel not in KERNEL_SOURCES or ent.get("source_digest") != source_digest(kernel):
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(w, seconds):
    """The CPU oracle on a bounded sample of the same workload: heads of
    layer 0 (then layer 1, ...) in a thread pool, until `seconds` of wall time
    have passed after a full round."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    from oracle import snapkv_oracle as O
    from prompt_kv_selection_amd import workloads as WL

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    jobs = [(l, h) for l in range(w.layers) for h in range(w.heads)]
    inputs = {}

    def prepare(job):
        q, k, v = WL.head_arrays(w, job[1], layer=job[0])
        return job, (WL.to_float64(q, w.dtype), WL.to_float64(k, w.dtype), WL.to_float64(v, w.dtype))

    def run(job):
        q, k, v = inputs.pop(job)
        O.snapkv_select(q, k, v, w.W, w.C, w.kernel, w.pooling)

    done = 0
    elapsed = 0.0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while done < len(jobs) and elapsed < seconds:
            batch = jobs[done:done + threads]
            inputs.update(dict(ex.map(prepare, batch)))     # input drawing is not timed
            t0 = time.perf_counter()
            list(ex.map(run, batch))
            elapsed += time.perf_counter() - t0
            done += len(batch)
    tokens = w.L * done / w.heads
    return {"value": tokens / elapsed, "unit": "prompt tokens scored/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} heads (layer-major) of the same workload, {elapsed:.1f} s of oracle time; "
                      f"value = L * heads_done / heads_per_layer / time"}


def refresh_bench(args, B, torch, np):
    """The refresh selection of a cache of J kept plus h recent tokens per
    head (h = J / 4), 32 heads per call, one call per layer, with a protected
    head (sinks) and tail (recent window); scores, K, V and token ids are
    synthetic and resident in HBM."""
    J, h = args.refresh, args.refresh // 4
    n, rows, layers, D = J + h, 32, args.layers or 32, 128
    head, tail = 4, 64
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(7)
    S = [(torch.rand((rows, n), generator=g) * 4).cuda() for _ in range(layers)]
    K = [torch.randn((rows, n, D), generator=g).to(torch.bfloat16).cuda() for _ in range(layers)]
    V = [torch.randn((rows, n, D), generator=g).to(torch.bfloat16).cuda() for _ in range(layers)]
    T = [torch.randint(0, 1 << 30, (rows, n), generator=g, dtype=torch.int32).cuda() for _ in range(layers)]
    idx = [torch.empty((rows, J), dtype=torch.int32, device=dev) for _ in range(layers)]
    Ko = [torch.empty((rows, J, D), dtype=torch.bfloat16, device=dev) for _ in range(layers)]
    Vo = [torch.empty_like(Ko[0]) for _ in range(layers)]
    To = [torch.empty((rows, J), dtype=torch.int32, device=dev) for _ in range(layers)]
    ws = torch.empty(B.kvsel_refresh_workspace_bytes(rows, n), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        for l in range(layers):
            B.kvsel_refresh(S[l], rows, n, J, head, tail, K[l], V[l], D, torch.bfloat16, T[l], idx[l], Ko[l], Vo[l],
                            To[l], ws, stream=stream)

    for _ in range(args.warmup):
        step()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    B.kvsel_profile_enable(True)
    step()
    torch.cuda.synchronize()
    per_kernel = B.kvsel_profile_read()
    B.kvsel_profile_enable(False)
    moved = rows * (n * 4 + J * 4 * 2 + 4 * J * D * 2 + 2 * J * 4)  # scores, indices, K/V read and written, tokens
    print(json.dumps({
        "metric": "refresh selection: cached tokens scored/s (32 heads per call)",
        "value": round(rows * n * layers / (ms / 1e3), 1), "unit": "cached tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"refresh_J{J}_h{h}_h32", "layers": layers, "J": J, "h": h, "protect_head": head,
                   "protect_tail": tail, "D": D},
        "path": {"alg_bytes_per_call": moved, "alg_GBps": round(moved * layers / (ms / 1e3) / 1e9, 1)},
        "kernels": {k: {"launches": c, "avg_us": round(t / c * 1e3, 2)} for k, (c, t) in per_kernel.items()},
    }), flush=True)


def jacap_alg(name, H, N, D, S):
    """(bytes, flops) one launch of a Jacap kernel moves and computes for H
    heads of N cached tokens (S Gram slices per head); flops count each
    product of the two N D^2 contractions once (the bf16 high/low split
    issues 3 and 2 times as many)."""
    e = 2
    if name == "jacap_logits":      # K once, z and kappa out, mu and lambda
        return H * N * D * e + H * N * 8 + H * D * 8, 0
    if name == "jacap_weights":     # z and kappa in, w out
        return H * N * 12, 0
    if name == "jacap_gram":        # U once, w, the slices' D x D parts out
        return H * N * D * e + H * N * 4 + H * S * D * D * 4, 2 * H * N * D * D
    if name == "jacap_reduce":      # the slices' lower tiles in, their sum out
        return (S + 1) * H * D * D * 4 * 10 // 16, (S - 1) * H * D * D * 10 // 16
    if name == "jacap_factor":      # the summed Gram matrix in, L^-1 (high, low) out
        return H * D * D * 4 + H * D * D * 4, H * D ** 3 // 3 * 2
    if name == "jacap_leverage":    # U once, w in, r out, L^-1
        return H * N * D * e + H * N * 8 + H * D * D * 4, 2 * H * N * D * D
    return None, None


def jacap_bench(args, B, torch, np):
    """One Jacap eviction event per layer (kvsel_jacap_select): 32 heads of N
    cached tokens, D = 128, bf16, U = V (the page's cheaper proxy for W_O v),
    tau = 10, keep = N / 5 (compression 0.8), 4 sink and 64 recent tokens
    protected.  K, V ~ N(0, 1), mu_q ~ N(0, 1), lambda_q ~ U[0.1, 2), drawn on
    the device from a seeded generator; every layer has its own K and V."""
    N, H, D, layers = args.jacap, 32, 128, args.layers or 32
    keep, head, tail, tau = N // 5, 4, 64, 10.0
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(17)
    K = [torch.randn((H, N, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(layers)]
    V = [torch.randn((H, N, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(layers)]
    mu = [torch.randn((H, D), generator=g, device=dev) for _ in range(layers)]
    lam = [torch.rand((H, D), generator=g, device=dev) * 1.9 + 0.1 for _ in range(layers)]
    idx = [torch.empty((H, keep), dtype=torch.int32, device=dev) for _ in range(layers)]
    Ko = [torch.empty((H, keep, D), dtype=torch.bfloat16, device=dev) for _ in range(layers)]
    Vo = [torch.empty_like(Ko[0]) for _ in range(layers)]
    nst = max(1, args.streams)
    ws = [torch.empty(B.kvsel_jacap_workspace_bytes(H, N, D), dtype=torch.uint8, device=dev) for _ in range(nst)]
    stream = torch.cuda.current_stream()
    side = [stream] + [torch.cuda.Stream(device=dev) for _ in range(nst - 1)]  # default priority
    fork = [torch.cuda.Event() for _ in range(nst)]
    torch.cuda.synchronize()

    def step():
        # Layer l goes to stream l % nst (its own workspace); the side streams
        # start after the step's start on the timing stream and end before its end.
        if nst > 1:
            fork[0].record(stream)
            for k in range(1, nst):
                side[k].wait_event(fork[0])
        for l in range(layers):
            k = l % nst
            B.kvsel_jacap_select(K[l], V[l], V[l], mu[l], lam[l], tau, H, N, D, "bf16", keep, head, tail, None,
                                 idx[l], Ko[l], Vo[l], None, None, ws[k], stream=side[k])
        for k in range(1, nst):
            fork[k].record(side[k])
            stream.wait_event(fork[k])

    for _ in range(args.warmup):
        step()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    for k in range(nst):  # the last timed calls' device-side outcome
        if B.kvsel_status(ws[k], side[k]) != B.KVSEL_OK:
            raise SystemExit("Jacap event reported a device-side error: " + B.kvsel_last_error())
    B.kvsel_profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    per_kernel = B.kvsel_profile_read()
    B.kvsel_profile_enable(False)
    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("copy probe: 1 GiB device-to-device copy done")
    S = max(1, min(32, (256 + H - 1) // H, (N + 511) // 512))
    kern = {}
    for k, (c, t) in per_kernel.items():
        avg = t / c / 1e3
        ab, fl = jacap_alg(k, H, N, D, S)
        kern[k] = {"launches": c, "avg_us": round(avg * 1e6, 2),
                   "alg_GBps": None if ab is None else round(ab / avg / 1e9, 1),
                   "alg_TFLOPs": None if not fl else round(fl / avg / 1e12, 2)}
    dom = max((k for k in per_kernel if jacap_alg(k, H, N, D, S)[0] is not None), key=lambda k: per_kernel[k][1])
    c, t = per_kernel[dom]
    achieved = jacap_alg(dom, H, N, D, S)[0] / (t / c / 1e3) / 1e9
    moved = H * N * D * 2 * 3 + 4 * H * keep * D * 2 + H * keep * 4  # K once, U twice, kept rows, indices
    print(json.dumps({
        "metric": f"Jacap eviction event: cached tokens scored/s (32 heads, N={N}, D=128)",
        "value": round(H * N * layers / (ms / 1e3), 1), "unit": "cached tokens/s (all heads)", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"jacap_h32_n{N}_d128", "layers": layers, "N": N, "keep": keep,
                   "protect_head": head, "protect_tail": tail, "tau": tau, "u": "v", "streams": nst},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profiles(dom) if N == 32768 else None},
        "path": {"alg_bytes_per_call": moved, "alg_GBps": round(moved * layers / (ms / 1e3) / 1e9, 1),
                 "us_per_call": round(ms * 1e3 / layers, 2)},
        "kernels": kern,
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="spike_l32x_h32_l32k")
    ap.add_argument("--layers", type=int, default=0, help="layers per step (default: the workload's)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--scoring", choices=("auto", "two_pass", "single_read"), default="auto",
                    help="scoring path (auto: single-read wherever it applies)")
    ap.add_argument("--lse", action="store_true",
                    help="row statistics handed over (kvsel_select_lse), as prefill attention would; each "
                         "layer's log-sum-exps come from one untimed call of the full path")
    ap.add_argument("--gqa", type=int, default=1,
                    help="query heads per K/V head: the layer's K/V has heads / GQA heads, each streamed once for "
                         "its group (kvsel_select_gqa)")
    ap.add_argument("--refresh", type=int, default=0,
                    help="time the refresh selection instead: J kept of J + J/4 cached tokens per head")
    ap.add_argument("--jacap", type=int, default=0,
                    help="time the Jacap eviction event instead: 32 heads of N cached tokens per layer call")
    ap.add_argument("--streams", type=int, default=1,
                    help="with --jacap: independent layer calls spread over this many streams (own workspaces)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one 1 GiB device copy (reference for HBM counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: this build measures one GPU's share "
              f"(--gpus {args.gpus} requested); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from prompt_kv_selection_amd import binding as B
    from prompt_kv_selection_amd import workloads as WL

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a HIP device")
    if args.refresh:
        refresh_bench(args, B, torch, np)
        return
    if args.jacap:
        jacap_bench(args, B, torch, np)
        return
    w = WL.get(args.workload)
    if w.ragged:
        raise SystemExit("bench.py times single-length workloads")
    layers = args.layers or w.layers
    dev = torch.device("cuda:0")
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    H, L, W, C, D = w.heads, w.L, w.W, w.C, w.D

    log(f"drawing {layers} layer(s) of {w.name}")
    t0 = time.time()
    G = args.gqa
    if G < 1 or H % G:
        raise SystemExit(f"--gqa must divide the {H} heads")
    Hkv = H // G
    Qs, Ks, Vs = [], [], []
    for layer in range(layers):
        if G > 1:  # K/V of the K/V heads only; Qwin of every query head
            _, K, V = WL.layer_arrays(w, layer=layer, heads=range(Hkv))
            Q, _, _ = WL.layer_arrays(WL.reduced(w, L=W, C=W + 1), layer=layer)
        else:
            Q, K, V = WL.layer_arrays(w, layer=layer)
        conv = (lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)) if w.dtype == "bf16" else \
            (lambda a: torch.from_numpy(a))
        Qs.append(conv(Q).to(dev))
        Ks.append(conv(K).to(dev))
        Vs.append(conv(V).to(dev))
        del Q, K, V
    torch.cuda.synchronize()
    log(f"inputs resident in HBM after {time.time() - t0:.1f} s")

    ws_bytes = B.kvsel_gqa_workspace_bytes(H, Hkv, L, W, C, D, td)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    idx = [torch.empty((H, C), dtype=torch.int32, device=dev) for _ in range(layers)]
    Ko = [torch.empty((H, C, D), dtype=td, device=dev) for _ in range(layers)]
    Vo = [torch.empty((H, C, D), dtype=td, device=dev) for _ in range(layers)]
    stream = torch.cuda.current_stream()
    B.kvsel_set_option(B.KVSEL_OPT_SCORING, B.SCORING[args.scoring])

    lses = []
    if args.lse:
        rs = torch.empty((H, W, 2), dtype=torch.float32, device=dev)
        for layer in range(layers):
            B.kvsel_select_gqa(Qs[layer], Ks[layer], Vs[layer], None, L, W, C, D, H, Hkv, w.kernel, w.pooling, td,
                               idx[layer], Ko[layer], Vo[layer], rs, None, None, ws, stream=stream)
            lses.append((rs[:, :, 0].double() + rs[:, :, 1].double().log()).float().contiguous())
        torch.cuda.synchronize()
        log("row log-sum-exps of every layer ready")

    def step():
        for layer in range(layers):
            if G > 1:
                B.kvsel_select_gqa(Qs[layer], Ks[layer], Vs[layer], lses[layer] if args.lse else None, L, W, C, D, H,
                                   Hkv, w.kernel, w.pooling, td, idx[layer], Ko[layer], Vo[layer], None, None, None,
                                   ws, stream=stream)
            elif args.lse:
                B.kvsel_select_lse(Qs[layer], Ks[layer], Vs[layer], lses[layer], L, W, C, D, H, w.kernel,
                                   w.pooling, td, idx[layer], Ko[layer], Vo[layer], None, None, ws, stream=stream)
            else:
                B.kvsel_select(Qs[layer], Ks[layer], Vs[layer], L, W, C, D, H, w.kernel, w.pooling, td,
                               idx[layer], Ko[layer], Vo[layer], None, None, None, ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps bracketed by synchronisation, no instrumentation.
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)

    # The same K steps again with every kernel bracketed by HIP events on its
    # launch stream: per-kernel durations for the roofline.
    B.kvsel_profile_enable(True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_events = start.elapsed_time(stop)
    per_kernel = B.kvsel_profile_read()
    B.kvsel_profile_enable(False)

    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("copy probe: 1 GiB device-to-device copy done")

    ms_step = ms_total / args.steps
    tokens_per_s = L * layers * args.steps / (ms_total / 1e3)
    nch = (L + 1023) // 1024
    kern = {}
    for name, (n, ms) in per_kernel.items():
        ab = kernel_alg_bytes(name, w, nch, args.lse, G)
        avg = ms / n
        kern[name] = {"launches": n, "avg_us": round(avg * 1e3, 2),
                      "alg_GBps": None if ab is None else round(ab / (avg / 1e3) / 1e9, 1)}
    dom = max((k for k in per_kernel if kernel_alg_bytes(k, w, nch) is not None), key=lambda k: per_kernel[k][1])
    n_dom, ms_dom = per_kernel[dom]
    ab_dom = kernel_alg_bytes(dom, w, nch, args.lse, G)
    achieved = ab_dom / (ms_dom / n_dom / 1e3) / 1e9
    traffic = None if G > 1 else traffic_from_profiles(dom + "_lse" if args.lse else dom)
    path_gbps = path_alg_bytes(w, G) * layers / (ms_step / 1e3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "prompt tokens scored/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "layers": layers, "heads": H, "L": L, "W": W, "C": C, "D": D,
                   "pooling": w.pooling, "kernel": w.kernel, "keys": w.keys,
                   "scoring": args.scoring, "row_stats": "handed_over" if args.lse else "computed",
                   "kv_heads": Hkv},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic},
        "path": {"alg_bytes_per_layer": path_alg_bytes(w, G), "alg_GBps": round(path_gbps, 1),
                 "frac_of_peak": round(path_gbps / HBM_PEAK_GBPS, 4),
                 "ms_per_step_with_kernel_events": round(ms_events / args.steps, 4)},
        "kernels": kern,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
