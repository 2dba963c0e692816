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


def seq_shapes(w):
    """[(L_b, C_b)] of the workload's sequences (one for single-length ones)."""
    from prompt_kv_selection_amd import workloads as WL
    if w.ragged:
        return list(zip(WL.seq_lengths(w), WL.budgets(w)))
    return [(w.L, w.C)]


def kernel_alg_bytes(name, w, lse=False, group=1, seqs=None, rows=False):
    """Algorithmic bytes one launch of a kernel moves for one call of w.heads
    heads over the sequences seqs [(L, C)] (lse: the row statistics are handed
    over, so only the prefix keys, Qwin and the W log-sum-exps per head are
    read for the votes; group: query heads per K/V head, whose K is read once
    for the whole group; rows: the selection ran one workgroup per row and
    the gather kernel copied the rows)."""
    e = 2 if w.dtype == "bf16" else 4
    H, W, D = w.heads, w.W, w.D
    seqs = seqs or seq_shapes(w)
    Hkv = H // group
    q = len(seqs) * H * W * D * e
    sumL = sum(L for L, _ in seqs)
    sumP = sum(L - W for L, _ in seqs)
    sumC = sum(min(L, C) for L, C in seqs)
    nch = sum((L + 1023) // 1024 for L, _ in seqs)
    if group > 1:
        if name == "window_stats":      # K of every K/V head once, Qwin, partials
            return Hkv * sumL * D * e + q + H * nch * W * 8
        if name == "window_votes":      # prefix K of every K/V head, Qwin, partials (or lse), votes out
            return Hkv * sumP * D * e + q + (len(seqs) * H * W * 4 if lse else H * nch * W * 8) + H * sumP * 4
    if lse and name in ("window_fused", "window_votes"):
        return H * sumP * D * e + q + len(seqs) * H * W * 4 + H * sumP * 4
    if name == "window_fused":      # K once, Qwin, votes out (exchange slots are noise)
        return H * sumL * D * e + q + H * sumP * 4
    if name == "window_stats":      # K once, Qwin, partial (max, sum) per chunk
        return H * sumL * D * e + q + H * nch * W * 8
    if name == "window_votes":      # prefix K, Qwin, partials, votes out
        return H * sumP * D * e + q + H * nch * W * 8 + H * sumP * 4
    if name == "pool":              # votes in, pooled out
        return H * sumP * 8
    if name == "candidates":        # pooled scores read once (the histogram reads hit L2)
        return H * sumP * 4
    if name == "threshold":         # histograms, segment counts (the candidates: data-dependent, few)
        return len(seqs) * H * (2048 * 4 + 2 * 512 * 4)
    if name == "emit":              # pooled scores, kept K and V rows read and written, indices
        return H * sumP * 4 + 4 * H * sumC * D * e + H * sumC * 4
    if name == "select" and rows:   # whole rows: pooled scores read, indices written (the copy is gather's)
        return H * sumP * 4 + H * sumC * 4
    if name == "select":            # votes read, indices written, kept K and V rows read and written
        return H * sumP * 4 + H * sumC * 4 + 4 * H * sumC * D * e
    if name == "gather":            # indices read, kept K and V rows read and written
        return H * sumC * 4 + 4 * H * sumC * D * e
    return None                     # fill: workspace clearing, not the method's traffic


def path_alg_bytes(w, group=1, seqs=None):
    """Minimum bytes of the whole path per layer call: K of every K/V head
    once, Qwin, the kept K/V rows read and written, the indices."""
    e = 2 if w.dtype == "bf16" else 4
    seqs = seqs or seq_shapes(w)
    total = 0
    for L, C in seqs:
        n = min(L, C)
        total += (w.heads // group) * L * w.D * e + w.heads * (w.W * w.D * e + 4 * n * w.D * e + 4 * n)
    return total


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
    "probe_tiles": ("kvsel_probe.hip",),
    "probe_vector": ("kvsel_probe.hip",),
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


def numpy_threads():
    """Thread settings of numpy's native libraries (BLAS/OpenMP pools)."""
    try:
        from threadpoolctl import threadpool_info
        return [{"api": d.get("user_api"), "lib": d.get("internal_api"), "threads": d.get("num_threads")}
                for d in threadpool_info()]
    except Exception as exc:  # pragma: no cover - informational only
        return [{"error": repr(exc)}]


def cpu_baseline(w, seconds):
    """The CPU oracle on a bounded sample of the same workload: (sequence,
    head) units of layer 0 (then layer 1, ...) in a thread pool, until
    `seconds` of oracle time have passed after a full batch of units.  The
    pool holds one thread per core of the process's affinity mask, at most
    16: the host share of one GPU on the boxes this runs on, whatever larger
    mask the container shows."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import snapkv_oracle as O
    from prompt_kv_selection_amd import workloads as WL

    affinity = len(os.sched_getaffinity(0))
    threads = max(1, min(16, affinity))
    seqs = seq_shapes(w)
    jobs = [(l, b, h) for l in range(w.layers) for b in range(len(seqs)) for h in range(w.heads)]
    inputs = {}

    def prepare(job):
        l, b, h = job
        q, k, v = WL.head_arrays(w, h, layer=l, seq=b, L=seqs[b][0])
        return job, (WL.to_float64(q, w.dtype), WL.to_float64(k, w.dtype), WL.to_float64(v, w.dtype))

    def run(job):
        q, k, v = inputs.pop(job)
        O.snapkv_select(q, k, v, w.W, seqs[job[1]][1], w.kernel, w.pooling)

    done = 0
    tokens = 0.0
    elapsed = 0.0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while done < len(jobs) and elapsed < seconds:
            batch = jobs[done:done + threads]
            inputs.update(dict(ex.map(prepare, batch)))     # input drawing is not timed
            t0 = time.perf_counter()
            list(ex.map(run, batch))
            elapsed += time.perf_counter() - t0
            done += len(batch)
            tokens += sum(seqs[j[1]][0] for j in batch) / w.heads
    return {"value": tokens / elapsed, "unit": "prompt tokens scored/s", "cores": threads, "kind": "oracle",
            "affinity_cores": affinity, "numpy_threads": numpy_threads(),
            "sample": f"{done} (sequence, head) units (layer-major) of the same workload, {elapsed:.1f} s of oracle "
                      f"time; value = sum of L over the units / heads per layer / time"}


def measure_ceiling(B, torch, dev, stream):
    """Streaming-read ceilings of this device (kvsel_probe_stream), in GB/s:
    the scoring kernel's pattern (mode 0: 8 waves per CU, one 8 KiB
    direct-to-LDS tile in flight each) over a cold 256 MiB buffer (eight
    consecutive slices of a 2 GiB buffer, so the previous passes evicted it
    from the last-level cache), the same slice read twice in a row (warm),
    one 2 GiB pass, and the same patterns with non-temporal loads (mode 4),
    with two tiles per wave (mode 1) and with 16-byte vector loads (mode 3)
    cold."""
    big = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    big.view(torch.int32).random_()
    sink = torch.empty(B.kvsel_probe_sink_bytes(), dtype=torch.uint8, device=dev)
    sl = 256 << 20
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(src, mode):
        ev[0].record(stream)
        B.kvsel_probe_stream(src, mode, sink, stream=stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / 1e3

    out = {}
    for mode, tag in ((0, "tiles1x8"), (4, "tiles1x8nt"), (1, "tiles2x8"), (3, "vector")):
        times = []
        for rep in range(2):
            for i in range(8):
                times.append(timed(big[i * sl:(i + 1) * sl], mode))
        times.sort()
        out[f"{tag}_cold_256MiB_GBps"] = round(sl / times[len(times) // 2] / 1e9, 1)
    timed(big[:sl], 0)
    out["tiles1x8_warm_256MiB_GBps"] = round(sl / timed(big[:sl], 0) / 1e9, 1)
    out["tiles1x8_2GiB_GBps"] = round(big.numel() / timed(big, 0) / 1e9, 1)
    out["note"] = "median of 16 passes for the cold figures; kvsel_probe_stream, HIP events on the launch stream"
    del big
    torch.cuda.synchronize()
    return out


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
                     "traffic": counters_from_profiles(dom).get("bytes_per_launch") if N == 32768 else None},
        "path": {"alg_bytes_per_call": moved, "alg_GBps": round(moved * layers / (ms / 1e3) / 1e9, 1),
                 "us_per_call": round(ms * 1e3 / layers, 2)},
        "kernels": kern,
    }), flush=True)


# Profiling runs summarised by --digest: the bench arguments of each tag.
# Every run is `python3 bench.py` under rocprofv3 (committed files only).
PROFILE_TAGS = {
    "auto": [],
    "two_pass": ["--scoring", "two_pass"],
    "lse": ["--lse"],
    "gqa4": ["--gqa", "4"],
    "fallback": ["--force-fallback"],
    "c2": ["--workload", "lognorm_h32_l16k"],
    "c4": ["--workload", "ragged_b8_h32_l4k_64k"],
    "c5": ["--workload", "tied_h64_l128k"],
    "fold": ["--fold"],
}
# The kernels whose counters a tag records in profiles/traffic.json: only
# the ones that tag's timed calls launch (the --lse run also makes untimed
# full-path calls for its log-sum-exps, whose kernels it does not own).
TRAFFIC_OWNER = {"auto": ("window_fused", "select", "fill"), "lse": ("window_fused_lse",),
                 "two_pass": ("window_stats", "window_votes")}
# (pattern in the mangled kernel name, short name), first match wins.
SHORT_NAMES = [("window_fused_kernelILi128ELb1E", "window_fused_lse"), ("window_fused", "window_fused"),
               ("select_coop", "select"), ("select_split", "select"), ("fill_u32", "fill"), ("zero_kernel", "fill"),
               ("window_stats", "window_stats"), ("window_votes", "window_votes"), ("pool_hist", "pool"),
               ("candidates", "candidates"), ("threshold", "threshold"), ("emit_kernel", "emit"),
               ("gather_kernel", "gather"), ("select_hist", "select_hist"), ("copyBuffer", "copy"),
               ("probe_tiles", "probe_tiles"), ("probe_vector", "probe_vector"), ("check_finite", "check")]


def short_name(n):
    for k, v in SHORT_NAMES:
        if k in n:
            return v
    return n[:40]


def profile_commands(tag):
    """The rocprofv3 commands of a profiling tag: kernel trace, FETCH_SIZE,
    WRITE_SIZE and the MFMA counters, each its own run."""
    extra = " ".join(PROFILE_TAGS[tag])
    layered = "--workload" not in PROFILE_TAGS[tag] and "--fold" not in PROFILE_TAGS[tag]
    short = f"--steps 1 --warmup 0 {'--layers 4 ' if layered else ''}--no-cpu-baseline --no-ceiling"
    base = "python3 bench.py"
    return {
        "trace": f"rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_trace_{tag} -o trace -- "
                 f"{base} --steps 3 --warmup 1 --no-cpu-baseline --no-ceiling {extra}".rstrip(),
        "fetch": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/prof_fetch_{tag} -o fetch -- "
                 f"{base} {short} --copy-probe {extra}".rstrip(),
        "write": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/prof_write_{tag} -o write -- "
                 f"{base} {short} --copy-probe {extra}".rstrip(),
        "mfma": f"rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 --output-format csv "
                f"-d gpurun_out/prof_mfma_{tag} -o mfma -- {base} {short} {extra}".rstrip(),
    }


def digest(tag, name, title):
    """profiles/NAME.md from the rocprofv3 outputs of a profiling tag, and,
    for the benchmark workload's default paths, the counter-derived figures
    per kernel in profiles/traffic.json (with the digest of the kernel's
    sources, so that a later source change invalidates them)."""
    import collections
    import csv

    from prompt_kv_selection_amd import workloads as WL

    out_dir = os.path.join(ROOT, "gpurun_out")
    cmds = profile_commands(tag)
    args = PROFILE_TAGS[tag]
    wname = args[args.index("--workload") + 1] if "--workload" in args else "spike_l32x_h32_l32k"
    wl = WL.get(wname)
    if "--fold" in args:  # one launch covers every layer
        wl = WL.reduced(wl, name=wl.name, heads=wl.heads * wl.layers, layers=1)
    lse, group = "--lse" in args, int(args[args.index("--gqa") + 1]) if "--gqa" in args else 1

    def rows(path):
        with open(path) as f:
            return list(csv.DictReader(f))

    def per_kernel(path, counter):
        """Average counter value per dispatch of each kernel, and dispatch
        counts.  For the probe copy, the largest dispatch: the runtime also
        launches a few tiny copies of its own."""
        if not os.path.exists(path):
            return {}, {}
        agg = collections.defaultdict(list)
        for r in rows(path):
            if r["Counter_Name"] == counter:
                agg[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
        avg = {k: (max(v) if k == "copy" else sum(v) / len(v)) for k, v in agg.items()}
        return avg, {k: len(v) for k, v in agg.items()}

    stats = rows(os.path.join(out_dir, f"prof_trace_{tag}", "trace_kernel_stats.csv"))
    fetch, nf = per_kernel(os.path.join(out_dir, f"prof_fetch_{tag}", "fetch_counter_collection.csv"), "FETCH_SIZE")
    write, _ = per_kernel(os.path.join(out_dir, f"prof_write_{tag}", "write_counter_collection.csv"), "WRITE_SIZE")
    mpath = os.path.join(out_dir, f"prof_mfma_{tag}", "mfma_counter_collection.csv")
    mutil, _ = per_kernel(mpath, "MfmaUtil")
    mops, _ = per_kernel(mpath, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    avg_ns = {short_name(r["Name"]): float(r["AverageNs"]) for r in stats}
    bench_line = {}
    logp = os.path.join(out_dir, f"prof_trace_{tag}.log")
    if os.path.exists(logp):
        lines = [ln for ln in open(logp) if ln.startswith("{")]
        bench_line = json.loads(lines[-1]) if lines else {}

    md = [f"# {title}", ""]
    if bench_line:
        md.append(f"Bench line of the traced run: value {bench_line.get('value', 0):.4g} prompt tokens scored/s, "
                  f"{bench_line.get('ms_per_step', 0)} ms per step; path {bench_line.get('config', {}).get('path')}, "
                  f"fallbacks {bench_line.get('config', {}).get('fallbacks')} (the profiler adds a little).")
        md.append("")
    md += ["## Kernel trace (rocprofv3 --kernel-trace --stats)", "", "```", cmds["trace"], "```", "",
           "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["Percentage"])):
        md.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    traffic_path = os.path.join(ROOT, "profiles", "traffic.json")
    traffic = json.load(open(traffic_path)) if os.path.exists(traffic_path) else {"kernels": {}}
    if fetch and "copy" in fetch and "copy" in write:
        copy_bytes = 1 << 30
        fs, wsc = copy_bytes / 1024 / fetch["copy"], copy_bytes / 1024 / write["copy"]
        md += ["", "## HBM traffic per dispatch (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)", "", "```",
               cmds["fetch"], cmds["write"], "```", "",
               f"Scale: a 1 GiB device copy (`__amd_rocclr_copyBuffer`, run by `--copy-probe`: its one large "
               f"dispatch) reads FETCH_SIZE = "
               f"{fetch['copy']:.0f} KiB and writes WRITE_SIZE = {write['copy']:.0f} KiB, so FETCH_SIZE is "
               f"multiplied by {fs:.3f} and WRITE_SIZE by {wsc:.3f} to get bytes.", "",
               "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (scaled) | write MB (scaled) | "
               "algorithmic MB |", "|---|---|---|---|---|---|---|"]
        # Calls profiled: one dispatch of a scoring kernel starts each.
        starts = [k for k in ("window_fused", "window_fused_lse", "window_stats") if k in nf] or \
            [k for k in ("window_votes",) if k in nf]
        n_calls = sum(nf[k] for k in starts) if starts else None
        for k in fetch:
            if k == "copy":
                continue
            rb, wb = fetch[k] * 1024 * fs, write.get(k, 0) * 1024 * wsc
            ab = kernel_alg_bytes(k.replace("_lse", ""), wl, k.endswith("_lse") or lse, group, None, "gather" in fetch)
            if ab is not None and n_calls:  # per dispatch: a call may launch a kernel several times
                ab /= max(1.0, nf[k] / n_calls)
            md.append(f"| `{k}` | {nf[k]} | {fetch[k]:.0f} | {write.get(k, 0):.0f} | {rb / 1e6:.1f} | "
                      f"{wb / 1e6:.1f} | {'' if ab is None else f'{ab / 1e6:.1f}'} |")
            if k in TRAFFIC_OWNER.get(tag, ()) and k in KERNEL_SOURCES:
                ent = traffic["kernels"].get(k, {})
                ent.update({"read_bytes": rb, "write_bytes": wb, "bytes_per_launch": rb + wb,
                            "source_digest": source_digest(k), "workload": wname,
                            "commands": [cmds["fetch"], cmds["write"]]})
                traffic["kernels"][k] = ent
        if TRAFFIC_OWNER.get(tag):
            traffic["scale"] = {"FETCH_SIZE": fs, "WRITE_SIZE": wsc}
    if mutil:
        md += ["", "## MFMA utilisation per dispatch (rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16)", "",
               "```", cmds["mfma"], "```", "",
               "MfmaUtil is rocprofv3's derived counter: the SIMDs' MFMA-busy cycles over (GPU-active cycles x "
               "SIMDs), in percent. MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; the rate divides them by "
               "the kernel's average duration in the trace above.", "",
               "| kernel | MfmaUtil % | bf16 MFMA GFLOP per dispatch | TFLOP/s at the traced duration |",
               "|---|---|---|---|"]
        for k in mutil:
            fl = mops.get(k, 0.0) * 512
            t = avg_ns.get(k)
            rate = f"{fl / (t * 1e-9) / 1e12:.1f}" if t else ""
            md.append(f"| `{k}` | {mutil[k]:.2f} | {fl / 1e9:.2f} | {rate} |")
            if k in TRAFFIC_OWNER.get(tag, ()) and k in KERNEL_SOURCES and k in traffic["kernels"]:
                traffic["kernels"][k].update({"mfma_busy": round(mutil[k] / 100.0, 5), "mfma_flops": fl,
                                              "mfma_command": cmds["mfma"]})
    for k in list(traffic["kernels"]):
        if k not in KERNEL_SOURCES or traffic["kernels"][k].get("source_digest") != source_digest(k):
            traffic["kernels"].pop(k)
    traffic.pop("commands", None)
    traffic["workload"] = "spike_l32x_h32_l32k"
    traffic["written_by"] = "python3 bench.py --digest TAG NAME TITLE"
    with open(os.path.join(ROOT, "profiles", f"{name}.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    with open(traffic_path, "w") as f:
        json.dump(traffic, f, indent=1)
    print("\n".join(md))


def counters_from_profiles(kernel):
    """Counter-derived figures of a kernel (HBM bytes per launch, MFMA busy
    fraction) stored in profiles/traffic.json, if they were taken on the
    kernel's current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get("kernels", {}).get(kernel)
    if not ent or kernel not in KERNEL_SOURCES or ent.get("source_digest") != source_digest(kernel):
        return {}
    return ent


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="spike_l32x_h32_l32k")
    ap.add_argument("--layers", type=int, default=0, help="layers per step (default: the workload's)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling probes")
    ap.add_argument("--scoring", choices=("auto", "two_pass", "single_read"), default="auto",
                    help="scoring path (auto: single-read wherever it applies)")
    ap.add_argument("--select", choices=("auto", "split", "exchange"), default="auto",
                    help="selection kernels (auto: the cooperative selection where its grid fits, else split)")
    ap.add_argument("--force-fallback", action="store_true",
                    help="time the residency fallbacks (the handshakes decide ABORT from the host)")
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
    ap.add_argument("--fold", action="store_true",
                    help="all layers of a step in one call of layers x heads query heads (the per-layer calls "
                         "stay the headline)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one 1 GiB device copy (reference for HBM counter scaling)")
    ap.add_argument("--digest", nargs=3, metavar=("TAG", "NAME", "TITLE"),
                    help="no GPU work: summarise the rocprofv3 outputs gpurun_out/prof_{trace,fetch,write,mfma}_TAG "
                         "into profiles/NAME.md and profiles/traffic.json")
    args = ap.parse_args()

    if args.digest:
        digest(*args.digest)
        return
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
    layers = args.layers or w.layers
    dev = torch.device("cuda:0")
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    H, W, D = w.heads, w.W, w.D
    seqs = seq_shapes(w)
    G = args.gqa
    if G < 1 or H % G:
        raise SystemExit(f"--gqa must divide the {H} heads")
    if w.ragged and (G > 1 or args.lse or args.fold):
        raise SystemExit("--gqa, --lse and --fold time single-length workloads")
    if args.fold and (G > 1 or args.lse):
        raise SystemExit("--fold times the computed-statistics path of one query head per K/V head")
    Hkv = H // G
    stream = torch.cuda.current_stream()

    if w.dtype == "bf16":
        def conv(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        def conv(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    log(f"drawing {layers} layer(s) of {w.name}")
    t0 = time.time()
    Qs, Ks, Vs = [], [], []
    for layer in range(layers):
        if w.ragged:
            Q, K, V, _, _, _ = WL.ragged_arrays(w, layer=layer)
        elif G > 1:  # K/V of the K/V heads only; Qwin of every query head
            _, K, V = WL.layer_arrays(w, layer=layer, heads=range(Hkv))
            Q, _, _ = WL.layer_arrays(WL.reduced(w, L=W, C=W + 1), layer=layer)
        else:
            Q, K, V = WL.layer_arrays(w, layer=layer)
        Qs.append(conv(Q))
        Ks.append(conv(K))
        Vs.append(conv(V))
        del Q, K, V
    # Folded: the layers' heads side by side, one call per step.
    wc = w
    if args.fold:
        Qs, Ks, Vs = [torch.cat(Qs, 0)], [torch.cat(Ks, 0)], [torch.cat(Vs, 0)]
        wc = WL.reduced(w, name=w.name, heads=H * layers, layers=1)
    torch.cuda.synchronize()
    log(f"inputs resident in HBM after {time.time() - t0:.1f} s")
    calls = 1 if args.fold else layers  # calls per step
    Hc = wc.heads                       # query heads per call

    cuL = [0]
    for L, _ in seqs:
        cuL.append(cuL[-1] + L)
    Cs = [C for _, C in seqs]
    n_out = sum(min(L, C) for L, C in seqs)
    if w.ragged:
        ws_bytes = B.kvsel_varlen_workspace_bytes(cuL, Cs, H, W, D, td)
        idx = [torch.empty((H * sum(Cs),), dtype=torch.int32, device=dev) for _ in range(layers)]
        Ko = [torch.empty((H * sum(Cs), D), dtype=td, device=dev) for _ in range(layers)]
        Vo = [torch.empty((H * sum(Cs), D), dtype=td, device=dev) for _ in range(layers)]
    else:
        L, C = seqs[0]
        ws_bytes = B.kvsel_gqa_workspace_bytes(Hc, Hc // G, L, W, C, D, td)
        idx = [torch.empty((Hc, C), dtype=torch.int32, device=dev) for _ in range(calls)]
        Ko = [torch.empty((Hc, C, D), dtype=td, device=dev) for _ in range(calls)]
        Vo = [torch.empty((Hc, C, D), dtype=td, device=dev) for _ in range(calls)]
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    B.kvsel_set_option(B.KVSEL_OPT_SCORING, B.SCORING[args.scoring])
    B.kvsel_set_option(B.KVSEL_OPT_FORCE_FALLBACK, 1 if args.force_fallback else 0)
    B.kvsel_set_option(B.KVSEL_OPT_SELECT, {"auto": B.KVSEL_SELECT_AUTO, "split": B.KVSEL_SELECT_SPLIT,
                                            "exchange": B.KVSEL_SELECT_EXCHANGE}[args.select])

    lses = []
    if args.lse:
        L, C = seqs[0]
        rs = torch.empty((H, W, 2), dtype=torch.float32, device=dev)
        for layer in range(layers):
            B.kvsel_select_gqa(Qs[layer], Ks[layer], Vs[layer], None, L, W, C, D, H, Hkv, w.kernel, w.pooling, td,
                               idx[layer], Ko[layer], Vo[layer], rs, None, None, ws, stream=stream)
            lses.append((rs[:, :, 0].double() + rs[:, :, 1].double().log()).float().contiguous())
        torch.cuda.synchronize()
        log("row log-sum-exps of every layer ready")

    def step():
        for layer in range(calls):
            if w.ragged:
                B.kvsel_select_varlen(Qs[layer], Ks[layer], Vs[layer], cuL, Cs, W, D, H, w.kernel, w.pooling, td,
                                      idx[layer], Ko[layer], Vo[layer], None, None, None, ws, stream=stream)
                continue
            L, C = seqs[0]
            if G > 1:
                B.kvsel_select_gqa(Qs[layer], Ks[layer], Vs[layer], lses[layer] if args.lse else None, L, W, C, D, H,
                                   Hkv, w.kernel, w.pooling, td, idx[layer], Ko[layer], Vo[layer], None, None, None,
                                   ws, stream=stream)
            elif args.lse:
                B.kvsel_select_lse(Qs[layer], Ks[layer], Vs[layer], lses[layer], L, W, C, D, H, w.kernel,
                                   w.pooling, td, idx[layer], Ko[layer], Vo[layer], None, None, ws, stream=stream)
            else:
                B.kvsel_select(Qs[layer], Ks[layer], Vs[layer], L, W, C, D, Hc, w.kernel, w.pooling, td,
                               idx[layer], Ko[layer], Vo[layer], None, None, None, ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    B.kvsel_status_flags(ws, stream, reset=True)  # the sticky flags now cover the timed calls only

    # Timed region: K steps bracketed by synchronisation, no instrumentation.
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)

    # Validity of the timed calls: every call's device-side flags.
    rc = B.kvsel_status(ws, stream)
    last, sticky = B.kvsel_status_flags(ws, stream, reset=True)
    errors = [f for f in B.flag_names(sticky) if not f.endswith("fallback")]
    if rc != B.KVSEL_OK or errors:
        log(f"the timed calls reported device-side errors {errors} (status {rc}: {B.kvsel_last_error()}): "
            "their outputs are unreliable and no figure is printed")
        sys.exit(3)
    path = B.path_names(B.kvsel_last_path())
    fallbacks = [f for f in B.flag_names(sticky) if f.endswith("fallback")]

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
    B.kvsel_set_option(B.KVSEL_OPT_FORCE_FALLBACK, 0)

    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("copy probe: 1 GiB device-to-device copy done")

    ms_step = ms_total / args.steps
    tokens_step = layers * sum(L for L, _ in seqs)
    tokens_per_s = tokens_step * args.steps / (ms_total / 1e3)
    kern = {}
    rows = "gather" in per_kernel
    # The algorithmic bytes are per call; a kernel launched several times in
    # one call (the cooperative selection over several launches) is rated on
    # its time per call, not per launch.
    n_calls = args.steps * calls
    for name, (n, ms) in per_kernel.items():
        ab = kernel_alg_bytes(name, wc, args.lse, G, seqs, rows)
        kern[name] = {"launches": n, "avg_us": round(ms / n * 1e3, 2),
                      "alg_GBps": None if ab is None else round(ab / (ms / n_calls / 1e3) / 1e9, 1)}
        if n > n_calls:
            kern[name]["launches_per_call"] = round(n / n_calls, 2)
    dom = max((k for k in per_kernel if kernel_alg_bytes(k, wc, False, 1, seqs, rows) is not None),
              key=lambda k: per_kernel[k][1])
    ms_dom = per_kernel[dom][1]
    ab_dom = kernel_alg_bytes(dom, wc, args.lse, G, seqs, rows)
    achieved = ab_dom / (ms_dom / n_calls / 1e3) / 1e9
    counted = {} if (G > 1 or w.name != "spike_l32x_h32_l32k" or args.force_fallback or args.fold) else \
        counters_from_profiles(dom + "_lse" if args.lse else dom)
    path_gbps = path_alg_bytes(w, G, seqs) * layers / (ms_step / 1e3) / 1e9

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
        "config": {"workload": w.name, "layers": layers, "heads": H, "W": W, "D": D,
                   "L": [L for L, _ in seqs] if w.ragged else seqs[0][0],
                   "C": Cs if w.ragged else Cs[0],
                   "pooling": w.pooling, "kernel": w.kernel, "keys": w.keys,
                   "scoring": args.scoring, "select": args.select, "row_stats": "handed_over" if args.lse else "computed",
                   "kv_heads": Hkv, "path": path, "fallbacks": fallbacks,
                   "calls_per_step": calls, "heads_per_call": Hc,
                   "forced_fallback": bool(args.force_fallback), "status": "ok"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": counted.get("bytes_per_launch"),
                     "mfma_busy": counted.get("mfma_busy")},
        "path": {"alg_bytes_per_layer": path_alg_bytes(w, G, seqs), "alg_GBps": round(path_gbps, 1),
                 "frac_of_peak": round(path_gbps / HBM_PEAK_GBPS, 4),
                 "ms_per_step_with_kernel_events": round(ms_events / args.steps, 4)},
        "kernels": kern,
    }
    if not args.no_ceiling:
        log("streaming-read ceiling probes")
        del Ks, Vs
        result["ceiling"] = measure_ceiling(B, torch, dev, stream)
        # The scoring kernel's pattern, cached or non-temporal: the higher.
        ce = max(result["ceiling"]["tiles1x8_cold_256MiB_GBps"], result["ceiling"]["tiles1x8nt_cold_256MiB_GBps"])
        result["roofline"]["frac_of_ceiling"] = round(achieved / ce, 4)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
