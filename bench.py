#!/usr/bin/env python3
"""Benchmark of the Focus-dLLM sparse attention step on one MI355X (gfx950).

Workload (the 32K-context, 32-layer LLaDA-8B-shaped stack): 32 query and 32 KV
heads, head dim 128, bf16; 32256 prompt + 512 generation tokens with 256 still
masked; n(t) = 16, rho = 2 (k = 32), window w = 32, blocks of 128 keys, top-C = 64,
16 sinks identified at layer l_dense = 2 and reused by layers 3..32.

One step = PCGI + 2 dense layers on the active rows (+ log-sum-exp) + sink
identification + 30 x (block top-C + sparse attention), every part in
libfdl.so's HIP kernels.  Q, K and V of all 32 layers, the confidence and the
mask are drawn once (seeded, synthetic) and stay resident in HBM; the timed
region replays the captured step K times between two HIP events.

Printed: one JSON line.  value = algorithmic HBM bytes of the step / step time
(GB/s); ms_per_step = step time.  Extra fields: per-stage breakdown from events
recorded around every entry-point call of K timed eager steps (block means inline
on the caller's stream there, in the graph on a second stream), the roofline of
the dominant entry point, the block-entry dense refresh of one layer (TFLOP/s), and
the fp64 oracle timed on the host cores on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import hashlib

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, vendor figure
METRIC = "sparse-attn step µs + achieved HBM GB/s (% peak) at 32K ctx, 1 MI355X"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--mode", choices=("graph", "eager"), default="graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-refresh", action="store_true", help="skip the dense-refresh measurement")
    ap.add_argument("--no-cached-means", action="store_true",
                    help="skip the step variant that refreshes the KV cache and its touched block means")
    ap.add_argument("--refresh-reps", type=int, default=3)
    ap.add_argument("--means-ahead", type=int, default=0,
                    help="side-stream block means run this many sparse layers ahead (0: all at the step start)")
    ap.add_argument("--no-dcu", action="store_true", help="skip the dynamic cache update scoring measurement")
    ap.add_argument("--dcu-reps", type=int, default=20)
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (8K, 16K, the 32K batch of 4, the pages' defaults)")
    ap.add_argument("--config-reps", type=int, default=10)
    ap.add_argument("--refresh-only", action="store_true",
                    help="only the block-entry dense refresh of one layer (the run profiled for MFMA counters)")
    ap.add_argument("--conf-only", action="store_true",
                    help="only the confidence / unmask measurement (the run profiled for it)")
    ap.add_argument("--dcu-only", action="store_true",
                    help="only the dynamic cache update scoring measurement (the run profiled for it)")
    ap.add_argument("--serial-means", action="store_true",
                    help="block means right before each layer's scoring instead of on a second stream")
    ap.add_argument("--peaks-only", action="store_true",
                    help="only the achievable read / MFMA rates of the library's measurement kernels")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--kernel-reps", type=int, default=3,
                    help="passes over the sparse layers in the per-launch timing of the dominant entry point")
    ap.add_argument("--kernel-only", action="store_true",
                    help="after one warm-up step only run the per-launch timing of sparse attention "
                         "(the run profiled with hardware counters)")
    return ap.parse_args()


# ------------------------------------------------------------------ accounting

def step_accounting(wl, n_active, sinks, blocks_per_layer, dense_tail=0, per_head=False):
    """Algorithmic HBM bytes and flops of every stage of one step (realised sets).

    `bytes` is what the method must move: every input read once and every output written
    once.  The block means and the relevance parts are intermediates between two entry
    points, and the queries that scoring reads are read again by the attention: those
    extra bytes are counted in `io_bytes` only.  n_active, sinks and blocks_per_layer hold
    one entry per sequence (blocks_per_layer[l][b], per KV head when per_head)."""
    E = 2 if wl.dtype == "bf16" else 4
    d, Hq, Hkv, L, P = wl.d, wl.Hq, wl.Hkv, wl.L, wl.P
    nb = -(-P // wl.bs)
    n_sparse = len(blocks_per_layer)
    n_dense = wl.layers - n_sparse
    acc = {k: dict(bytes=0, io_bytes=0, flops=0, calls=0) for k in ("pcgi", "dense", "sinks", "means", "blocks",
                                                                      "sparse")}
    acc["pcgi"]["calls"] = 1
    acc["dense"]["calls"] = n_dense
    acc["sinks"]["calls"] = 1
    acc["means"]["calls"] = acc["blocks"]["calls"] = acc["sparse"]["calls"] = n_sparse
    kv_all = 2 * Hkv * L * d * E
    scan = Hkv * P * d * E
    for b in range(wl.B):
        na = int(n_active[b])
        q_rows = Hq * na * d * E
        acc["pcgi"]["bytes"] += L * 5 + na * 4
        acc["dense"]["bytes"] += n_dense * (kv_all + 2 * q_rows + Hq * na * 4)
        acc["dense"]["flops"] += n_dense * 4 * na * L * d * Hq
        acc["sinks"]["bytes"] += Hkv * L * d * E + q_rows + Hq * na * 4 + L * 4
        acc["sinks"]["flops"] += 2 * na * L * d * Hq
        acc["means"]["bytes"] += n_sparse * scan
        acc["means"]["io_bytes"] += n_sparse * (scan + Hkv * nb * d * 4)
        snk = set(int(x) for x in sinks[b] if x >= 0)
        for layer_blocks in blocks_per_layer:
            lists = layer_blocks[b] if per_head else [layer_blocks[b]] * Hkv
            n_sel = 0
            for g in range(Hkv):
                sel = [int(x) for x in lists[g] if x >= 0]
                n_sel += len(sel)
                blk_keys = sum(min(wl.bs, P - x * wl.bs) for x in sel)
                covered = set(sel)
                extra = sum(1 for x in snk if x < P and x // wl.bs not in covered)
                n_keys = blk_keys + (L - P) + extra
                acc["sparse"]["bytes"] += 2 * n_keys * d * E
                acc["sparse"]["flops"] += 4 * na * n_keys * d * (Hq // Hkv)
            acc["sparse"]["bytes"] += 2 * q_rows                          # Q rows read, O rows written
            acc["blocks"]["io_bytes"] += Hkv * nb * d * 4 + q_rows + n_sel * 4
            acc["blocks"]["flops"] += 2 * Hq * na * d + 2 * Hkv * nb * d
    for a in acc.values():
        a["io_bytes"] = max(a["io_bytes"], a["bytes"])
    acc["sparse"]["io_bytes"] = acc["sparse"]["bytes"]
    return acc


def percentiles(samples):
    import numpy as np
    x = np.asarray(samples, dtype=np.float64)
    return {"median": round(float(np.median(x)), 4), "p10": round(float(np.percentile(x, 10)), 4),
            "p90": round(float(np.percentile(x, 90)), 4), "n": int(x.size)}


def timed_replays(graph, stream, reps):
    """Per-replay durations (ms) of a captured graph: one event between consecutive replays."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    evs[0].record(stream)
    for i in range(reps):
        graph.replay()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    return [evs[i].elapsed_time(evs[i + 1]) for i in range(reps)]


# ------------------------------------------------------------------ CPU baseline

def cpu_baseline(wl, conf, mask, layer_host, step_bytes, rows_frac=1.0, n_sparse_sample=16):
    """The fp64 oracle on a bounded sample of the step, timed on the host cores."""
    import numpy as np
    from oracle import focus_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing
        threads = 1
    t = {}
    t0 = time.perf_counter()
    focus = O.pcgi_focus(conf[0], mask[0], O.focus_count(wl.n_t, wl.rho))
    active = O.window_active(focus, wl.w, wl.L)
    t["pcgi"] = time.perf_counter() - t0
    na = len(active)
    sub = active[: max(1, int(round(na * rows_frac)))]
    scale_rows = na / len(sub)
    Q, K, V = layer_host(wl.l_dense - 1)
    t0 = time.perf_counter()
    _, lse = O.dense_attention(Q[:, sub], K, V, wl.scale)
    t["dense_layer"] = (time.perf_counter() - t0) * scale_rows
    t0 = time.perf_counter()
    O.sink_scores(Q[:, sub], K, lse, wl.scale)
    t["sinks"] = (time.perf_counter() - t0) * scale_rows
    sinks = synth_sinks = None
    sparse_times = []
    sample_layers = sorted(set(int(round(x)) for x in
                               __import__("numpy").linspace(wl.l_dense, wl.layers - 1, n_sparse_sample)))
    for l in sample_layers:
        Q, K, V = layer_host(l)
        t0 = time.perf_counter()
        R = O.block_relevance(Q[:, active], O.block_means(K, wl.P, wl.bs), wl.scale)
        blocks = O.top_blocks(R, wl.C)
        if sinks is None:
            from workloads import synth
            synth_sinks = synth.sink_positions(wl, 0)
            sinks = synth_sinks
        I_p = O.key_set(sinks, blocks, wl.bs, wl.P, wl.L)
        O.sparse_attention(Q[:, active], K, V, I_p, wl.scale)
        sparse_times.append(time.perf_counter() - t0)
    t["sparse_layer"] = float(np.mean(sparse_times))
    # the same stages on one thread (BLAS limited to one), on a smaller row sample
    t1 = {}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            sub1 = active[: max(1, na // 16)]
            s1 = na / len(sub1)
            Q, K, V = layer_host(wl.l_dense - 1)
            t0 = time.perf_counter()
            _, lse1 = O.dense_attention(Q[:, sub1], K, V, wl.scale)
            t1["dense_layer"] = (time.perf_counter() - t0) * s1
            t0 = time.perf_counter()
            O.sink_scores(Q[:, sub1], K, lse1, wl.scale)
            t1["sinks"] = (time.perf_counter() - t0) * s1
            Q, K, V = layer_host(wl.l_dense)
            t0 = time.perf_counter()
            R = O.block_relevance(Q[:, sub1], O.block_means(K, wl.P, wl.bs), wl.scale)
            I_p = O.key_set(sinks, O.top_blocks(R, wl.C), wl.bs, wl.P, wl.L)
            t_score = time.perf_counter() - t0
            t0 = time.perf_counter()
            O.sparse_attention(Q[:, sub1], K, V, I_p, wl.scale)
            t1["sparse_layer"] = t_score + (time.perf_counter() - t0) * s1
    except ImportError:  # threadpoolctl missing: no single-thread figures
        t1 = {}
    step_s = (t["pcgi"] + wl.l_dense * t["dense_layer"] + t["sinks"] +
              (wl.layers - wl.l_dense) * t["sparse_layer"])
    measured = t["pcgi"] + t["dense_layer"] / scale_rows + t["sinks"] / scale_rows + sum(sparse_times)
    return {
        "value": step_bytes / step_s / 1e9,
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "step_s_extrapolated": step_s,
        "measured_s": measured,
        "sample": (f"fp64 NumPy oracle on host: PCGI; layer {wl.l_dense} dense attention and sink scores "
                   f"on {len(sub)} of {na} active rows (scaled x{scale_rows:.2f}); block means, top-C and "
                   f"sparse attention of layers {[l + 1 for l in sample_layers]} on all rows (mean x "
                   f"{wl.layers - wl.l_dense}); dense layers x{wl.l_dense}; sinks taken as the injected "
                   f"positions; extrapolated to one full step"),
        "stage_s": {k: round(v, 4) for k, v in t.items()},
        "stage_s_one_thread": {k: round(v, 4) for k, v in t1.items()},
        "one_thread_sample": "BLAS limited to one thread; 1/16 of the active rows, scaled (the block "
                             "scoring of the sparse layer on those rows, unscaled)",
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
    }


# ------------------------------------------------------------------ traffic

# HBM bytes per sparse-attention launch, measured with hardware counters and kept
# as text beside the profiles; it only applies to the kernel sources it was taken on
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_attention_ctx32k_traffic.md")
KERNEL_SOURCES = ("attention_d128.hip", "attention_tiles.cuh", "attention.hip", "attention.cuh", "common.cuh")


def kernel_sources_sha256():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "long_context_diffusion_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """(bytes per launch, note): the counter figure, or None when missing or stale."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None, "no counter summary"
    fields = dict(line.split(":", 1) for line in text.splitlines() if line.startswith(("traffic_", "kernel_")))
    fields = {k.strip(): v.strip() for k, v in fields.items()}
    if fields.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None, "counters taken on other kernel sources"
    try:
        return int(fields["traffic_bytes_per_launch"]), "rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated"
    except (KeyError, ValueError):
        return None, "counter summary unreadable"


# ------------------------------------------------------------------ main

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.peaks_only:
        print(json.dumps({"peaks_measured": achievable_peaks("cuda")}), flush=True)
        return
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        c0.record()
        for _ in range(reps):
            dst.copy_(src)
        c1.record()
        torch.cuda.synchronize()
        ms = c0.elapsed_time(c1) / reps
        # a copy reads and writes every byte once
        print(json.dumps({"calibrate_copy_bytes": n, "reps": reps + 2, "ms_per_copy": round(ms, 4),
                          "GBps_read_plus_write": round(2 * n / (ms / 1000) / 1e9, 1)}))
        return

    import long_context_diffusion_amd as F
    from long_context_diffusion_amd.step import StepRunner
    from workloads import configs, synth

    wl = configs.CTX32K_STACK
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    F.fdl.lib()
    if args.dcu_only:
        print(json.dumps({"dcu": dcu_measurement(F, dev, torch.cuda.current_stream(), args)}), flush=True)
        return
    if args.conf_only:
        print(json.dumps({"confidence_unmask": confidence_measurement(F, dev, args)}), flush=True)
        return
    if args.refresh_only:
        q = synth.make_q(wl, 0, 0, dev)
        k, v = synth.make_kv(wl, 0, dev)
        vt = F.transpose_v(v)
        out = torch.empty_like(q)
        F.dense_attention(q, k, v, vt=vt, out=out, want_lse=False, scale=wl.scale)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.refresh_reps):
            F.dense_attention(q, k, v, vt=vt, out=out, want_lse=False, scale=wl.scale)
        e1.record()
        torch.cuda.synchronize()
        rms = e0.elapsed_time(e1) / args.refresh_reps
        rflops = 4.0 * wl.L * wl.L * wl.d * wl.Hq
        print(json.dumps({"dense_refresh": {"ms_per_layer": round(rms, 3),
                                            "TFLOPps": round(rflops / (rms / 1000) / 1e12, 1),
                                            "reps": args.refresh_reps}}), flush=True)
        return
    t_setup = time.time()
    conf_np, mask_np = synth.step_inputs(wl)
    conf = torch.from_numpy(conf_np).to(dev)
    mask = torch.from_numpy(mask_np).to(dev)
    qs, ks, vs = [], [], []
    for l in range(wl.layers):
        k, v = synth.make_kv(wl, l, dev)
        ks.append(k)
        vs.append(v)
        qs.append(synth.make_q(wl, l, 0, dev))
    # V with the keys contiguous, beside V: the attention loads runs of consecutive keys from it
    vts = [F.transpose_v(v) for v in vs]
    torch.cuda.synchronize()
    print(f"# inputs resident: {wl.layers} layers, {sum(t.numel() * 2 for t in qs + ks + vs + vts) / 2**30:.1f} GiB "
          f"(Q, K, V, V^T) in {time.time() - t_setup:.1f}s", file=sys.stderr, flush=True)

    run = StepRunner(B=wl.B, L=wl.L, P=wl.P, Hq=wl.Hq, Hkv=wl.Hkv, d=wl.d, dtype=torch.bfloat16,
                     n_t=wl.n_t, rho=wl.rho, w=wl.w, bs=wl.bs, C=wl.C, n_sinks=wl.n_sinks,
                     layers=wl.layers, l_dense=wl.l_dense, scale=wl.scale, device=dev,
                     overlap_means=not args.serial_means,
                     means_ahead=args.means_ahead if args.means_ahead > 0 else None)
    stream = torch.cuda.current_stream()

    def step(hooks=None):
        run.sparse_step(conf, mask, qs, ks, vs, hooks=hooks, vts=vts)

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()

    # sanity: the injected sinks are found (a cheap guard; the parity tests check everything)
    sinks_found = sorted(run.sinks[0, : wl.n_sinks].cpu().tolist())
    if sinks_found != sorted(synth.sink_positions(wl, 0).tolist()):
        print(f"# warning: sinks {sinks_found} differ from the injected positions", file=sys.stderr)

    def eager_launches(reps):
        """Sparse attention of every sparse layer called back to back on one stream: one
        untimed call, then `reps` passes (the launches whose counters rocprofv3 reads)."""
        run.attend(wl.l_dense, qs[wl.l_dense], ks[wl.l_dense], vs[wl.l_dense], vts[wl.l_dense])
        for _ in range(reps):
            for l in range(wl.l_dense, wl.layers):
                run.attend(l, qs[l], ks[l], vs[l], vts[l])
        torch.cuda.synchronize()
        return reps * (wl.layers - wl.l_dense)

    def launch_timing(reps):
        """Average duration of one sparse-attention call (key list, attention, split merge):
        one pass over every sparse layer is captured in a HIP graph and replayed `reps` times
        back to back on this stream between two HIP events, after one untimed replay.  The
        replays keep the host out of the timing (one launch per pass), also under a
        profiler whose per-dispatch host cost can exceed a kernel's duration.  Returns
        microseconds per call and the number of calls timed."""
        layers = range(wl.l_dense, wl.layers)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for l in layers:
                run.attend(l, qs[l], ks[l], vs[l], vts[l])
        g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        n = reps * len(layers)
        return 1000.0 * a.elapsed_time(b) / n, n

    if args.kernel_only:
        n = eager_launches(args.kernel_reps)
        print(json.dumps({"kernel": "fdl_sparse_attention", "launches": n, "n_active": int(run.n_active[0]),
                          "kernel_sources_sha256": kernel_sources_sha256()}), flush=True)
        return

    # stage events: one pair around every entry-point call
    stage_events = {}

    def make_hooks():
        hooks = {}
        for name in ("pcgi", "dense", "sinks", "means", "blocks", "sparse"):
            def before(name=name):   # on the stream the stage runs on (block means: the second one)
                ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                stage_events.setdefault(name, []).append(ev)
                ev[0].record()

            def after(name=name):
                stage_events[name][-1][1].record()
            hooks[name] = (before, after)
        return hooks

    # eager steps with per-call events (kernel durations of every entry point); the block
    # means run inline here, so that no stage's events also span another stage's kernels
    hooks = make_hooks()
    overlap = run.overlap_means
    run.overlap_means = False
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step(hooks)
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / args.steps
    run.overlap_means = overlap

    mode = args.mode
    if mode == "graph":
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
        except Exception as exc:  # capture unsupported: report eager numbers
            print(f"# graph capture failed ({exc}); timing eager steps", file=sys.stderr)
            mode = "eager"
    if mode == "graph":
        for _ in range(max(args.warmup, 1)):
            graph.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
    else:
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps

    nsteps = max(args.steps, 1)
    stage_ms = {k: [a.elapsed_time(b) / nsteps for a, b in v] for k, v in stage_events.items()}
    n_active = int(run.n_active[0])
    sinks = run.sinks[0, : wl.n_sinks].cpu().numpy()
    blocks = [[run.blocks[l][0, : wl.C].cpu().numpy()] for l in range(wl.l_dense, wl.layers)]
    acc = step_accounting(wl, [n_active], [sinks], blocks)
    step_bytes = sum(a["bytes"] for a in acc.values())
    step_flops = sum(a["flops"] for a in acc.values())
    breakdown = {}
    for name, a in acc.items():
        times = stage_ms.get(name, [])
        tot = sum(times)              # per step (averaged over the timed eager steps)
        calls = len(times) // nsteps
        breakdown[name] = {
            "calls": calls, "ms_total": round(tot, 4),
            "us_per_call": round(1000 * tot / max(calls, 1), 2),
            "GBps": round(a["io_bytes"] / (tot / 1000) / 1e9, 1) if tot else None,
            "TFLOPps": round(a["flops"] / (tot / 1000) / 1e12, 1) if tot and a["flops"] else None,
        }
    # the dominant entry point (largest share of the step) is sparse attention; its launches
    # are timed on their own, back to back, after the timed steps
    dom = max(breakdown, key=lambda n: breakdown[n]["ms_total"])
    if dom != "sparse":
        print(f"# warning: {dom} took more time than sparse attention in the eager steps; "
              "the roofline below is still that of sparse attention", file=sys.stderr)
    dom = "sparse"
    a = acc[dom]
    us_launch, n_launch = launch_timing(args.kernel_reps)
    # the per-step spread: the step's replays again, one event between consecutive ones (after
    # the launch timing, which earlier bench runs took right after the timed steps)
    spread = percentiles(timed_replays(graph, stream, args.steps)) if mode == "graph" else None
    per_call_s = us_launch / 1e6
    bytes_call = a["bytes"] / a["calls"]
    flops_call = a["flops"] / a["calls"]
    t_hbm = bytes_call / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops_call / (BF16_PEAK_TFLOPS * 1e12)
    if t_mfma > t_hbm:
        achieved = flops_call / per_call_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
    else:
        achieved = bytes_call / per_call_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    traffic, traffic_note = measured_traffic()
    roof.update({"traffic": traffic, "traffic_note": traffic_note,
                 "kernel": "fdl_sparse_attention (key list, attention, split merge)",
                 "us_per_launch": round(per_call_s * 1e6, 2), "launches_timed": n_launch,
                 "algorithmic_bytes_per_launch": int(bytes_call), "algorithmic_flops_per_launch": int(flops_call)})

    result = {
        "metric": METRIC,
        "value": round(step_bytes / (ms / 1000) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "global_batch": wl.B, "seq_len": wl.L, "prompt": wl.P, "gen": wl.G,
                   "masked": wl.masked, "heads_q_kv": [wl.Hq, wl.Hkv], "head_dim": wl.d, "layers": wl.layers,
                   "l_dense": wl.l_dense, "k": run.k, "w": wl.w, "block": wl.bs, "top_c": wl.C,
                   "n_sinks": wl.n_sinks, "parallelism": "single GPU"},
        "step_us": round(ms * 1000, 1),
        "ms_per_step_spread": spread,
        "pct_hbm_peak": round(100 * step_bytes / (ms / 1000) / 1e9 / HBM_PEAK_GBS, 2),
        "timing": mode,
        "eager_ms_per_step_with_call_events": round(eager_ms, 4),
        "step_algorithmic_bytes": int(step_bytes),
        "step_algorithmic_flops": int(step_flops),
        "n_active": n_active,
        "breakdown": breakdown,
        "roofline": roof,
    }

    if not args.no_refresh:
        # block-entry refresh of one layer: all 32768 rows attend to all keys
        out = torch.empty_like(qs[0])
        F.dense_attention(qs[0], ks[0], vs[0], vt=vts[0], out=out, want_lse=False, scale=wl.scale)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.refresh_reps):
            F.dense_attention(qs[0], ks[0], vs[0], vt=vts[0], out=out, want_lse=False, scale=wl.scale)
        e1.record(stream)
        torch.cuda.synchronize()
        rms = e0.elapsed_time(e1) / args.refresh_reps
        rflops = 4.0 * wl.L * wl.L * wl.d * wl.Hq
        result["dense_refresh"] = {"ms_per_layer": round(rms, 3),
                                   "TFLOPps": round(rflops / (rms / 1000) / 1e12, 1),
                                   "frac_bf16_peak": round(rflops / (rms / 1000) / 1e12 / BF16_PEAK_TFLOPS, 4),
                                   "flops_per_layer": rflops}
        del out

    if not args.no_cpu_baseline:
        def layer_host(l):
            return (synth.to_f64(qs[l])[0], synth.to_f64(ks[l])[0], synth.to_f64(vs[l])[0])
        result["cpu_baseline"] = cpu_baseline(wl, conf_np, mask_np, layer_host, step_bytes)

    if not args.no_cached_means:
        # Separate variant, never mixed with the headline: the approximate-KV refresh writes
        # the active rows' new K/V into every layer's cache, and the block means of the sparse
        # layers are kept from the previous step and refreshed only where those rows fall
        # (instead of the full scan).  Runs last: it changes the caches' active rows.
        g_new = torch.Generator(device=dev)
        g_new.manual_seed(7)
        shp = (wl.B, wl.Hkv, run.nq_max, wl.d)
        knew = [torch.randn(shp, generator=g_new, device=dev).to(torch.bfloat16) for _ in range(wl.layers)]
        vnew = [torch.randn(shp, generator=g_new, device=dev).to(torch.bfloat16) for _ in range(wl.layers)]

        def cached_step():
            # each layer refreshes its cache rows (and touched block means) right before it
            # attends: its new rows come from its own forward pass, after the previous layer
            run.cached_step(conf, mask, qs, ks, vs, knew, vnew, vts=vts)

        run.init_means(ks)
        for _ in range(2):
            cached_step()
        torch.cuda.synchronize()
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg):
            cached_step()
        cg.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            cg.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1) / args.steps
        na = int(run.n_active[0])
        touched = len({int(r) // wl.bs for r in run.active[0, :na].tolist() if int(r) < wl.P})
        row_b = wl.Hkv * wl.d * 2
        refresh_bytes = wl.layers * na * 5 * row_b          # new K, V read; K, V rows and V^T written
        means_bytes = (wl.layers - wl.l_dense) * touched * wl.Hkv * (wl.bs * wl.d * 2 + wl.d * 4)
        cbytes = step_bytes - acc["means"]["bytes"] + refresh_bytes + means_bytes
        result["cached_means_step"] = {
            "ms_per_step": round(cms, 4), "GBps": round(cbytes / (cms / 1000) / 1e9, 1),
            "algorithmic_bytes": int(cbytes), "refreshed_rows": na, "prompt_blocks_touched": touched,
            "note": "each layer refreshes the active rows of its KV cache and the block means they touch "
                    "right before attending, instead of the full per-layer means scan; not the headline workload"}
    del qs, ks, vs, vts, run
    torch.cuda.empty_cache()
    if not args.no_configs:
        result["configs"] = other_configs(F, dev, args)
        result["peaks_measured"] = achievable_peaks(dev)
        result["confidence_unmask"] = confidence_measurement(F, dev, args)
    if not args.no_dcu:
        result["dcu"] = dcu_measurement(F, dev, stream, args)
    print(json.dumps(result), flush=True)


def roof(bytes_, flops, seconds):
    """The bound of a launch (larger of bytes / HBM peak and flops / bf16 peak) and the
    fraction of it reached in `seconds`."""
    if flops / (BF16_PEAK_TFLOPS * 1e12) > bytes_ / (HBM_PEAK_GBS * 1e9):
        ach = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / BF16_PEAK_TFLOPS, 4)}
    ach = bytes_ / seconds / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4)}


def measure_config(F, dev, wl, args, *, step=0, refresh=False):
    """One sparse step of workload `wl` as bench.py times the headline: inputs resident, the
    step captured in a HIP graph and replayed; then the sparse layers' attention alone, and
    optionally one layer's block-entry dense refresh.  A one-layer workload runs its layer
    both ways (dense with the sinks, then scored and attended sparsely)."""
    import numpy as np
    import torch
    from long_context_diffusion_amd.step import StepRunner
    from workloads import synth
    t0 = time.time()
    if step == 0:
        conf_np, mask_np = synth.step_inputs(wl)
    else:
        states = [synth.scenario(wl, b)[step] for b in range(wl.B)]
        conf_np = np.stack([c for _, c in states])
        mask_np = np.stack([m.astype(np.uint8) for m, _ in states])
    conf = torch.from_numpy(np.ascontiguousarray(conf_np)).to(dev)
    mask = torch.from_numpy(np.ascontiguousarray(mask_np)).to(dev)
    one = wl.layers == wl.l_dense == 1
    n_layers = 2 if one else wl.layers
    qs, ks, vs = [], [], []
    for l in range(wl.layers):
        k, v = synth.make_kv(wl, l, dev)
        ks.append(k)
        vs.append(v)
        qs.append(synth.make_q(wl, l, step, dev))
    if one:
        qs, ks, vs = qs * 2, ks * 2, vs * 2
    vts = [F.transpose_v(v) for v in vs[: wl.layers]]
    if one:
        vts = vts * 2
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    run = StepRunner(B=wl.B, L=wl.L, P=wl.P, Hq=wl.Hq, Hkv=wl.Hkv, d=wl.d, dtype=dt, n_t=wl.n_t, rho=wl.rho,
                     w=wl.w, bs=wl.bs, C=wl.C, n_sinks=wl.n_sinks, layers=n_layers, l_dense=wl.l_dense,
                     scale=wl.scale, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        run.sparse_step(conf, mask, qs, ks, vs, vts=vts)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.sparse_step(conf, mask, qs, ks, vs, vts=vts)
    g.replay()
    torch.cuda.synchronize()
    samples = timed_replays(g, stream, args.config_reps)
    ms = float(np.mean(samples))
    sparse_layers = list(range(wl.l_dense, n_layers))
    n_active = run.n_active.cpu().numpy()
    sinks = run.sinks[:, : wl.n_sinks].cpu().numpy()
    blocks = [run.blocks[l][:, : wl.C].cpu().numpy() for l in sparse_layers]
    acc = step_accounting(dataclass_layers(wl, n_layers), n_active, sinks, blocks)
    step_bytes = sum(a["bytes"] for a in acc.values())
    step_flops = sum(a["flops"] for a in acc.values())
    ga = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ga):
        for l in sparse_layers:
            run.attend(l, qs[l], ks[l], vs[l], vts[l])
    ga.replay()
    torch.cuda.synchronize()
    a_samples = timed_replays(ga, stream, args.config_reps)
    us_call = 1000.0 * float(np.median(a_samples)) / len(sparse_layers)
    sp = acc["sparse"]
    res = {
        "workload": wl.name, "batch": wl.B, "seq_len": wl.L, "heads_q_kv": [wl.Hq, wl.Hkv], "head_dim": wl.d,
        "dtype": wl.dtype, "layers": wl.layers, "l_dense": wl.l_dense, "k": run.k, "w": wl.w, "block": wl.bs,
        "top_c": wl.C, "n_sinks": wl.n_sinks, "step": step, "n_active": [int(x) for x in n_active],
        "ms_per_step": round(ms, 4), "ms_per_step_spread": percentiles(samples),
        "step_algorithmic_bytes": int(step_bytes), "step_algorithmic_flops": int(step_flops),
        "GBps": round(step_bytes / (ms / 1000) / 1e9, 1),
        "pct_hbm_peak": round(100 * step_bytes / (ms / 1000) / 1e9 / HBM_PEAK_GBS, 2),
        "TFLOPps": round(step_flops / (ms / 1000) / 1e12, 1),
        "sparse_attention": dict(roof(sp["bytes"] / sp["calls"], sp["flops"] / sp["calls"], us_call / 1e6),
                                 us_per_call=round(us_call, 2), calls_per_replay=len(sparse_layers),
                                 replays=len(a_samples)),
    }
    if one:
        res["note"] = "one layer, run both ways: dense on the active rows with the sinks, then scored and sparse"
    if refresh:
        out = torch.empty_like(qs[0])
        F.dense_attention(qs[0], ks[0], vs[0], vt=vts[0], out=out, want_lse=False, scale=wl.scale)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        F.dense_attention(qs[0], ks[0], vs[0], vt=vts[0], out=out, want_lse=False, scale=wl.scale)
        e1.record(stream)
        torch.cuda.synchronize()
        rms = e0.elapsed_time(e1)
        rflops = 4.0 * wl.B * wl.L * wl.L * wl.d * wl.Hq
        res["dense_refresh"] = {"ms_per_layer": round(rms, 3), "TFLOPps": round(rflops / (rms / 1000) / 1e12, 1),
                                "frac_bf16_peak": round(rflops / (rms / 1000) / 1e12 / BF16_PEAK_TFLOPS, 4),
                                "flops_per_layer": rflops}
        del out
    res["setup_and_timing_s"] = round(time.time() - t0, 1)
    del qs, ks, vs, vts, run, g, ga
    torch.cuda.empty_cache()
    return res


def dataclass_layers(wl, layers):
    import dataclasses
    return dataclasses.replace(wl, layers=layers)


def other_configs(F, dev, args):
    """The 8K and 16K one-layer workloads, the 32K Dream-shaped batch of 4 (a sparse step
    after the block entry, and one layer of its dense refresh) and the pages' default
    hyper-parameters on the 32K stack."""
    import torch
    from workloads import configs
    out = {}
    for wl, kw in ((configs.CTX8K_MHA, {}), (configs.CTX16K_GQA, {}),
                   (configs.CTX32K_GQA_B4, dict(step=1, refresh=True)), (configs.CTX32K_PAPER, {})):
        print(f"# config {wl.name}", file=sys.stderr, flush=True)
        out[wl.name] = measure_config(F, dev, wl, args, **kw)
        torch.cuda.empty_cache()
    return out


def achievable_peaks(dev):
    """What plain kernels sustain on this GPU, beside the published peaks: the library's own
    streaming read (fdl_calibrate_read: 4 GiB once with non-temporal 16-byte loads, best of
    three grid sizes) and MFMA loop (fdl_calibrate_mfma: one wave per SIMD issuing
    v_mfma_f32_32x32x16_bf16 back to back for about 20 ms); then library rates for context
    (torch's sum over the same 4 GiB, torch.mm bf16 8192^3 through hipBLASLt)."""
    import torch
    import long_context_diffusion_amd as F
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1000

    x = torch.empty(1 << 31, dtype=torch.bfloat16, device=dev).normal_()
    nbytes = x.numel() * 2
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    read = {}
    for per_cu in (4, 8, 16):
        sink = torch.empty((cus * per_cu,), dtype=torch.int32, device=dev)
        read[per_cu] = nbytes / timed(lambda: F.calibrate_read(x, cus * per_cu, sink=sink)) / 1e9
    best_wg = max(read, key=read.get)
    torch_read = nbytes / timed(lambda: x.sum()) / 1e9
    del x
    iters = 200000
    sink = torch.empty((cus * 4, 2), dtype=torch.float32, device=dev)
    t = timed(lambda: F.calibrate_mfma(cus, iters, 1.0, 0.5, sink=sink))
    ok = bool((sink[:, 0] == 16.0 * 0.5 * iters).all() and (sink[:, 1] == 0).all())
    mfma_tf = cus * 4 * iters * F.fdl.CALIBRATE_MFMA_FLOPS_PER_WAVE_ROUND / t / 1e12
    n = 8192
    a = torch.randn((n, n), device=dev).to(torch.bfloat16)
    b = torch.randn((n, n), device=dev).to(torch.bfloat16)
    tf = 2.0 * n ** 3 / timed(lambda: torch.mm(a, b)) / 1e12
    del a, b
    torch.cuda.empty_cache()
    return {"read_GBps": round(read[best_wg], 1), "read_frac_of_8000": round(read[best_wg] / HBM_PEAK_GBS, 4),
            "read_GBps_by_workgroups_per_cu": {k: round(v, 1) for k, v in read.items()},
            "mfma_bf16_TFLOPps": round(mfma_tf, 1), "mfma_frac_of_2500": round(mfma_tf / BF16_PEAK_TFLOPS, 4),
            "mfma_ms": round(t * 1e3, 3), "mfma_result_exact": ok,
            "kernels": "fdl_calibrate_read over 4 GiB; fdl_calibrate_mfma, one wave per SIMD, 8 chains",
            "library": {"torch_sum_read_GBps": round(torch_read, 1), "torch_mm_bf16_TFLOPps": round(tf, 1),
                        "kernels": "torch.sum over 4 GiB bf16; torch.mm bf16 8192 x 8192 x 8192"}}


def confidence_measurement(F, dev, args):
    """fdl_confidence_unmask on the 32K step's masked rows: 256 rows of logits over a
    126464-token vocabulary (LLaDA-8B's), bf16, n(t) = 16.  Algorithmic bytes: the logits
    read once."""
    import torch
    from workloads import synth
    B, M, V, L = 1, 256, 126464, 32768
    logits = synth.make_logits(B, M, V, seed=5, device=dev)
    pos = torch.arange(L - M, L, dtype=torch.int32, device=dev).reshape(1, M)
    mask = torch.ones((B, L), dtype=torch.uint8, device=dev)
    conf = torch.zeros((B, L), dtype=torch.float32, device=dev)
    ws = F.Workspace(dev)
    stream = torch.cuda.current_stream()
    F.confidence_unmask(logits, pos, mask, conf, 16, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    reps = 20
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    evs[0].record(stream)
    for i in range(reps):
        mask.fill_(1)
        F.confidence_unmask(logits, pos, mask, conf, 16, workspace=ws, stream=stream)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    # each interval holds one small fill kernel besides the call
    us = [1000.0 * evs[i].elapsed_time(evs[i + 1]) for i in range(reps)]
    import numpy as np
    med = float(np.median(us))
    nbytes = B * M * V * 2
    return {"workload": f"{M} masked rows x {V} vocabulary, bf16, n(t) = 16", "us_per_call_median": round(med, 2),
            "us_spread": percentiles(us), "algorithmic_bytes": nbytes,
            "roofline": roof(nbytes, 0, med / 1e6), "note": "each timed interval also holds a mask fill kernel"}


def dcu_measurement(F, dev, stream, args):
    """The dynamic cache update scoring of one denoising step (fdl_dcu_select) over the same
    32-layer, 32768-token stack: hidden size 4096, bf16 inputs of two adjacent steps, the 16
    tokens decoded at the step (drawn from the 512-token generation block) as key tokens,
    mandatory windows of 32 and an update budget of a tenth of the stack's layer-tokens.
    Algorithmic bytes per call: both inputs read once (2 H 2 bytes a token), the fp32
    distance written (4 bytes a token) and the update lists written (4 bytes an entry)."""
    import numpy as np
    import torch
    from workloads import synth
    B, NL, L, H, n_keys, w_m = 1, 32, 32768, 4096, 16, 32
    total = NL * L // 10
    x_now, x_prev = synth.make_dcu_inputs(B, NL, L, H, seed=31, device=dev, dtype=torch.bfloat16)
    keys = torch.from_numpy(synth.make_key_tokens(B, n_keys, L - 512, L, seed=31)).to(dev)
    ws = F.Workspace(dev)
    out = F.dcu_select(x_now, x_prev, keys, w_m, total, workspace=ws, stream=stream)
    for _ in range(2):
        F.dcu_select(x_now, x_prev, keys, w_m, total, out=out, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.dcu_reps):
        F.dcu_select(x_now, x_prev, keys, w_m, total, out=out, workspace=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.dcu_reps
    n_upd = int(out[4].sum())
    nbytes = B * NL * L * (2 * H * 2 + 4) + 4 * n_upd
    gbs = nbytes / (ms / 1000) / 1e9
    res = {
        "workload": f"dynamic cache update scoring: {NL} layers x {L} tokens, hidden {H}, bf16, {n_keys} key "
                    f"tokens, window {w_m}, budget {total} layer-tokens",
        "ms_per_call": round(ms, 4), "tokens_per_s": round(B * NL * L / (ms / 1000), 1),
        "update_entries": n_upd, "algorithmic_bytes_per_call": int(nbytes),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "fdl_dcu_select (distance, activity, selection)", "calls_timed": args.dcu_reps},
    }
    if not args.no_cpu_baseline:
        # the oracle's distance on a bounded sample: 2048 tokens of each of 4 layers
        from oracle import focus_oracle as O
        layers = [0, 10, 20, 31]
        rows = np.sort(np.random.default_rng(3).choice(L, 2048, replace=False))
        xs = [(synth.to_f64(x_now[0, l, rows]), synth.to_f64(x_prev[0, l, rows])) for l in layers]
        t0 = time.perf_counter()
        for x, y in xs:
            O.dcu_distance(x, y)
        sec = time.perf_counter() - t0
        n_tok = len(layers) * len(rows)
        res["cpu_baseline"] = {"value": round(n_tok / sec, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"the oracle's fp64 distance of {n_tok} tokens (2048 of each of "
                                         f"{len(layers)} layers); budgets and selection not included"}
    del x_now, x_prev
    return res


if __name__ == "__main__":
    main()
