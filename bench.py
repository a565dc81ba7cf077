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
    ap.add_argument("--no-dcu", action="store_true", help="skip the dynamic cache update scoring measurement")
    ap.add_argument("--dcu-reps", type=int, default=20)
    ap.add_argument("--dcu-only", action="store_true",
                    help="only the dynamic cache update scoring measurement (the run profiled for it)")
    ap.add_argument("--serial-means", action="store_true",
                    help="block means right before each layer's scoring instead of on a second stream")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--kernel-reps", type=int, default=3,
                    help="passes over the sparse layers in the per-launch timing of the dominant entry point")
    ap.add_argument("--kernel-only", action="store_true",
                    help="after one warm-up step only run the per-launch timing of sparse attention "
                         "(the run profiled with hardware counters)")
    return ap.parse_args()


# ------------------------------------------------------------------ accounting

def step_accounting(wl, n_active, sinks, blocks_per_layer):
    """Algorithmic HBM bytes and flops of every stage of one step (realised sets)."""
    E = 2  # bf16
    d, Hq, Hkv, L, P = wl.d, wl.Hq, wl.Hkv, wl.L, wl.P
    na = int(n_active)
    q_rows = Hq * na * d * E
    acc = {}
    acc["pcgi"] = dict(bytes=L * 5 + na * 4, flops=0, calls=1)
    kv_all = 2 * Hkv * L * d * E
    acc["dense"] = dict(bytes=wl.l_dense * (kv_all + 2 * q_rows + Hq * na * 4),
                        flops=wl.l_dense * 4 * na * L * d * Hq, calls=wl.l_dense)
    acc["sinks"] = dict(bytes=Hkv * L * d * E + q_rows + Hq * na * 4 + L * 4,
                        flops=2 * na * L * d * Hq, calls=1)
    n_sparse = wl.layers - wl.l_dense
    nb = -(-P // wl.bs)
    scan = Hkv * P * d * E
    # block means of every sparse layer: one read of the prompt keys, the means written
    acc["means"] = dict(bytes=n_sparse * (scan + Hkv * nb * d * 4), flops=0, calls=n_sparse)
    sb, sf, kb, kf = 0, 0, 0, 0
    snk = set(int(s) for s in sinks if s >= 0)
    for blocks in blocks_per_layer:
        sel = [int(b) for b in blocks if b >= 0]
        blk_keys = sum(min(wl.bs, P - b * wl.bs) for b in sel)
        covered = set(b for b in sel)
        extra = sum(1 for s in snk if s < P and s // wl.bs not in covered)
        n_keys = blk_keys + (L - P) + extra
        kb += Hkv * nb * d * 4 + q_rows + len(sel) * 4       # scoring reads the means and the queries
        kf += 2 * Hq * na * d + 2 * Hkv * nb * d
        sb += 2 * Hkv * n_keys * d * E + 2 * q_rows
        sf += 4 * na * n_keys * d * Hq
    acc["blocks"] = dict(bytes=kb, flops=kf, calls=n_sparse)
    acc["sparse"] = dict(bytes=sb, flops=sf, calls=n_sparse)
    return acc


# ------------------------------------------------------------------ CPU baseline

def cpu_baseline(wl, conf, mask, layer_host, step_bytes, rows_frac=0.25):
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
    for l in (wl.l_dense, wl.layers - 1):
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
                   f"on {len(sub)} of {na} active rows (scaled x{scale_rows:.2f}); block top-C + sparse "
                   f"attention of layers {wl.l_dense + 1} and {wl.layers} on all rows (mean x "
                   f"{wl.layers - wl.l_dense}); dense layers x{wl.l_dense}; sinks taken as the injected "
                   f"positions; extrapolated to one full step"),
        "stage_s": {k: round(v, 4) for k, v in t.items()},
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
    }


# ------------------------------------------------------------------ traffic

# HBM bytes per sparse-attention launch, measured with hardware counters and kept
# as text beside the profiles; it only applies to the kernel sources it was taken on
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_attention_ctx32k_traffic.md")
KERNEL_SOURCES = ("attention_d128.hip", "attention.hip", "attention.cuh", "common.cuh")


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
                     overlap_means=not args.serial_means)
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
    blocks = [run.blocks[l][0, : wl.C].cpu().numpy() for l in range(wl.l_dense, wl.layers)]
    acc = step_accounting(wl, n_active, sinks, blocks)
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
            "GBps": round(a["bytes"] / (tot / 1000) / 1e9, 1) if tot else None,
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
    if not args.no_dcu:
        result["dcu"] = dcu_measurement(F, dev, stream, args)
    print(json.dumps(result), flush=True)


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
