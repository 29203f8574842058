#!/usr/bin/env python3
"""Throughput of the ISA forward hot path on one MI355X.

One step = one call of isa_attention (pool, saliency, context top-rho,
pack, sharpness + Taylor, query top-gamma, full attention and merge) over one
batch of seeded synthetic inputs already resident in HBM.  Each timed step is
bracketed by HIP events on the launch stream and preceded, outside the timed
region, by a 1 GiB write that flushes the L2 and the Infinity Cache; the
headline is the median step (p10 and p90 beside it), and a warm-cache median
of back-to-back steps is reported too.  Prints one JSON line: the metric
(queries/s), ms per layer call, the library's own dense flash attention on
the same inputs, per-stage times from HIP events placed between the stages of
the same stream, the roofline of the dominant kernel (full attention, bf16
MFMA), the other workload shapes, and the CPU oracle timed on the host cores.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gamma G]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "ISA attn queries/s + ms vs own dense FA, Ns=Nc=17550 H=24 d=128 bf16"
PEAK_FP8_TFLOPS = 5000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="video_dit_layer")
    ap.add_argument("--gamma", type=float, default=None, help="override the workload's gamma")
    ap.add_argument("--dense-steps", type=int, default=3)
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads of the CPU-oracle sample (0: every head of the layer)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-stages", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip timing isa_backward")
    ap.add_argument("--backward-steps", type=int, default=5)
    ap.add_argument("--no-context", action="store_true", help="skip timing the context-token query rows")
    ap.add_argument("--no-fp8", action="store_true", help="skip timing the FP8 variant of the full route")
    ap.add_argument("--no-others", action="store_true", help="skip timing the other workload shapes")
    ap.add_argument("--other-steps", type=int, default=10, help="timed steps per other workload shape")
    ap.add_argument("--profile-pass", action="store_true",
                    help="for counter collection: one layer call, one dense call and a 1 GiB elementwise copy "
                         "(the copy calibrates byte counters), no timing")
    return ap.parse_args()


def full_route_flops(views, w, kq_gamma):
    """Algorithmic FLOPs of one full-attention launch: 4 d per (query, key)
    pair, counting only real rows and real keys (short tail blocks included
    at their size)."""
    Ns, Nc, b, d = w.Ns, w.Nc, w.b, w.d
    full = views["full_q"].cpu().numpy()
    kept = views["kept_ctx"].cpu().numpy()
    n_src = np.array([min(b, Ns - i * b) for i in range((Ns + b - 1) // b)], dtype=np.int64)
    n_ctx = np.array([min(b, Nc - c * b) for c in range((Nc + b - 1) // b)], dtype=np.int64)
    total = 0
    for x in range(full.shape[0]):
        for h in range(full.shape[1]):
            rows = int(n_src[full[x, h]].sum()) if full.shape[2] else 0
            keys = Ns + (int(n_ctx[kept[x, h]].sum()) if kept.shape[2] else 0)
            total += 4 * d * rows * keys
    return total


ROOT = os.path.dirname(os.path.abspath(__file__))
COUNTERS = os.path.join(ROOT, "profiles", "isa_video_dit_counters.txt")


def counted_traffic(kernel_label):
    """HBM bytes per launch of `kernel_label` from the committed rocprofv3
    counter summary (FETCH_SIZE and WRITE_SIZE scaled by what they read for a
    1 GiB copy), or None when the summary is missing or was taken on another
    version of the kernel sources."""
    from sparse_attention_context_amd.profile_summary import sources_digest
    try:
        text = open(COUNTERS).read().splitlines()
    except OSError:
        return None
    digest = sources_digest()
    if not any(digest in ln for ln in text if "sha256" in ln):
        return None
    for ln in text:
        if ln.startswith(kernel_label):
            return float(ln.split()[-3]) * 1e6
    return None


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_head(args):
    from oracle import isa_oracle as orc
    Qh, Kh, Vh, b, rho, gamma = args
    p = orc.oracle_plan_head(Qh, Kh, Vh, b, rho, gamma)
    orc.oracle_forward_head(Qh, Kh, Vh, b, p["kept_ctx"], p["full_q"])


def _oracle_heads(jobs, workers):
    """Wall time of the oracle (plan + forward) on every (batch, head) job,
    `workers` threads, one BLAS thread each (NumPy releases the GIL in its
    array kernels, so the heads run side by side)."""
    import concurrent.futures
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        if workers == 1:
            for j in jobs:
                _oracle_head(j)
        else:
            with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
                list(ex.map(_oracle_head, jobs))
        return time.perf_counter() - t0


def cpu_baseline(w, Q, K, V, gamma, heads):
    """The fp64 oracle on `heads` heads of the same inputs, one worker per
    host core visible to the process (at most 16, the host share of one GPU),
    scaled to the layer; plus the one-core wall time of the two small
    workloads (every head)."""
    from sparse_attention_context_amd.configs import BY_NAME
    from sparse_attention_context_amd.synth import workload_inputs
    visible = len(os.sched_getaffinity(0))
    workers = max(1, min(visible, 16))
    heads = w.H if heads <= 0 else min(heads, w.H)
    jobs = [(Q[0, h], K[0, h], V[0, h], w.b, w.rho, gamma) for h in range(heads)]
    dt = _oracle_heads(jobs, workers)
    per_layer = dt / heads * w.H * w.B
    one_core = {}
    for name in ("tiny_isa_check", "small_video_layer"):
        s = BY_NAME[name]
        q, k, v = workload_inputs(s)
        t = _oracle_heads([(q[x, h], k[x, h], v[x, h], s.b, s.rho, s.gamma) for x in range(s.B) for h in range(s.H)], 1)
        one_core[name] = {"s": round(t, 3), "queries_per_s": round(s.B * s.Ns / t, 1)}
    return {"value": w.B * w.Ns / per_layer, "unit": "queries/s", "cores": workers, "kind": "oracle",
            "sample": "%d of %d heads of the same inputs (plan + forward, fp64 NumPy), %.1f s on %d threads, "
                      "scaled by H/%d" % (heads, w.H, dt, workers, heads),
            "cores_visible": visible, "cpu_model": cpu_model(), "one_core": one_core}


def time_fp8(args, w, gamma, Qd, Kd, Vd, O, ws, views, stream):
    """isa_attention_fp8 (full route in e4m3 on MX-scaled MFMA) on the same
    layer: whole call, its three full-route stages (HIP events), and the FP8
    flash kernel against the fp8 MFMA peak at 4 d FLOP per (query, key)."""
    import torch
    from sparse_attention_context_amd import isa
    O8, ws8, fws = isa.attention_fp8(Qd, Kd, Vd, w.b, w.rho, gamma)
    torch.cuda.synchronize()

    def fstep():
        isa.attention_fp8(Qd, Kd, Vd, w.b, w.rho, gamma, out=O8, workspace=ws8, fp8_workspace=fws)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        fstep()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    st = time_stage_pass(lambda name: isa.run_fp8_stage(name, Qd, Kd, Vd, ws8, fws, w.b, w.rho, gamma, out=O8),
                         isa.FP8_STAGES, args.steps, stream)
    flops = full_route_flops(views, w, gamma)
    tf = flops / (st["full"] * 1e-3) / 1e12 if st.get("full") else None
    log("isa_attention_fp8: %.3f ms/call; full-route stages: %s" % (ms, ", ".join("%s %.3f" % kv for kv in st.items())))
    return {"ms_per_call": round(ms, 4), "queries_per_s": round(w.B * w.Ns / (ms * 1e-3), 1),
            "full_route_stage_ms": {k: round(v, 4) for k, v in st.items()},
            "roofline": None if tf is None else {"kernel": "isa_flash_fp8_pp_kernel", "bound": "mfma",
                                                 "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS,
                                                 "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4)},
            "dtype": "e4m3 operands, fp32 accumulation (bf16 in and out)",
            "error": "3.7-3.8 % rel-L2 of the full-route rows against exact attention (GPU tests)"}


def time_backward(args, w, gamma, Qd, Kd, Vd, O, ws, views, stream):
    """isa_backward on the same layer (plan frozen, dO seeded N(0,1) in bf16):
    whole-call time, per-stage HIP events, and the full-route kernels against
    the bf16 MFMA peak at their algorithmic FLOPs per (query, key) pair."""
    import torch
    from sparse_attention_context_amd import isa
    g = torch.Generator(device=Qd.device).manual_seed(7)
    dO = torch.randn(Qd.shape, generator=g, device=Qd.device, dtype=torch.float32).to(Qd.dtype)
    isa.attention(Qd, Kd, Vd, w.b, w.rho, gamma, out=O, workspace=ws)
    dQ, dK, dV, bws = isa.backward(Qd, Kd, Vd, O, dO, ws, w.b, w.rho, gamma)

    def bstep():
        isa.backward(Qd, Kd, Vd, O, dO, ws, w.b, w.rho, gamma, bwd_workspace=bws, dQ=dQ, dK=dK, dV=dV)

    bstep()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.backward_steps):
        bstep()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.backward_steps
    st = time_stage_pass(lambda name: isa.run_backward_stage(name, Qd, Kd, Vd, O, dO, ws, bws, dQ, dK, dV, w.b, w.rho,
                                                             gamma), isa.BWD_STAGES, args.backward_steps, stream)
    log("isa_backward: %.3f ms/call; stages: %s" % (ms, ", ".join("%s %.3f" % kv for kv in st.items())))
    pairs = full_route_flops(views, w, gamma) // (4 * w.d)
    # per (query, key) pair of the full route: dK kernel S, dP, dK (6 d); dV kernel S, dV (4 d); dQ kernel S, dP, dQ (6 d)
    kernels = {"dk_full": ("isa_bwd_dk_pp_kernel (full route)", 6), "dv_full": ("isa_bwd_dv_pp_kernel (full route)", 4),
               "dq_full": ("isa_bwd_dq_pp_kernel (full route)", 6)}
    rooflines = []
    for key, (label, per) in kernels.items():
        if st.get(key):
            flops = per * w.d * pairs
            tf = flops / (st[key] * 1e-3) / 1e12
            rooflines.append({"kernel": label, "bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "flops_per_launch": flops,
                              "avg_launch_ms": round(st[key], 4)})
    dominant = max(rooflines, key=lambda r: r["avg_launch_ms"]) if rooflines else None
    return {"ms_per_call": round(ms, 4), "queries_per_s": round(w.B * w.Ns / (ms * 1e-3), 1),
            "stage_ms": {k: round(v, 4) for k, v in st.items()}, "dominant": dominant, "rooflines": rooflines,
            "data": "dO seeded N(0,1) in bf16; plan of the timed forward"}


def time_steps(fn, steps, stream, flush):
    """Per-step milliseconds of `steps` calls of fn, each bracketed by HIP
    events on `stream`.  flush (a device tensor) is overwritten before every
    step, outside the events, so each step starts with cold caches; None
    times the steps back to back (warm caches).  The events are read after
    one synchronisation at the end."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for k, (e0, e1) in enumerate(evs):
        if flush is not None:
            flush.fill_(float(k))
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def time_stage_pass(run, names, steps, stream):
    """Per-stage milliseconds: HIP events between the stages of one stream,
    one untimed pass first, then `steps` passes; the median over the passes
    (a pass whose host launches fell behind the GPU shows up as an outlier,
    which the median ignores)."""
    import torch
    for name in names:
        run(name)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    for s in range(steps):
        for i, name in enumerate(names):
            evs[s][i].record(stream)
            run(name)
        evs[s][-1].record(stream)
    torch.cuda.synchronize()
    return {name: float(np.median([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(steps)]))
            for i, name in enumerate(names)}


def summary(ms_list):
    a = np.asarray(ms_list, dtype=np.float64)
    return {"median_ms": round(float(np.median(a)), 4), "p10_ms": round(float(np.percentile(a, 10)), 4),
            "p90_ms": round(float(np.percentile(a, 90)), 4), "mean_ms": round(float(a.mean()), 4), "n": int(a.size)}


def time_other_workloads(args, stream, flush):
    """isa_attention and the dense baseline on the other workload shapes
    (inputs drawn on the device by the same recipe): flushed median, p10,
    p90, warm median, dense ratio and the full-route stage."""
    import torch
    from sparse_attention_context_amd import isa
    from sparse_attention_context_amd.configs import ALL
    from sparse_attention_context_amd.synth import make_inputs_device
    dev = torch.device("cuda:0")
    out = []
    for w in ALL:
        if w.name == args.workload:
            continue
        Qd, Kd, Vd = make_inputs_device(w.B, w.H, w.d, w.Ns, w.Nc, w.seed, dev, w.dtype, w.clips, w.sharp)
        O = torch.empty_like(Qd)
        # the dense kernel takes f32 too
        isa.dense_forward(Qd, Kd, Vd, out=O)
        dense = float(np.median(time_steps(lambda: isa.dense_forward(Qd, Kd, Vd, out=O), 3, stream, flush)))
        for g in (w.gammas or (w.gamma,)):
            desc = isa.desc_for(Qd, Kd, w.b, w.rho, g)
            ws = isa.new_workspace(desc, dev)

            def step():
                isa.attention(Qd, Kd, Vd, w.b, w.rho, g, out=O, workspace=ws)

            step()
            step()
            cold = time_steps(step, args.other_steps, stream, flush)
            warm = time_steps(step, args.other_steps, stream, None)
            layer = isa.CapturedAttention(Qd, Kd, Vd, w.b, w.rho, g, out=O, workspace=ws)
            g_cold = time_steps(layer.replay, args.other_steps, stream, flush)
            del layer
            views = isa.plan_views(Qd, Kd, ws, w.b, w.rho, g)
            names = list(isa.ATTENTION_STAGES)
            if views["counts"]["kq"] == views["counts"]["nb_s"]:
                names[names.index("sharp_taylor")] = "sharp"
            stages = time_stage_pass(lambda name: isa.run_stage(name, Qd, Kd, Vd, ws, w.b, w.rho, g, out=O),
                                     names, 5, stream)
            full_ms = stages["full"] if views["counts"]["kq"] > 0 else None
            c = summary(cold)
            rec = {"workload": w.name, "B": w.B, "H": w.H, "d": w.d, "Ns": w.Ns, "Nc": w.Nc, "b": w.b, "rho": w.rho,
                   "gamma": g, "dtype": w.dtype, "kc": views["counts"]["kc"], "kq": views["counts"]["kq"],
                   "ms": c, "warm_median_ms": round(float(np.median(warm)), 4),
                   "graph_median_ms": round(float(np.median(g_cold)), 4),
                   "queries_per_s": round(w.B * w.Ns / (c["median_ms"] * 1e-3), 1),
                   "dense_ms": None if dense is None else round(dense, 4),
                   "dense_over_isa": None if dense is None else round(dense / c["median_ms"], 3),
                   "stage_ms": {k: round(v, 4) for k, v in stages.items()}}
            if full_ms:
                fl = full_route_flops(views, w, g)
                rec["full_route_ms"] = round(full_ms, 4)
                rec["full_route_tflops"] = round(fl / (full_ms * 1e-3) / 1e12, 1)
            out.append(rec)
            log("other workload %s gamma=%g: %.3f ms (p10 %.3f p90 %.3f, warm %.3f, graph %.3f), dense %s"
                % (w.name, g, c["median_ms"], c["p10_ms"], c["p90_ms"], rec["warm_median_ms"], rec["graph_median_ms"],
                   "-" if dense is None else "%.3f ms" % dense))
            del ws
        del Qd, Kd, Vd, O
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the ISA path here runs on a single MI355X with no "
              "sharding or collectives (--gpus %d requested)" % max(args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_attention_context_amd import isa
    from sparse_attention_context_amd.configs import BY_NAME
    from sparse_attention_context_amd.synth import workload_inputs

    w = BY_NAME[args.workload]
    gamma = w.gamma if args.gamma is None else args.gamma
    log("workload %s B=%d H=%d d=%d Ns=%d Nc=%d b=%d rho=%g gamma=%g %s" %
        (w.name, w.B, w.H, w.d, w.Ns, w.Nc, w.b, w.rho, gamma, w.dtype))
    Q, K, V = workload_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    Qd = torch.from_numpy(Q).to(dev).to(dt)
    Kd = torch.from_numpy(K).to(dev).to(dt)
    Vd = torch.from_numpy(V).to(dev).to(dt)
    O = torch.empty_like(Qd)
    desc = isa.desc_for(Qd, Kd, w.b, w.rho, gamma)
    ws = isa.new_workspace(desc, dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    log("inputs resident: %.1f MB" % ((Qd.numel() + Kd.numel() + Vd.numel()) * Qd.element_size() / 1e6))

    def step():
        isa.attention(Qd, Kd, Vd, w.b, w.rho, gamma, out=O, workspace=ws)

    if args.profile_pass:
        step()
        torch.cuda.synchronize()
        if w.dtype == "bf16":
            isa.dense_forward(Qd, Kd, Vd, out=O)
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)                                  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        log("profile pass done (copy probe: 1 GiB read + 1 GiB written by the elementwise mul kernel)")
        return

    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB: more than L2 + Infinity Cache
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    cold = time_steps(step, args.steps, stream, flush)
    warm = time_steps(step, args.steps, stream, None)
    ms = float(np.median(cold))
    log("isa_attention: %.3f ms/call (median of %d flushed steps; p10 %.3f, p90 %.3f; warm median %.3f)"
        % (ms, len(cold), np.percentile(cold, 10), np.percentile(cold, 90), np.median(warm)))
    # the same call captured in a HIP graph: one host launch per step
    layer = isa.CapturedAttention(Qd, Kd, Vd, w.b, w.rho, gamma, out=O, workspace=ws)
    g_cold = time_steps(layer.replay, args.steps, stream, flush)
    g_warm = time_steps(layer.replay, args.steps, stream, None)
    log("isa_attention as a graph: %.3f ms/replay (median, flushed; p10 %.3f, p90 %.3f; warm median %.3f)"
        % (np.median(g_cold), np.percentile(g_cold, 10), np.percentile(g_cold, 90), np.median(g_warm)))
    views = isa.plan_views(Qd, Kd, ws, w.b, w.rho, gamma)
    counts = views["counts"]

    # per-stage durations: events between the stages of the same stream
    stage_ms = {}
    if not args.no_stages:
        names = list(isa.ATTENTION_STAGES)
        if counts["kq"] == counts["nb_s"]:
            names[names.index("sharp_taylor")] = "sharp"
        stage_ms = time_stage_pass(lambda name: isa.run_stage(name, Qd, Kd, Vd, ws, w.b, w.rho, gamma, out=O),
                                   names, args.steps, stream)
        log("stages (median of %d passes): %s" % (args.steps, ", ".join("%s %.3f" % kv for kv in stage_ms.items())))
    # host time to enqueue one call (the binding's argument checks and the
    # library's launches), against which the GPU time per call is measured
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(10):
        step()
    host_us = (time.perf_counter() - t0) / 10 * 1e6
    torch.cuda.synchronize()
    log("host time to enqueue one isa_attention call: %.1f us" % host_us)

    dense_ms = None
    if not args.no_dense and w.dtype == "bf16":
        isa.dense_forward(Qd, Kd, Vd, out=O)
        dense_ms = float(np.median(time_steps(lambda: isa.dense_forward(Qd, Kd, Vd, out=O), args.dense_steps,
                                              stream, flush)))
        log("isa_dense_forward: %.3f ms/call (median of %d flushed calls)" % (dense_ms, args.dense_steps))

    # roofline of the dominant kernel (full attention)
    flops = full_route_flops(views, w, gamma)
    full_ms = stage_ms.get("full")
    roofline = None
    if full_ms and flops:
        achieved = flops / (full_ms * 1e-3) / 1e12
        traffic = None
        if w.name == "video_dit_layer":
            traffic = counted_traffic("isa_flash_pps_kernel full route") or counted_traffic("isa_flash_pp_kernel<1,1> full route")
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                    "kernel": "full-route flash kernel (isa_flash_pps_kernel, persistent: whole row tiles, then stream-K ranges; isa_flash_pp_kernel<1,1> when K and V have different row maps; gathered K/V; merge of the split row tiles timed separately)", "flops_per_launch": flops,
                    "avg_launch_ms": round(full_ms, 4)}
    dense_flops = 4 * w.d * w.Ns * (w.Ns + w.Nc) * w.B * w.H

    # the other kernels against their own rooflines (algorithmic work per launch)
    others = []
    es = 2 if w.dtype == "bf16" else 4
    nb_s = (w.Ns + w.b - 1) // w.b
    M = nb_s + (w.Nc + w.b - 1) // w.b
    if stage_ms.get("pool"):
        pool_bytes = w.B * w.H * ((w.Ns + (w.Ns + w.Nc) + w.Ns) * w.d * es + (nb_s + 2 * M) * w.d * 4)
        gbs = pool_bytes / (stage_ms["pool"] * 1e-3) / 1e9
        others.append({"kernel": "isa_pool_kernel", "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                       "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": pool_bytes,
                       "avg_launch_ms": round(stage_ms["pool"], 4),
                       "traffic": counted_traffic("isa_pool_kernel") if w.name == "video_dit_layer" else None})
    if stage_ms.get("sharp_taylor"):
        mk = nb_s + counts["kc"]
        pooled_flops = 6 * w.d * w.Ns * mk * w.B * w.H
        tf = pooled_flops / (stage_ms["sharp_taylor"] * 1e-3) / 1e12
        # its HBM floor: Q read, O and the per-row peak written once, the packed kept set read once per head
        pooled_bytes = w.B * w.H * (2 * w.Ns * w.d * es + 4 * w.Ns + mk * (3 * w.d * 2 + 4))
        others.append({"kernel": "isa_flash_pp_pooled_kernel (sharpness + Taylor)", "bound": "mfma",
                       "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                       "frac": round(tf / PEAK_BF16_TFLOPS, 4), "flops_per_launch": pooled_flops,
                       "avg_launch_ms": round(stage_ms["sharp_taylor"], 4), "hbm_bytes_floor": pooled_bytes,
                       "traffic": counted_traffic("isa_flash_pp_pooled_kernel") if w.name == "video_dit_layer" else None,
                       "note": "6 d FLOP per (query, kept block): the hi and the lo key products (2 d each) and P.V "
                               "(2 d); bf16 MFMA"})

    context = None
    if not args.no_context and w.dtype == "bf16" and w.Nc > 0:
        # context-token query rows (dense over all keys): the other half of the in-context layer
        g = torch.Generator(device=dev).manual_seed(11)
        Qc = torch.randn((w.B, w.H, w.Nc, w.d), generator=g, device=dev, dtype=torch.float32).to(Qd.dtype)
        Oc = isa.context_forward(Qc, Kd, Vd)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(args.dense_steps):
            isa.context_forward(Qc, Kd, Vd, out=Oc)
        c1.record(stream)
        torch.cuda.synchronize()
        cms = c0.elapsed_time(c1) / args.dense_steps
        cflops = 4 * w.d * w.Nc * (w.Ns + w.Nc) * w.B * w.H
        context = {"ms": round(cms, 4), "tflops": round(cflops / (cms * 1e-3) / 1e12, 2),
                   "layer_ms_with_isa_source_rows": round(cms + ms, 4),
                   "note": "isa_context_forward: Nc context query rows, dense over all keys"}
        log("isa_context_forward: %.3f ms/call" % cms)

    fp8 = None
    if not args.no_fp8 and w.dtype == "bf16":
        fp8 = time_fp8(args, w, gamma, Qd, Kd, Vd, O, ws, views, stream)

    backward = None
    if not args.no_backward and w.dtype == "bf16":
        backward = time_backward(args, w, gamma, Qd, Kd, Vd, O, ws, views, stream)

    others_wl = None
    if not args.no_others:
        others_wl = time_other_workloads(args, stream, flush)

    cpu = None
    if not args.no_cpu:
        log("cpu oracle on %s heads ..." % (args.cpu_heads or "all"))
        cpu = cpu_baseline(w, Q, K, V, gamma, args.cpu_heads)
        log("cpu oracle: %.1f queries/s" % cpu["value"])

    out = {
        "metric": METRIC,
        "value": round(w.B * w.Ns / (ms * 1e-3), 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "timing": dict(summary(cold), warm_median_ms=round(float(np.median(warm)), 4), host_enqueue_us=round(host_us, 1),
                       graph=dict(summary(g_cold), warm_median_ms=round(float(np.median(g_warm)), 4)),
                       protocol="HIP events around each step on the launch stream; a 1 GiB write before each "
                                "step (outside the events) flushes L2 and the Infinity Cache; value and "
                                "ms_per_step use the median"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, context keys scaled, sharpened queries)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "d": w.d, "Ns": w.Ns, "Nc": w.Nc, "b": w.b,
                   "rho": w.rho, "gamma": gamma, "kc": counts["kc"], "kq": counts["kq"]},
        "dense_ms": None if dense_ms is None else round(dense_ms, 4),
        "dense_over_isa": None if dense_ms is None else round(dense_ms / ms, 3),
        "latency_reduction_vs_dense": None if dense_ms is None else round(1 - ms / dense_ms, 4),
        "dense_tflops": None if dense_ms is None else round(dense_flops / (dense_ms * 1e-3) / 1e12, 2),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "roofline": roofline,
        "other_rooflines": others,
        "cpu_baseline": cpu,
        "backward": backward,
        "context_rows": context,
        "fp8_variant": fp8,
        "other_workloads": others_wl,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
