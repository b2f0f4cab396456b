"""Benchmark: the fp16 batch-1 decode-step linear stream on one MI355X.

One step is the whole hot path once: 28 layers x {qkv 2048x1024, o
1024x1024, gate+up 6144x1024, down 1024x3072} plus the 248320x1024 lm_head,
each GEMV on its own seeded activation.  The timed plan is GROUPED: the 113
GEMVs run as one kernel launch over a work table, enqueued directly each
step (a one-launch plan is not captured into a graph: a graph launch costs
more than the kernel launch it would replace; the ORDERED plan, one node per
linear, is the captured hipGraph timed in the extras).  Inputs are resident
in HBM before timing starts.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
from weight_streaming_gemv_decode_amd.profsum import measured_traffic, measured_traffic_all  # noqa: E402
METRIC = "achieved HBM GB/s (% of peak) for batch-1 GEMV; ms per decode-step stream"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extras", action="store_true", help="only the decode-step stream")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", default="", help="comma list of extras to run (c1,c2,c4,c5,c6,token,conv,graph,topk,probe,ordered,chain,shard)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run a plain 1 GiB fp32 copy kernel (reads 1 GiB, writes 1 GiB) to calibrate "
                         "the FETCH_SIZE / WRITE_SIZE counters of a profiler pass")
    ap.add_argument("--traffic", default=os.path.join(HERE, "profiles", "traffic_hbm_counters_per_config.md"),
                    help="profile summary holding the counter-measured per-launch HBM traffic of every config; "
                         "used only while the kernel sources still hash to the measured ones")
    ap.add_argument("--chain-trace", default="", metavar="OUT_MD",
                    help="trace one persistent step of the dependent C3 chain per work unit "
                         "(wsg_decode_step_trace) and write the stage breakdown to OUT_MD, then exit")
    ap.add_argument("--counter-pass", default="", metavar="MANIFEST",
                    help="run every config a few times for a rocprofv3 counter pass (FETCH_SIZE, WRITE_SIZE), "
                         "after a copy kernel of known size, and write which launches belong to which config "
                         "to MANIFEST (JSON); no timing, no JSON line")
    return ap.parse_args()


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def event_times(torch, fn, reps, stream):
    """Per-call GPU durations (ms) of fn() on `stream`, calls enqueued back to back."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    with torch.cuda.stream(stream):
        evs[0].record(stream)
        for i in range(reps):
            fn(i)
            evs[i + 1].record(stream)
    stream.synchronize()
    return [evs[i].elapsed_time(evs[i + 1]) for i in range(reps)]


def region_time(torch, fn, reps, stream):
    """Mean GPU time (ms) per call of fn(i), i = 0..reps-1, enqueued back to
    back on `stream` with events only before the first and after the last."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
    stream.synchronize()
    return e0.elapsed_time(e1) / reps


def graph_times(torch, fn, inner, reps, stream):
    """Per-call GPU time (ms) of fn(i), i = 0..inner-1 captured once into a
    graph and replayed `reps` times back to back (no host dispatch cost)."""
    with torch.cuda.stream(stream):
        for i in range(inner):
            fn(i)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(inner):
            fn(i)
    with torch.cuda.stream(stream):
        g.replay()
    stream.synchronize()
    out = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        stream.synchronize()
        out.append(e0.elapsed_time(e1) / inner)
    del g
    return out


def probe_same_size(torch, wsgemv, nbytes, stream, graph_inner=0, reps=30, back_to_back=False):
    """Median time (us) of the read probe over `nbytes`, rotated over enough
    copies to defeat the 256 MB Infinity Cache, timed like the workload it
    is compared with: an event after each launch, or launches back to back
    with events around them (back_to_back), or graph_inner calls captured in
    one graph.  Every kernel pays a fixed ramp and drain (about 5 us here),
    so the attainable rate depends on the size."""
    nb = max(16, nbytes // 16 * 16)
    copies = max(1, min(64, -(-(768 << 20) // nb)))
    bufs = [torch.ones(nb, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    out = torch.empty(1 << 14, device="cuda")
    g = wsgemv.read_probe_grid(nb)
    fn = lambda i: wsgemv.read_probe(bufs[i % copies], out, grid=g, stream=stream)  # noqa: E731
    for i in range(3):
        fn(i)
    if graph_inner:
        ts = graph_times(torch, fn, graph_inner, 10, stream)
    elif back_to_back:
        ts = [region_time(torch, fn, reps, stream) for _ in range(5)]
    else:
        ts = event_times(torch, fn, reps, stream)
    del bufs
    return statistics.median(ts) * 1e3


def attainable(torch, wsgemv, nbytes, achieved_us, stream, graph_inner=0, back_to_back_us=None):
    """The read probe over the same bytes, timed as `achieved_us` was; with
    back_to_back_us (the workload's time with launches back to back), also
    the probe timed that way, as a second, separately labelled comparison."""
    t = probe_same_size(torch, wsgemv, nbytes, stream, graph_inner)
    r = {"probe_us": round(t, 2), "probe_GBps": round(nbytes / (t * 1e-6) / 1e9, 1),
         "frac_of_probe": round(t / achieved_us, 4)}
    if back_to_back_us is not None:
        tb = probe_same_size(torch, wsgemv, nbytes, stream, back_to_back=True)
        r["back_to_back"] = {"probe_us": round(tb, 2), "achieved_us": round(back_to_back_us, 2),
                             "frac_of_probe": round(tb / back_to_back_us, 4)}
    return r


def summary(ts):
    ts = sorted(ts)
    return {"median_ms": statistics.median(ts), "p10_ms": ts[len(ts) // 10], "p90_ms": ts[(9 * len(ts)) // 10],
            "mean_ms": sum(ts) / len(ts)}


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo, with its family and
    model numbers (a virtualised host may give only a short name)."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            k, _, v = line.partition(":")
            k = k.strip()
            if k in ("model name", "cpu family", "model") and k not in fields:
                fields[k] = v.strip()
            if line.strip() == "":
                break
    except OSError:
        pass
    name = fields.get("model name") or platform.processor() or platform.machine()
    if "cpu family" in fields and "model" in fields:
        name += f" (family {fields['cpu family']}, model {fields['model']})"
    return name


def oracle_per_config(oracle, synth, step_in, cores):
    """The oracle on one call of each config (one whole int4 step), on 1
    thread and on `cores` threads: ms and GB/s over the config's
    algorithmic bytes."""
    out = {}

    def timed(label, nbytes, fn, fn1=None, bytes1=None, sample1=None):
        """fn on 1 and on `cores` threads (fn1 over bytes1 on 1 thread, when
        the whole config would take too long there)."""
        rec = {"bytes": int(nbytes)}
        for n in (1, cores):
            oracle.set_threads(n)
            f, b = (fn1, bytes1) if (n == 1 and fn1 is not None) else (fn, nbytes)
            t0 = time.perf_counter()
            f()
            dt = time.perf_counter() - t0
            rec[f"threads_{n}"] = {"ms": round(dt * 1e3, 1), "GBps": round(b / dt / 1e9, 3)}
            if n == 1 and fn1 is not None:
                rec["threads_1"]["sample"] = sample1
        out[label] = rec
        log(f"oracle {label}: {rec}")

    N, K = synth.C1_SHAPE
    W = synth.f16_normal(1, 0, (N, K), synth.W_SIGMA)
    x = synth.f16_normal(1, 1, (K,), synth.X_SIGMA)
    timed("c1_2048x2048", N * K * 2 + K * 2 + N * 4, lambda: oracle.gemv_f16(W, x))
    _, W, x = step_in[-1]
    N, K = W.shape
    timed("c2_lm_head_248320x1024", N * K * 2 + K * 2 + N * 4, lambda: oracle.gemv_f16(W, x))
    for (N, K) in synth.C4_SHAPES:
        Wq = synth.int8_uniform(4, 0, (N, K))
        xq = synth.int8_uniform(4, 1, (K,))
        sw = synth.f32_uniform(4, 2, (N,), 0.001, 0.01)
        timed(f"c4_w8a8_{N}x{K}", N * K + N * 4 + K + N * 4 + N * 4,
              lambda: oracle.gemv_w8a8(Wq, sw, xq, synth.X_SCALE_W8A8))
    for M in (1, 4):
        w4 = synth.decode_step_w4(workload=5, M=M)
        nbytes = lambda ls: sum(Wc.nbytes + s4.nbytes + X.nbytes + M * Wc.shape[0] * 4  # noqa: E731
                                for _, Wc, s4, X in ls)
        step = lambda ls: [oracle.gemv_w4a16(Wc, s4, X) for _, Wc, s4, X in ls]  # noqa: E731
        few = w4[:28] if M > 1 else None
        timed(f"c5_w4a16_step_M{M}", nbytes(w4), lambda: step(w4),
              (lambda: step(few)) if few else None, nbytes(few) if few else None,
              "the first 7 decoder layers (28 linears) on 1 thread" if few else None)
        nb = nbytes(w4)
        if M == 1:
            def w4a8():
                for _, Wc, s4, X in w4:
                    xq, sx = oracle.quantize_x_i8(X.reshape(-1))
                    oracle.gemv_w4a8(Wc, s4, xq, sx)
            timed("c6_w4a8_step_M1", nb, w4a8)
        del w4
    return out


def counter_pass(args, torch, synth, wsgemv, dev, stream):
    """Every config a few steps, for a FETCH_SIZE or WRITE_SIZE pass; the
    manifest says which launches belong to which config (in launch order)."""
    configs = []

    def run(label, workload, kernels, steps, nbytes, fn):
        for i in range(steps):
            fn(i)
        stream.synchronize()
        configs.append({"label": label, "workload": workload, "kernels": kernels, "steps": steps,
                        "algorithmic_bytes": int(nbytes)})
        log(f"counter pass: {label} ({steps} steps)")

    with torch.cuda.stream(stream):
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        run("calibration", "plain fp32 copy of 1 GiB", ["AUnaryFunctor"], 3, 2 << 30,
            lambda i: torch.mul(src, 1.0, out=dst))
        del src, dst

        step_in = synth.decode_step_f16(workload=3)
        lins = [wsgemv.Linear(wsgemv.F16, torch.from_numpy(W).to(dev), torch.from_numpy(x).to(dev),
                              torch.empty(W.shape[0], device=dev), W.shape[0], W.shape[1]) for _, W, x in step_in]
        step_bytes = sum(W.nbytes + x.nbytes + W.shape[0] * 4 for _, W, x in step_in)
        g = wsgemv.DecodeStep(lins, wsgemv.STEP_GROUPED, stream=stream)
        run("c3_grouped", "C3 fp16 decode step, GROUPED", ["dense_grouped_kernel<0, 2, 2"], 6, step_bytes,
            lambda i: g(stream))
        g.close()
        y16s, cl = [], []
        x = lins[0].x
        for l in lins:
            y16 = torch.empty(l.N, dtype=torch.float16, device=dev)
            cl.append(wsgemv.Linear(l.kind, l.W, x[:l.K], torch.empty(l.N, device=dev), l.N, l.K, y16=y16))
            y16s.append(y16)
            x = y16
        pc = wsgemv.DecodeStep(cl, wsgemv.STEP_PERSISTENT, stream=stream)
        run("c3_chain_persistent", "C3 as one dependent chain, persistent launch", ["chain_kernel<"], 6, step_bytes,
            lambda i: pc(stream))
        pc.close()
        del cl, y16s

        lm = lins[-1]
        Ws = [lm.W, lm.W.clone()]
        b = lm.N * lm.K * 2 + lm.K * 2 + lm.N * 4
        y = torch.empty(lm.N, device=dev)
        for S, ks in ((1, ["dense_gemv_kernel<0, 1, 2"]), (2, ["dense_gemv_kernel<0, 8, 1"])):
            ws = wsgemv.workspace(wsgemv.F16, 1, lm.N, lm.K, S, dev)
            run(f"c2_S{S}", f"C2 lm_head 248320x1024, S = {S}", ks, 6, b,
                lambda i: wsgemv.gemv_f16(Ws[i % 2], lm.x, y=y, splits=S, ws=ws, stream=stream))
        del Ws, lins, step_in

        N, K = synth.C1_SHAPE
        W = torch.from_numpy(synth.f16_normal(1, 0, (N, K), synth.W_SIGMA)).to(dev)
        xs1 = torch.from_numpy(synth.f16_normal(1, 1, (K,), synth.X_SIGMA)).to(dev)
        copies = [W] + [W.clone() for _ in range(63)]
        y1 = torch.empty(N, device=dev)
        run("c1", "C1 fp16 2048x2048 (64 copies)", ["dense_gemv_kernel<0, 2, 2"], 128, N * K * 2 + K * 2 + N * 4,
            lambda i: wsgemv.gemv_f16(copies[i % 64], xs1, y=y1, stream=stream))
        del copies, W

        for tag, (N, K) in zip("ab", synth.C4_SHAPES):
            Wq = torch.from_numpy(synth.int8_uniform(4, 0, (N, K))).to(dev)
            xq = torch.from_numpy(synth.int8_uniform(4, 1, (K,))).to(dev)
            sw = torch.from_numpy(synth.f32_uniform(4, 2, (N,), 0.001, 0.01)).to(dev)
            xsc = torch.tensor([synth.X_SCALE_W8A8], device=dev)
            xf = torch.from_numpy(synth.f16_normal(4, 3, (K,), synth.X_SIGMA)).to(dev)
            copies = [Wq] + [Wq.clone() for _ in range(8)]
            y4 = torch.empty(N, device=dev)
            acc = torch.empty(N, dtype=torch.int32, device=dev)
            run(f"c4{tag}_w8a8", f"C4{tag} W8A8 {N}x{K} (9 copies)", ["dense_gemv_kernel<1, "], 18,
                N * K + N * 4 + K + N * 4 + N * 4,
                lambda i: wsgemv.gemv_w8a8(copies[i % 9], sw, xq, xsc, y=y4, acc_out=acc, stream=stream))
            run(f"c4{tag}_w8a8_dyn", f"C4{tag} W8A8_DYN {N}x{K} (9 copies)", ["dense_gemv_kernel<4, "], 18,
                N * K + N * 4 + 2 * K + N * 4 + N * 4,
                lambda i: wsgemv.gemv_w8a8_dyn(copies[i % 9], sw, xf, y=y4, acc_out=acc, stream=stream))
            del copies, Wq

        for kind, M, label, kern in ((wsgemv.W4A16, 1, "c5_M1", "w4_grouped_kernel<1, 8, true, 0"),
                                     (wsgemv.W4A16, 4, "c5_M4", "w4_grouped_kernel<2, 4, true, 1"),
                                     (wsgemv.W4A16, 8, "c5_M8", "w4_grouped_kernel<2, 4, true, 1"),
                                     (wsgemv.W4A8, 1, "c6", "w4_grouped_kernel<1, 4, true, 2")):
            w4 = synth.decode_step_w4(workload=5, M=M)
            sets = [[], []]
            b = 0
            for name, Wc, s4, X in w4:
                N, K = Wc.shape[0], Wc.shape[1] * 8
                Xd = torch.from_numpy(X if kind == wsgemv.W4A16 else X.reshape(K)).to(dev)
                yw = torch.empty((M, N) if kind == wsgemv.W4A16 else (N,), device=dev)
                for c in sets:
                    Wp, Sp = wsgemv.pack_w4(torch.from_numpy(Wc.view(np.int32)).to(dev), torch.from_numpy(s4).to(dev),
                                            stream=stream)
                    c.append(wsgemv.Linear(kind, Wp, Xd, yw, N, K, M=M, scale=Sp, group=128))
                b += Wc.nbytes + s4.nbytes + X.nbytes + M * N * 4
            del w4
            sts = [wsgemv.DecodeStep(c, wsgemv.STEP_GROUPED, stream=stream) for c in sets]
            what = f"C5 W4A16 step, M = {M}" if kind == wsgemv.W4A16 else "C6 W4A8 step, M = 1"
            run(label, what + " (2 packed copies)", [kern], 6, b, lambda i: sts[i % 2](stream))
            for st in sts:
                st.close()
            del sets
    torch.cuda.synchronize()
    with open(args.counter_pass, "w") as f:
        json.dump({"calibration": {"label": "calibration", "read_bytes": 1 << 30, "write_bytes": 1 << 30},
                   "configs": configs}, f, indent=1)
    log(f"manifest written: {args.counter_pass}")


def chain_trace(args, torch, synth, wsgemv, profsum, dev, stream):
    """The C3 linears as one dependent chain (each reads the leading K entries
    of the previous linear's fp16 output, as in the chain extras), one
    persistent launch per step: time untraced steps, trace one step per work
    unit, and write where the stage time goes."""
    step_in = synth.decode_step_f16(workload=3)
    cl, names, x = [], [], torch.from_numpy(step_in[0][2]).to(dev)
    for name, W, _ in step_in:
        N, K = W.shape
        y16 = torch.empty(N, dtype=torch.float16, device=dev)
        cl.append(wsgemv.Linear(wsgemv.F16, torch.from_numpy(W).to(dev), x[:K], torch.empty(N, device=dev), N, K,
                                y16=y16))
        names.append(f"{name} {N}x{K}")
        x = y16
    pc = wsgemv.DecodeStep(cl, wsgemv.STEP_PERSISTENT, stream=stream)
    for _ in range(5):
        pc(stream)
    step_us = statistics.median(region_time(torch, lambda i: pc(stream), 20, stream) for _ in range(3)) * 1e3
    units = pc.info()[1]
    buf = torch.zeros(4 * units, dtype=torch.int64, device=dev)
    pc.set_trace(buf)
    pc(stream)  # one traced step to warm up, then the one kept
    traced_us = event_times(torch, lambda i: pc(stream), 1, stream)[0] * 1e3
    pc.set_trace(None)
    give_ups = pc.give_ups(stream)
    words = [int(v) & 0xFFFFFFFFFFFFFFFF for v in buf.cpu().tolist()]
    pc.close()
    stats = profsum.chain_trace_stats(words)
    cmd = f"python bench.py --chain-trace {args.chain_trace}"
    notes = [f"Waits that gave up in the traced steps: {give_ups}."]
    with open(args.chain_trace, "w") as f:
        f.write(profsum.render_chain_trace(stats, names, cmd, step_us, traced_us, notes))
    log(f"chain trace: {stats['units']} units, step {step_us:.1f} us untraced, {traced_us:.1f} us traced; "
        f"median stage {stats['median_stage']['stage_us']:.2f} us; written {args.chain_trace}")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "the library runs on exactly one GPU: the batch-1 GEMV is measured on one "
                                   "MI355X and no multi-GPU path exists; rerun with --gpus 1"}))
        sys.exit(2)

    import torch
    from weight_streaming_gemv_decode_amd import synth, wsgemv
    wsgemv.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)

    if args.counter_pass:
        counter_pass(args, torch, synth, wsgemv, dev, stream)
        return

    if args.chain_trace:
        from weight_streaming_gemv_decode_amd import profsum
        chain_trace(args, torch, synth, wsgemv, profsum, dev, stream)
        return

    if args.calib_copy:
        # plain copy of known size for the profiler's byte counters
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---- inputs (seeded, synthetic), copied to HBM once ----
    t0 = time.time()
    step_in = synth.decode_step_f16(workload=3)
    lins = []
    for name, W, x in step_in:
        N, K = W.shape
        lins.append(wsgemv.Linear(wsgemv.F16, torch.from_numpy(W).to(dev), torch.from_numpy(x).to(dev),
                                  torch.empty(N, dtype=torch.float32, device=dev), N, K))
    torch.cuda.synchronize()
    w_bytes = sum(W.nbytes for _, W, _ in step_in)
    x_bytes = sum(x.nbytes for _, _, x in step_in)
    y_bytes = sum(W.shape[0] * 4 for _, W, _ in step_in)
    step_bytes = w_bytes + x_bytes + y_bytes
    log(f"inputs ready in {time.time() - t0:.1f}s: {len(lins)} linears, {step_bytes} algorithmic bytes/step")

    # ---- the timed configuration: the GROUPED plan (one launch over a work table;
    # a single launch is cheaper than a one-node graph launch, so it is direct) ----
    with torch.cuda.stream(stream):
        step = wsgemv.DecodeStep(lins, wsgemv.STEP_GROUPED, stream=stream)
        for _ in range(args.warmup):
            step(stream)
    # HIP events on the plan's stream bracket the timed region: the grouped
    # kernel is the step's only launch, so their interval / K is its average
    # launch duration (back-to-back launches, nothing recorded in between)
    ev_start = torch.cuda.Event(enable_timing=True)
    ev_end = torch.cuda.Event(enable_timing=True)
    stream.synchronize()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    with torch.cuda.stream(stream):
        ev_start.record(stream)
        for _ in range(args.steps):
            step(stream)
        ev_end.record(stream)
    stream.synchronize()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"GROUPED plan (graph={step.uses_graph()}): {ms_per_step * 1e3:.1f} us/step, {value:.0f} GB/s")
    launch_avg_ms = ev_start.elapsed_time(ev_end) / args.steps
    launches, units = step.info()
    achieved = step_bytes / (launch_avg_ms * 1e-3) / 1e9

    # the distribution of single launches (an event after each launch adds a
    # little to every interval), on the same stream
    eager = wsgemv.DecodeStep(lins, wsgemv.STEP_GROUPED | wsgemv.STEP_EAGER, stream=stream)
    kt = event_times(torch, lambda i: eager(stream), max(50, min(args.steps, 200)), stream)
    ks = summary(kt)
    rec = measured_traffic(args.traffic)
    traffic = None if rec is None else rec["bytes"]
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel": "dense_grouped_kernel<f16> (one launch per step)",
                "bytes_per_launch": step_bytes,
                "launch_avg_ms": launch_avg_ms,
                "launch_avg_source": f"HIP events on the kernel's stream around the {args.steps} timed launches",
                "single_launch_ms": ks,
                "traffic_detail": None if rec is None else {k: rec[k] for k in ("read_bytes", "write_bytes",
                                                                               "ratio_to_algorithmic")}}
    log(f"grouped kernel: {launch_avg_ms * 1e3:.1f} us per launch over the timed region -> {achieved:.0f} GB/s "
        f"(single launches: median {ks['median_ms'] * 1e3:.1f} us)")
    if not args.no_extras:
        # like for like: the probe is timed with an event after each launch too, and again back to back
        roofline["attainable_same_size"] = attainable(torch, wsgemv, step_bytes, ks["mean_ms"] * 1e3, stream,
                                                      back_to_back_us=launch_avg_ms * 1e3)
        log(f"read probe over the same bytes: {roofline['attainable_same_size']}")

    extras = {"timing": "us / us_per_step: calls back to back on one stream with events around them (or host "
                        "time, or a captured graph where stated); single_launch_median_us: an event after each "
                        "call, which adds a few us to every interval"}
    only = set(filter(None, args.only.split(",")))
    want = (lambda k: (not args.no_extras) and (not only or k in only))

    if want("graph"):
        # the same GROUPED plan forced into a one-node hipGraph: a graph launch
        # costs more than the one direct launch the plan uses
        fg = wsgemv.DecodeStep(lins, wsgemv.STEP_GROUPED | wsgemv.STEP_FORCE_GRAPH, stream=stream)
        for _ in range(5):
            fg(stream)
        stream.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            for _ in range(args.steps):
                fg(stream)
        stream.synchronize()
        t = (time.perf_counter() - t0) * 1e6 / args.steps
        extras["c3_grouped_forced_graph"] = {"us_per_step": round(t, 2),
                                             "GBps": round(step_bytes / (t * 1e-6) / 1e9, 1)}
        fg.close()

    if want("ordered"):
        o = wsgemv.DecodeStep(lins, wsgemv.STEP_ORDERED, stream=stream)
        for _ in range(3):
            o(stream)
        s = summary(event_times(torch, lambda i: o(stream), 50, stream))
        t = region_time(torch, lambda i: o(stream), 50, stream)
        extras["c3_ordered_graph"] = {"us": t * 1e3, "GBps": step_bytes / (t * 1e-3) / 1e9,
                                      "single_launch_median_us": s["median_ms"] * 1e3, "launches": o.info()[0]}
        o.close()

    if want("chain"):
        # the same 113 linears as one dependent chain: every linear reads the
        # leading K entries of the previous linear's fp16 output (y16), which
        # stands in for the attention / activation glue between them; the
        # ORDERED plan (one graph) runs them in order
        y16s, cl = [], []
        x = lins[0].x
        for l in lins:
            y16 = torch.empty(l.N, dtype=torch.float16, device=dev)
            cl.append(wsgemv.Linear(l.kind, l.W, x[:l.K], torch.empty(l.N, device=dev), l.N, l.K, y16=y16))
            y16s.append(y16)
            x = y16
        ch = wsgemv.DecodeStep(cl, wsgemv.STEP_ORDERED, stream=stream)
        for _ in range(3):
            ch(stream)
        s = summary(event_times(torch, lambda i: ch(stream), 50, stream))
        t = region_time(torch, lambda i: ch(stream), 50, stream)
        extras["c3_dependent_chain_ordered_graph"] = {
            "us": t * 1e3, "GBps": step_bytes / (t * 1e-3) / 1e9, "single_launch_median_us": s["median_ms"] * 1e3,
            "launches": ch.info()[0],
            "note": "each linear's x is the leading K entries of the previous linear's fp16 output"}
        ch.close()
        # the same chain as one persistent cooperative launch per step: each
        # unit's weight loads go out before its input is ready, inputs are
        # handed over as tagged fp16 words
        pc = wsgemv.DecodeStep(cl, wsgemv.STEP_PERSISTENT, stream=stream)
        for _ in range(3):
            pc(stream)
        s = summary(event_times(torch, lambda i: pc(stream), 50, stream))
        t = region_time(torch, lambda i: pc(stream), 50, stream)
        extras["c3_dependent_chain_persistent"] = {
            "us": t * 1e3, "GBps": step_bytes / (t * 1e-3) / 1e9, "single_launch_median_us": s["median_ms"] * 1e3,
            "launches": pc.info()[0], "work_units": pc.info()[1], "give_ups": pc.give_ups(stream),
            "note": "the same dependent chain, one cooperative launch per step (WSG_STEP_PERSISTENT)"}
        pc.close()
        del y16s, cl

    if want("token"):
        # the timed step with the lm_head also taking the greedy token
        tok = torch.empty(1, dtype=torch.int32, device=dev)
        tl = [wsgemv.Linear(l.kind, l.W, l.x, l.y, l.N, l.K) for l in lins[:-1]]
        lm = lins[-1]
        tl.append(wsgemv.Linear(lm.kind, lm.W, lm.x, lm.y, lm.N, lm.K, argmax_idx=tok))
        st = wsgemv.DecodeStep(tl, wsgemv.STEP_GROUPED, stream=stream)
        for _ in range(5):
            st(stream)
        s = summary(event_times(torch, lambda i: st(stream), 100, stream))
        t = region_time(torch, lambda i: st(stream), 100, stream)
        extras["c3_step_with_token"] = {"us": t * 1e3, "GBps": step_bytes / (t * 1e-3) / 1e9,
                                        "single_launch_median_us": s["median_ms"] * 1e3}
        st.close()

    if want("c2"):
        lm = lins[-1]
        Wcopy = lm.W.clone()
        Ws = [lm.W, Wcopy]
        b = lm.N * lm.K * 2 + lm.K * 2 + lm.N * 4
        res = {}
        for S in (0, 1, 2):
            ws = wsgemv.workspace(wsgemv.F16, 1, lm.N, lm.K, S, dev)
            y = torch.empty(lm.N, device=dev)
            fn = lambda i: wsgemv.gemv_f16(Ws[i % 2], lm.x, y=y, splits=S, ws=ws, stream=stream)  # noqa: E731
            for i in range(10):
                fn(i)
            s = summary(event_times(torch, fn, 100, stream))
            t = region_time(torch, fn, 100, stream)
            res[f"S={S if S else wsgemv.plan_splits(0, 1, lm.N, lm.K)}{' (auto)' if S == 0 else ''}"] = {
                "us": t * 1e3, "GBps": b / (t * 1e-3) / 1e9, "pct_peak": 100 * b / (t * 1e-3) / 1e9 / PEAK_HBM_GBS,
                "single_launch_median_us": s["median_ms"] * 1e3}
        res["S=2"]["note"] = "split-K; the last workgroup of each row tile adds the two partials (no reduce kernel)"
        # ablation: the same split summed by a second, reduce kernel (same bits)
        wsgemv.tune_set("split_fuse", 0)
        try:
            ws = wsgemv.workspace(wsgemv.F16, 1, lm.N, lm.K, 2, dev)
            y = torch.empty(lm.N, device=dev)
            fn = lambda i: wsgemv.gemv_f16(Ws[i % 2], lm.x, y=y, splits=2, ws=ws, stream=stream)  # noqa: E731
            for i in range(10):
                fn(i)
            t = region_time(torch, fn, 100, stream)
        finally:
            wsgemv.tune_set("split_fuse", -1)
        res["S=2 reduce kernel"] = {"us": t * 1e3, "GBps": b / (t * 1e-3) / 1e9,
                                    "pct_peak": 100 * b / (t * 1e-3) / 1e9 / PEAK_HBM_GBS}
        # the same lm_head with the greedy token fused into the kernel that writes the logits
        tok = torch.empty(1, dtype=torch.int32, device=dev)
        ws = wsgemv.workspace(wsgemv.F16 | wsgemv.WITH_ARGMAX, 1, lm.N, lm.K, 0, dev)
        y = torch.empty(lm.N, device=dev)
        fn = lambda i: wsgemv.gemv_f16_argmax(Ws[i % 2], lm.x, y=y, token=tok, ws=ws, stream=stream)  # noqa: E731
        for i in range(10):
            fn(i)
        s = summary(event_times(torch, fn, 100, stream))
        t = region_time(torch, fn, 100, stream)
        res["with_token"] = {"us": t * 1e3, "GBps": b / (t * 1e-3) / 1e9,
                             "pct_peak": 100 * b / (t * 1e-3) / 1e9 / PEAK_HBM_GBS,
                             "single_launch_median_us": s["median_ms"] * 1e3,
                             "note": "the GEMV writing one key per workgroup, then the one-workgroup finish kernel"}
        # like for like: the probe is timed with an event after each launch, and again back to back
        res["attainable_same_size"] = attainable(torch, wsgemv, b, res["S=1"]["single_launch_median_us"], stream,
                                                 back_to_back_us=res["S=1"]["us"])
        res["timing"] = ("us: calls back to back with events around 100 of them; single_launch_median_us: "
                         "an event after each call")
        extras["c2_lm_head_248320x1024"] = {"bytes": b, "rotation": "2 weight copies (1.02 GB)", **res}
        del Wcopy

    if want("c1"):
        N, K = synth.C1_SHAPE
        W = torch.from_numpy(synth.f16_normal(1, 0, (N, K), synth.W_SIGMA)).to(dev)
        x = torch.from_numpy(synth.f16_normal(1, 1, (K,), synth.X_SIGMA)).to(dev)
        copies = [W] + [W.clone() for _ in range(63)]
        ws = wsgemv.workspace(wsgemv.F16, 1, N, K, 0, dev)
        y = torch.empty(N, device=dev)
        fn = lambda i: wsgemv.gemv_f16(copies[i % 64], x, y=y, ws=ws, stream=stream)  # noqa: E731
        s = summary(graph_times(torch, fn, 64, 10, stream))
        b = N * K * 2 + K * 2 + N * 4
        extras["c1_2048x2048"] = {"bytes": b, "median_us": s["median_ms"] * 1e3,
                                  "GBps": b / (s["median_ms"] * 1e-3) / 1e9, "rotation": "64 copies (537 MB)",
                                  "note": "64 calls captured in one graph, per-call time; launch-bound shape",
                                  "attainable_same_size": attainable(torch, wsgemv, b, s["median_ms"] * 1e3, stream,
                                                                     graph_inner=64)}
        del copies

    if want("c4"):
        for (N, K) in synth.C4_SHAPES:
            Wq = torch.from_numpy(synth.int8_uniform(4, 0, (N, K))).to(dev)
            xq = torch.from_numpy(synth.int8_uniform(4, 1, (K,))).to(dev)
            sw = torch.from_numpy(synth.f32_uniform(4, 2, (N,), 0.001, 0.01)).to(dev)
            xs = torch.tensor([synth.X_SCALE_W8A8], device=dev)
            copies = [Wq] + [Wq.clone() for _ in range(8)]
            ws = wsgemv.workspace(wsgemv.W8A8, 1, N, K, 0, dev)
            y = torch.empty(N, device=dev)
            acc = torch.empty(N, dtype=torch.int32, device=dev)
            fn = lambda i: wsgemv.gemv_w8a8(copies[i % 9], sw, xq, xs, y=y, acc_out=acc, ws=ws,  # noqa: E731
                                            stream=stream)
            s = summary(graph_times(torch, fn, 36, 10, stream))
            b = N * K + N * 4 + K + N * 4 + N * 4
            extras[f"c4_w8a8_{N}x{K}"] = {"bytes_incl_acc_out": b, "median_us": s["median_ms"] * 1e3,
                                          "GBps": b / (s["median_ms"] * 1e-3) / 1e9,
                                          "splits": wsgemv.plan_splits(1, 1, N, K),
                                          "rotation": "9 copies, 36 calls captured in one graph",
                                          "attainable_same_size": attainable(torch, wsgemv, b, s["median_ms"] * 1e3,
                                                                             stream, graph_inner=36)}
            # the same weights with fp16 activations quantised per token in the kernel
            xf = torch.from_numpy(synth.f16_normal(4, 3, (K,), synth.X_SIGMA)).to(dev)
            wsd = wsgemv.workspace(wsgemv.W8A8_DYN, 1, N, K, 0, dev)
            fn = lambda i: wsgemv.gemv_w8a8_dyn(copies[i % 9], sw, xf, y=y, acc_out=acc, ws=wsd,  # noqa: E731
                                                stream=stream)
            s = summary(graph_times(torch, fn, 36, 10, stream))
            b = N * K + N * 4 + 2 * K + N * 4 + N * 4
            extras[f"c4_w8a8_dyn_{N}x{K}"] = {"bytes_incl_acc_out": b, "median_us": s["median_ms"] * 1e3,
                                              "GBps": b / (s["median_ms"] * 1e-3) / 1e9,
                                              "note": "fp16 x quantised per token inside every work unit",
                                              "attainable_same_size": attainable(torch, wsgemv, b,
                                                                                 s["median_ms"] * 1e3, stream,
                                                                                 graph_inner=36)}
            del copies

    def w4_step_extra(kind, M, label):
        """The int4 step (113 linears, one GROUPED launch) over two packed
        weight copies alternated between calls (630 MB, past the 256 MB
        Infinity Cache): direct launch and forced one-node graph."""
        w4 = synth.decode_step_w4(workload=5, M=M)
        copies = [[], []]
        b = 0
        for name, Wc, s4, X in w4:
            N, K = Wc.shape[0], Wc.shape[1] * 8
            Xd = torch.from_numpy(X if kind == wsgemv.W4A16 else X.reshape(K)).to(dev)
            y = torch.empty((M, N) if kind == wsgemv.W4A16 else (N,), device=dev)
            for c in copies:
                Wp, Sp = wsgemv.pack_w4(torch.from_numpy(Wc.view(np.int32)).to(dev), torch.from_numpy(s4).to(dev))
                c.append(wsgemv.Linear(kind, Wp, Xd, y, N, K, M=M, scale=Sp, group=128))
            b += Wc.nbytes + s4.nbytes + X.nbytes + M * N * 4
        del w4
        torch.cuda.synchronize()
        rec = {"bytes": b, "rotation": "2 packed weight copies (630 MB)"}
        for tag, mode in (("launch", wsgemv.STEP_GROUPED), ("forced_graph", wsgemv.STEP_GROUPED | wsgemv.STEP_FORCE_GRAPH)):
            sts = [wsgemv.DecodeStep(c, mode, stream=stream) for c in copies]
            for i in range(6):
                sts[i % 2](stream)
            s = summary(event_times(torch, lambda i: sts[i % 2](stream), 100, stream))
            t = region_time(torch, lambda i: sts[i % 2](stream), 100, stream)
            rec[tag] = {"us": t * 1e3, "GBps": b / (t * 1e-3) / 1e9, "pct_peak": 100 * b / (t * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "single_launch_median_us": s["median_ms"] * 1e3}
            for st in sts:
                st.close()
        # like for like: the probe is timed with an event after each launch, and again back to back
        rec["attainable_same_size"] = attainable(torch, wsgemv, b, rec["launch"]["single_launch_median_us"], stream,
                                                 back_to_back_us=rec["launch"]["us"])
        rec["timing"] = ("us: steps back to back with events around 100 of them; single_launch_median_us: "
                         "an event after each step")
        extras[label] = rec
        del copies

    if want("c5"):
        for M in (1, 4, 8):
            w4_step_extra(wsgemv.W4A16, M, f"c5_w4a16_step_M{M}")

    if want("c6"):
        # the same int4 weights with per-token int8 activations (W4A8), M = 1
        w4_step_extra(wsgemv.W4A8, 1, "c6_w4a8_step_M1")

    if want("conv"):
        # causal-conv1d decode step over a 2048-channel qkv output, W = 4, SiLU:
        # standalone (64 calls in one graph), and fused into the 28 qkv linears of the step
        C, W = 2048, 4
        r = synth.rng(6, 0)
        cw = torch.from_numpy(r.normal(0, 0.5, (C, W)).astype(np.float16)).to(dev)
        cb = torch.from_numpy(r.normal(0, 1, C).astype(np.float32)).to(dev)
        xs_ = [torch.from_numpy(r.normal(0, 1, C).astype(np.float32)).to(dev) for _ in range(64)]
        st = torch.zeros((C, W - 1), device=dev)
        out = torch.empty(C, device=dev)
        fn = lambda i: wsgemv.causal_conv1d_step(xs_[i % 64], cw, st, bias=cb, out=out, silu=True,  # noqa: E731
                                                 stream=stream)
        s = summary(graph_times(torch, fn, 64, 10, stream))
        b = C * 4 + C * W * 2 + C * 4 + 2 * C * (W - 1) * 4 + C * 4
        rec = {"standalone_C2048_W4": {"bytes": b, "median_us": s["median_ms"] * 1e3,
                                       "note": "64 calls captured in one graph, per-call time; latency-bound"}}
        states, outs, tl = [], [], []
        for l in lins:
            kw = {}
            if l.N == 2048 and l.K == 1024:      # the qkv linears
                states.append(torch.zeros((l.N, W - 1), device=dev))
                outs.append(torch.empty(l.N, device=dev))
                kw = dict(conv_w=cw, conv_bias=cb, conv_state=states[-1], conv_out=outs[-1], conv_silu=True)
            tl.append(wsgemv.Linear(l.kind, l.W, l.x, l.y, l.N, l.K, **kw))
        st_ = wsgemv.DecodeStep(tl, wsgemv.STEP_GROUPED, stream=stream)
        for _ in range(5):
            st_(stream)
        s2 = summary(event_times(torch, lambda i: st_(stream), 100, stream))
        t2 = region_time(torch, lambda i: st_(stream), 100, stream)
        rec["c3_step_with_28_fused_convs"] = {"us": t2 * 1e3, "GBps": step_bytes / (t2 * 1e-3) / 1e9,
                                              "single_launch_median_us": s2["median_ms"] * 1e3}
        st_.close()
        extras["conv1d"] = rec

    if want("shard"):
        # One GPU's share of the step spread over G = 8 GPUs, timed like C3
        # (GROUPED, one launch; three weight copies rotated past the 256 MB
        # Infinity Cache), for two cuts of the decoder linears: Megatron
        # pairs (qkv and gate+up over N, o and down over K, whose partial
        # sums would be all-reduced), and every linear over N (outputs would
        # be all-gathered).  The lm_head is cut over the vocabulary.
        G = 8
        cuts = {"pairs": {"qkv": (G, 1), "o": (1, G), "gate_up": (G, 1), "down": (1, G)},
                "rows": {"qkv": (G, 1), "o": (G, 1), "gate_up": (G, 1), "down": (G, 1)}}
        rec = {"G": G, "note": "per-GPU product only; the collectives are not run"}
        for label, cut in cuts.items():
            shapes = []
            for name, N, K, wi, xi in synth.decode_step_shapes():
                if name == "lm_head":
                    shapes.append((name, N // G, K, wi, xi))
                else:
                    dn, dk = cut[name.split(".")[1]]
                    shapes.append((name, N // dn, K // dk, wi, xi))
            b = sum(N * K * 2 + K * 2 + N * 4 for _, N, K, _, _ in shapes)
            sets = []
            for c in range(3):
                lins_g = []
                for name, N, K, wi, xi in shapes:
                    Wg = torch.from_numpy(synth.f16_normal(8, 4 * wi + c, (N, K), synth.W_SIGMA)).to(dev)
                    xg = torch.from_numpy(synth.f16_normal(9, xi, (K,), synth.X_SIGMA)).to(dev)
                    lins_g.append(wsgemv.Linear(wsgemv.F16, Wg, xg, torch.empty(N, device=dev), N, K))
                sets.append(wsgemv.DecodeStep(lins_g, wsgemv.STEP_GROUPED, stream=stream))
            for i in range(6):
                sets[i % 3](stream)
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                ev0.record(stream)
                for i in range(60):
                    sets[i % 3](stream)
                ev1.record(stream)
            stream.synchronize()
            t = ev0.elapsed_time(ev1) * 1e3 / 60
            layer = ", ".join(f"{n.split('.')[1]} {N}x{K}" for n, N, K, _, _ in shapes[:4])
            rec[f"step_{label}"] = {"bytes_per_gpu": b, "step_us": round(t, 2),
                                    "GBps": round(b / (t * 1e-6) / 1e9, 1),
                                    "shapes": f"{layer} (x28), lm_head {shapes[-1][1]}x{shapes[-1][2]}"}
            for st in sets:
                st.close()
            del sets
        # the lm_head shard alone, 8 rotated copies in one graph
        N, K = synth.LMHEAD[0] // G, synth.LMHEAD[1]
        W = torch.from_numpy(synth.f16_normal(10, 0, (N, K), synth.W_SIGMA)).to(dev)
        copies = [W] + [W.clone() for _ in range(7)]
        x = torch.from_numpy(synth.f16_normal(10, 1, (K,), synth.X_SIGMA)).to(dev)
        y = torch.empty(N, device=dev)
        fn = lambda i: wsgemv.gemv_f16(copies[i % 8], x, y=y, stream=stream)  # noqa: E731
        s = summary(graph_times(torch, fn, 32, 10, stream))
        bl = N * K * 2 + K * 2 + N * 4
        rec["lm_head_31040x1024"] = {"bytes": bl, "median_us": round(s["median_ms"] * 1e3, 2),
                                     "GBps": round(bl / (s["median_ms"] * 1e-3) / 1e9, 1),
                                     "rotation": "8 copies, 32 calls captured in one graph"}
        extras["shard_8way_one_gpu"] = rec
        del copies

    if want("topk"):
        # top-k over the lm_head's 248,320 fp32 logits (64 calls captured in one graph)
        N = synth.LMHEAD[0]
        r = synth.rng(7, 0)
        ys = [torch.from_numpy(r.normal(0, 1, N).astype(np.float32)).to(dev) for _ in range(4)]
        rec = {}
        for k in (1, 8, 50):
            idx = torch.empty(k, dtype=torch.int32, device=dev)
            ws = torch.empty(max(256, wsgemv.lib().wsg_topk_ws_bytes(N, k)), dtype=torch.uint8, device=dev)
            fn = lambda i: wsgemv.topk_f32(ys[i % 4], k, idx=idx, ws=ws, stream=stream)  # noqa: E731
            s = summary(graph_times(torch, fn, 64, 10, stream))
            rec[f"k={k}"] = {"median_us": round(s["median_ms"] * 1e3, 2)}
        tok = torch.empty(1, dtype=torch.int32, device=dev)
        aws = torch.empty(wsgemv.ARGMAX_WS_BYTES, dtype=torch.uint8, device=dev)
        fn = lambda i: wsgemv.argmax_f32(ys[i % 4], token=tok, ws=aws, stream=stream)  # noqa: E731
        s = summary(graph_times(torch, fn, 64, 10, stream))
        rec["argmax_f32 (for comparison)"] = {"median_us": round(s["median_ms"] * 1e3, 2)}
        extras["topk_248320_logits"] = rec

    if want("probe"):
        # attainable streaming-read rate against transfer size (back-to-back launches)
        rec = {}
        for mb in (128, 512, 2048):
            t = probe_same_size(torch, wsgemv, mb << 20, stream, reps=20)
            rec[f"{mb}MiB"] = {"median_us": round(t, 2), "GBps": round((mb << 20) / (t * 1e-6) / 1e9, 1)}
        extras["hbm_read_probe"] = rec

    # ---- counter-measured HBM traffic of each extra (while its kernel sources are unchanged) ----
    recs = measured_traffic_all(args.traffic) or {}

    def attach(entry, label):
        r = recs.get(label)
        if entry is not None and r is not None:
            entry["traffic"] = {"bytes_per_step": r["bytes"], "ratio_to_algorithmic": r["ratio_to_algorithmic"],
                                "read_bytes": r["read_bytes"], "write_bytes": r["write_bytes"]}
    c2 = extras.get("c2_lm_head_248320x1024", {})
    attach(c2.get("S=1") or c2.get("S=1 (auto)"), "c2_S1")
    attach(c2.get("S=2"), "c2_S2")
    attach(extras.get("c1_2048x2048"), "c1")
    for tag, (N, K) in zip("ab", synth.C4_SHAPES):
        attach(extras.get(f"c4_w8a8_{N}x{K}"), f"c4{tag}_w8a8")
        attach(extras.get(f"c4_w8a8_dyn_{N}x{K}"), f"c4{tag}_w8a8_dyn")
    for M in (1, 4, 8):
        attach(extras.get(f"c5_w4a16_step_M{M}"), f"c5_M{M}")
    attach(extras.get("c6_w4a8_step_M1"), "c6")
    attach(extras.get("c3_dependent_chain_persistent"), "c3_chain_persistent")

    # ---- CPU oracle on the host cores, same step inputs ----
    cpu = None
    if not args.no_cpu:
        import oracle
        cores = len(os.sched_getaffinity(0))
        oracle.set_threads(cores)
        # whole decode steps, repeated until about 10 s of CPU work (at least 2 steps, at most 60)
        t1 = time.perf_counter()
        n_cpu = 0
        while n_cpu < 60 and (n_cpu < 2 or time.perf_counter() - t1 < 10.0):
            for _, W, x in step_in:
                oracle.gemv_f16(W, x)
            n_cpu += 1
        dt = (time.perf_counter() - t1) / n_cpu
        cpu = {"value": round(step_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "ms_per_step": round(dt * 1e3, 1),
               "sample": f"{n_cpu} full decode steps (all 113 GEMVs, 1.22 GB each) through the fp64 C oracle, "
                         f"OpenMP over rows on {cores} threads ({platform.processor() or platform.machine()})"}
        log(f"oracle: {dt:.2f}s/step on {cores} threads over {n_cpu} steps")
        # the same oracle on one thread: one whole step (a few seconds)
        oracle.set_threads(1)
        t1 = time.perf_counter()
        for _, W, x in step_in:
            oracle.gemv_f16(W, x)
        dt1 = time.perf_counter() - t1
        oracle.set_threads(cores)
        cpu["single_thread"] = {"value": round(step_bytes / dt1 / 1e9, 3), "unit": "GB/s",
                                "ms_per_step": round(dt1 * 1e3, 1), "sample": "1 full decode step on 1 thread"}
        log(f"oracle: {dt1:.2f}s/step on 1 thread")
        cpu["cpu_model"] = cpu_model()
        cpu["sample"] = cpu["sample"].replace(f"({platform.processor() or platform.machine()})",
                                              f"({cpu['cpu_model']})")
        if not args.no_extras:
            cpu["per_config"] = oracle_per_config(oracle, synth, step_in, cores)
        oracle.set_threads(cores)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic: seeded fp16 weights ~N(0,0.02), activations ~N(0,1); fp32 accumulate, fp32 outputs",
        "config": {"workload": "fp16 batch-1 decode-step linear stream: 28 x {qkv 2048x1024, o 1024x1024, "
                               "gate_up 6144x1024, down 1024x3072} + lm_head 248320x1024, GROUPED plan: "
                               f"one launch over a work table of {units:,} units (ORDERED, one node per "
                               "linear, is the captured hipGraph in extras)",
                   "bytes_per_step": step_bytes, "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
                   "launches_per_step": launches, "work_units": units},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(line))
    step.close()
    eager.close()


if __name__ == "__main__":
    main()
