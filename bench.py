#!/usr/bin/env python3
"""Benchmark: Effort approximate matvec on one MI355X.

Workload: W 4096 x 14336 fp16 (in x out, Mistral-7B w1/w3 shape) ~ N(0, 0.02),
v ~ 0.5 Student-t(3) fp32, effort 0.25, batch 1, P = 16 probes per row,
seeded synthetic data.  A step is one effort_matvec call: cutoff kernel,
dispatch kernel and the bucketMul stream with its flush.

Timing:
  * every timed loop cycles over R distinct device copies of the layout (and R
    vectors), R chosen so a cycle touches >= 1 GiB, so the 256 MB last-level
    cache cannot serve repeats; the dense comparator cycles over its own copies;
  * C calls (at least 64, and at least one whole cycle) are captured once in a
    HIP graph and the graph is replayed; the dense comparator's graph holds the
    same C calls, so the per-replay launch cost weighs on both paths alike;
    hipEvents on the replay stream bracket the timed region;
  * each kernel's own duration comes from a hipEvent pair that the runtime
    stamps with that kernel's begin and end (effort_matvec_timed, launched with
    hipExtLaunchKernelGGL), in eager calls queued behind graph replays.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs/matvec + HBM GB/s at effort 0.25, 4096×14336 fp16; speedup vs dense GEMV"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
COUNTERS = os.path.join(ROOT, "profiles", "counters_bucketmul_4096x14336_e0.25.txt")
KERNEL_SRC = os.path.join(ROOT, "dynamic_sparsity_approximate_amd", "csrc", "kernels.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--m", type=int, default=4096)
    ap.add_argument("--n", type=int, default=14336)
    ap.add_argument("--effort", type=float, default=0.25)
    ap.add_argument("--P", type=int, default=16)
    ap.add_argument("--groups", type=int, default=0)
    ap.add_argument("--format", choices=["u32", "r12", "q8"], default="r12",
                    help="entry format of the layout: r12 (3 bytes per entry, the default), u32 "
                         "(4 bytes) or q8 (2 bytes, the Q8 bucketed weights: the product of the "
                         "quantized matrix)")
    ap.add_argument("--crop", type=int, default=0, help="stored segments per row (0: all)")
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--graph-calls", type=int, default=64,
                    help="calls captured per graph, the same for the effort path and the dense "
                         "GEMV, so that the per-replay launch cost weighs on both alike")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=["full", "effort", "dense", "copy", "sweep", "batched",
                                       "decode", "moe", "moetraffic", "mallcheck"], default="full",
                    help="effort/dense: time only that path (for profiler runs); copy: plain "
                         "1 GiB device copies for counter calibration; sweep: the four "
                         "Mistral-7B shapes at efforts 1/.5/.25/.125; batched: b = 1..16 "
                         "vectors against the dense small GEMM; decode: a whole Mistral-7B-"
                         "shaped decode step; moe: a Mixtral-shaped expert block; moetraffic: "
                         "a few tokens of the grouped expert block and the kept bytes of their "
                         "six matvecs (for a FETCH_SIZE counter run); mallcheck: "
                         "kernel times with layout rotation, after a cache-evicting write, and warm")
    ap.add_argument("--layers", type=int, default=32, help="decode mode: decoder layers")
    ap.add_argument("--streams", type=int, default=6,
                    help="decode/moe modes: side streams for matvecs that do not depend on "
                         "each other (0: one stream)")
    return ap.parse_args()


def layout_opts(args, E) -> dict:
    """EffortMatrix options of the --format / --crop / --groups flags."""
    return {"entry_format": format_code(args.format, E), "crop": args.crop, "groups": args.groups}


def format_code(fmt: str, E) -> int:
    return {"u32": E.EFFORT_ENTRY_U32, "r12": E.EFFORT_ENTRY_R12, "q8": E.EFFORT_ENTRY_Q8}[fmt]


def entry_bytes(fmt: str) -> float:
    """Bytes the method reads per kept entry in this layout format."""
    return {"u32": 4.0, "r12": 3.0, "q8": 2.0}[fmt]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernels_sha():
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def read_counters(fmt: str):
    """HBM traffic of the bucketMul kernel from the committed rocprofv3 --pmc summary,
    or None if it is missing, was taken on a different kernels.hip or on another
    entry format."""
    if not os.path.exists(COUNTERS):
        return None
    kv = {}
    for line in open(COUNTERS):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernels_sha256") != kernels_sha() or kv.get("entry_format") != fmt:
        return None
    try:
        return float(kv["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def host_info():
    info = {"nproc": os.cpu_count()}
    try:
        out = subprocess.run(["lscpu"], stdout=subprocess.PIPE, text=True).stdout
        for line in out.splitlines():
            if line.startswith("Model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
    except OSError:
        pass
    return info


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def time_replays(torch, g, reps):
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b), (time.perf_counter() - t0) * 1e3


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import dynamic_sparsity_approximate_amd as E
    import synth

    dev = torch.device("cuda:0")
    m, n, P, effort = args.m, args.n, args.P, args.effort
    GiB = float(1 << 30)

    if args.mode == "copy":
        x = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes_per_copy": 1 << 30, "copies": 5}))
        return

    if args.mode in EXTRA_MODES:
        EXTRA_MODES[args.mode](args, torch, np, E, synth, dev)
        return

    log("generating W %dx%d and converting" % (m, n))
    W = synth.matrix("config1", m, n, seed=0)
    t0 = time.perf_counter()
    fmt = format_code(args.format, E)
    ebytes = entry_bytes(args.format)
    M = E.EffortMatrix(W, P=P, groups=args.groups, device=dev, entry_format=fmt, crop=args.crop)
    log("layout %.1f MB, G=%d, prepare %.1fs" % (M.layout_bytes / 1e6, M.groups, time.perf_counter() - t0))

    # kept counts of the vectors (parity-path run, untimed)
    v0 = torch.from_numpy(synth.vector("config1", m, seed=0)).to(dev)
    kept0 = M.matvec_debug(v0, effort, with_mask=False)["total_kept"]
    call_bytes = ebytes * kept0
    R = max(2, int(math.ceil(args.rotate_gib * GiB / call_bytes)))
    Rd = max(2, int(math.ceil(args.rotate_gib * GiB / (2.0 * m * n))))
    # both graphs hold C calls, cycling over their own copies
    C = max(R, Rd, args.graph_calls)
    log("rotation: %d layouts (%.0f MB read per call), %d dense copies, %d calls per graph"
        % (R, call_bytes / 1e6, Rd, C))

    result = {}
    if args.mode in ("full", "effort"):
        layouts = [M.layout] + [M.layout.clone() for _ in range(R - 1)]
        vs = [torch.from_numpy(synth.vector("config1", m, seed=r)).to(dev) for r in range(R)]
        ys = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(R)]
        kept = []
        for r in range(R):
            Mr = E.EffortMatrix.from_blob(M.desc, layouts[r])
            kept.append(Mr.matvec_debug(vs[r], effort, with_mask=False)["total_kept"])
        kept_mean = float(np.mean(kept))
        ws, wsb = M.ws, M.ws_bytes

        def cycle():
            for i in range(C):
                r = i % R
                E.effort_matvec(M.desc, layouts[r], vs[r], effort, ys[r], ws, wsb)

        for _ in range(3):  # eager warm-up (and JIT of code objects)
            cycle()
        torch.cuda.synchronize()
        g = capture(torch, cycle)
        wreps = max(1, args.warmup // C)
        time_replays(torch, g, wreps)
        reps = max(1, int(math.ceil(args.steps / C)))
        steps = reps * C
        log("timing %d steps" % steps)
        ms, host_ms = time_replays(torch, g, reps)
        us_per = ms * 1e3 / steps

        # per-stage durations: events around each kernel of R eager calls.  A few
        # graph replays go first so the GPU is busy while the host enqueues the
        # eager calls; the eager calls then run back to back.
        evs = [[E.effort_event_create() for _ in range(6)] for _ in range(R)]
        head = max(1, int(math.ceil(3000.0 / max(us_per * R, 1.0))))
        sel, dsp, mul = [], [], []
        treps = max(1, min(reps, 50))
        for _ in range(treps):
            for _ in range(head):
                g.replay()
            for r in range(R):
                E.effort_matvec_timed(M.desc, layouts[r], vs[r], effort, ys[r], ws, wsb, evs[r])
            torch.cuda.synchronize()
            for r in range(R):
                e = evs[r]
                sel.append(E.effort_event_elapsed_ms(e[0], e[1]))
                dsp.append(E.effort_event_elapsed_ms(e[2], e[3]))
                mul.append(E.effort_event_elapsed_ms(e[4], e[5]))
        mul_us = statistics.mean(mul) * 1e3
        alg_mul = ebytes * kept_mean + 4.0 * m + 4.0 * n
        alg_step = ebytes * kept_mean + 2.0 * m * P + 4.0 * m + 4.0 * n
        achieved = alg_mul / (mul_us * 1e-6) / 1e9
        traffic = read_counters(args.format)
        result.update({
            "us_per_matvec": us_per,
            "ms_per_step": ms / steps,
            "steps": steps,
            "host_ms": host_ms,
            "kept_fraction": kept_mean / (m * n),
            "hbm_gbs": alg_step / (us_per * 1e-6) / 1e9,
            "stages_us": {"select": statistics.mean(sel) * 1e3, "dispatch": statistics.mean(dsp) * 1e3,
                          "bucketmul": mul_us},
            "roofline": {"bound": "hbm", "kernel": "k_bucketmul", "achieved": achieved,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "traffic": traffic, "alg_bytes": alg_mul, "kernel_us": mul_us,
                         # the same kernel time over the bytes it actually moved
                         "traffic_frac": (traffic / (mul_us * 1e-6) / 1e9 / HBM_PEAK_GBS) if traffic else None,
                         "traffic_source": (os.path.relpath(COUNTERS, ROOT) + ": rocprofv3 FETCH_SIZE + "
                                            "WRITE_SIZE per dispatch of this kernels.hip and entry format, "
                                            "scaled by a 1 GiB copy") if traffic else None},
            "rotation": R, "graph_calls": C, "groups": M.groups,
        })
        for e in sum(evs, []):
            E.effort_event_destroy(e)
        del layouts

    if args.mode in ("full", "dense"):
        Wd0 = torch.from_numpy(W.view(np.int16)).to(dev)
        Wds = [Wd0] + [Wd0.clone() for _ in range(Rd - 1)]
        vds = [torch.from_numpy(synth.vector("config1", m, seed=r)).to(dev) for r in range(Rd)]
        yds = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(Rd)]

        def dcycle():
            for i in range(C):
                r = i % Rd
                E.dense_gemv(Wds[r], vds[r], m, n, yds[r])

        for _ in range(3):
            dcycle()
        gd = capture(torch, dcycle)
        time_replays(torch, gd, max(1, args.warmup // C))
        dreps = max(1, int(math.ceil(args.steps / C)))
        dms, _ = time_replays(torch, gd, dreps)
        dense_us = dms * 1e3 / (dreps * C)
        result["dense_us"] = dense_us
        result["dense_gbs"] = 2.0 * m * n / (dense_us * 1e-6) / 1e9
        # library sanity reference: torch's fp16 matmul (hipBLASLt / rocBLAS) on the
        # same rotation, v rounded to fp16, fp16 output
        Whs = [w.view(torch.float16) for w in Wds]
        vhs = [x.to(torch.float16).reshape(1, m) for x in vds]
        yhs = [torch.empty((1, n), dtype=torch.float16, device=dev) for _ in range(Rd)]

        def lcycle():
            for i in range(C):
                r = i % Rd
                torch.matmul(vhs[r], Whs[r], out=yhs[r])

        for _ in range(3):
            lcycle()
        gl = capture(torch, lcycle)
        time_replays(torch, gl, max(1, args.warmup // Rd))
        lms, _ = time_replays(torch, gl, dreps)
        result["library_dense_us"] = lms * 1e3 / (dreps * C)
        if "us_per_matvec" in result:
            result["speedup_vs_dense"] = dense_us / result["us_per_matvec"]

    cpu = None
    if args.mode == "full" and not args.no_cpu_baseline:
        import oracle

        log("cpu baseline: oracle probes (untimed precompute)")
        pr = oracle.probes(W, P)
        times = []
        t_end = time.perf_counter() + args.cpu_seconds
        s = 0
        while (time.perf_counter() < t_end or len(times) < 3) and s < 100:
            v = synth.vector("config1", m, seed=s)
            t = time.perf_counter()
            oracle.run(W, pr, v, effort)
            times.append(time.perf_counter() - t)
            s += 1
        cpu = {"value": statistics.median(times) * 1e6, "unit": "µs/matvec", "cores": 1,
               "kind": "oracle",
               "sample": "oracle.run (single-threaded C, brute-force keep test over all %dx%d "
                         "products) on %d seeded vectors of the same workload, probes precomputed; "
                         "median" % (m, n, len(times))}
        cpu.update(host_info())
        # context: a plain dense fp32 matvec on one host core (numpy, one BLAS thread)
        try:
            from threadpoolctl import threadpool_limits
            Wf = W.view(np.float16).astype(np.float32)
            vf = synth.vector("config1", m, seed=0)
            dts = []
            with threadpool_limits(limits=1):
                for _ in range(5):
                    t = time.perf_counter()
                    vf @ Wf
                    dts.append(time.perf_counter() - t)
            cpu["dense_context"] = {"value": statistics.median(dts) * 1e6, "unit": "µs/matvec", "cores": 1,
                                    "kind": "numpy float32 v @ W (W widened from fp16 beforehand), "
                                            "one BLAS thread, median of 5"}
            del Wf
        except ImportError:
            pass

    if args.mode == "full":
        out = {
            "metric": METRIC, "value": result["us_per_matvec"], "unit": "µs/matvec",
            "n_gpus": 1, "steps": result["steps"], "warmup": args.warmup,
            "ms_per_step": result["ms_per_step"], "higher_is_better": False, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32 (fp16 weights)", "data": "synthetic",
            "config": {"workload": "effort matvec %dx%d fp16, effort %g, batch 1" % (m, n, effort),
                       "in_dim": m, "out_dim": n, "effort": effort, "P": P,
                       "groups": result["groups"], "rotation_copies": result["rotation"],
                       "graph_calls": result["graph_calls"],
                       "entry_format": args.format, "crop_segments": args.crop or P},
            "hbm_gbs": result["hbm_gbs"], "kept_fraction": result["kept_fraction"],
            "dense_us": result["dense_us"], "dense_gbs": result["dense_gbs"],
            "library_dense_us": result["library_dense_us"],
            "speedup_vs_dense": result["speedup_vs_dense"], "stages_us": result["stages_us"],
            "roofline": result["roofline"], "cpu_baseline": cpu,
        }
    else:
        out = dict(result, mode=args.mode)
    print(json.dumps(out))


# ---------------------------------------------------------------- other configurations
# Each prints one JSON line of its own; the headline line above is unchanged.

def graph_time_us(torch, fn, reps, warm=3):
    """Capture fn() once, replay it `reps` times, return µs per replay."""
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    g = capture(torch, fn)
    time_replays(torch, g, warm)
    ms, _ = time_replays(torch, g, reps)
    return ms * 1e3 / reps


def rotation_copies(call_bytes, rotate_gib=1.0):
    return max(2, int(math.ceil(rotate_gib * (1 << 30) / max(call_bytes, 1.0))))


def run_sweep(args, torch, np, E, synth, dev):
    """Mistral-7B matrix shapes x efforts {1, .5, .25, .125}: µs/matvec with the
    same rotation rule as the headline, beside the dense GEMV."""
    shapes = [(4096, 4096), (4096, 1024), (4096, 14336), (14336, 4096)]
    rows = []
    for (m, n) in shapes:
        W = synth.matrix("config1", m, n, seed=0)
        M = E.EffortMatrix(W, P=args.P, device=dev, **layout_opts(args, E))
        Wd = torch.from_numpy(W.view(np.int16)).to(dev)
        Rd = rotation_copies(2.0 * m * n)
        Wds = [Wd] + [Wd.clone() for _ in range(Rd - 1)]
        vd = torch.from_numpy(synth.vector("config1", m, seed=0)).to(dev)
        yd = torch.empty(n, dtype=torch.float32, device=dev)
        Cd = max(Rd, args.graph_calls)
        dense_us = graph_time_us(torch, lambda: [E.dense_gemv(Wds[i % Rd], vd, m, n, yd) for i in range(Cd)],
                                 max(5, 2000 // Cd)) / Cd
        del Wds
        for effort in (1.0, 0.5, 0.25, 0.125):
            v0 = torch.from_numpy(synth.vector("config1", m, seed=0)).to(dev)
            kept = M.matvec_debug(v0, effort, with_mask=False)["total_kept"]
            R = rotation_copies(entry_bytes(args.format) * kept)
            layouts = [M.layout] + [M.layout.clone() for _ in range(R - 1)]
            vs = [torch.from_numpy(synth.vector("config1", m, seed=r)).to(dev) for r in range(R)]
            ys = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(R)]

            C = max(R, args.graph_calls)

            def cyc():
                for i in range(C):
                    r = i % R
                    E.effort_matvec(M.desc, layouts[r], vs[r], effort, ys[r], M.ws, M.ws_bytes)

            us = graph_time_us(torch, cyc, max(5, 2000 // C)) / C
            rows.append({"in": m, "out": n, "effort": effort, "us": round(us, 2),
                         "kept_fraction": round(kept / (m * n), 4),
                         "alg_GBps": round((entry_bytes(args.format) * kept + 2.0 * m * args.P
                                            + 4.0 * (m + n)) / us / 1e3, 1),
                         "dense_us": round(dense_us, 2), "speedup_vs_dense": round(dense_us / us, 3),
                         "rotation": R})
            log(json.dumps(rows[-1]))
            del layouts
    print(json.dumps({"mode": "sweep", "unit": "µs/matvec", "P": args.P, "points": rows}))


def run_batched(args, torch, np, E, synth, dev):
    """b independent vectors through one matrix, each with its own cutoff, against
    the dense small GEMM that reads W once for all b."""
    m, n, effort = args.m, args.n, args.effort
    W = synth.matrix("config1", m, n, seed=0)
    M = E.EffortMatrix(W, P=args.P, device=dev, batch=16, **layout_opts(args, E))
    Wd = torch.from_numpy(W.view(np.int16)).to(dev)
    Rd = rotation_copies(2.0 * m * n)
    Wds = [Wd] + [Wd.clone() for _ in range(Rd - 1)]
    v0 = torch.from_numpy(synth.vector("config1", m, seed=0)).to(dev)
    kept = M.matvec_debug(v0, effort, with_mask=False)["total_kept"]
    R = rotation_copies(entry_bytes(args.format) * kept)
    layouts = [M.layout] + [M.layout.clone() for _ in range(R - 1)]
    rows = []
    for b in (1, 2, 4, 8, 16):
        V = torch.from_numpy(np.stack([synth.vector("config4", m, seed=s) for s in range(b)])).to(dev)
        Y = torch.empty((b, n), dtype=torch.float32, device=dev)

        C = max(R, args.graph_calls)
        Cd = max(Rd, args.graph_calls)

        def cyc():
            for i in range(C):
                E.effort_matvec_batched(M.desc, layouts[i % R], V, b, effort, Y, M.ws, M.ws_bytes)

        us = graph_time_us(torch, cyc, max(5, 400 // C)) / C
        dense_us = graph_time_us(torch, lambda: [E.dense_gemm_small(Wds[i % Rd], V, b, m, n, Y)
                                                 for i in range(Cd)], max(5, 400 // Cd)) / Cd
        rows.append({"batch": b, "effort_us": round(us, 2), "dense_gemm_us": round(dense_us, 2),
                     "effort_faster": us < dense_us})
        log(json.dumps(rows[-1]))
    cross = next((r["batch"] for r in rows if not r["effort_faster"]), None)
    print(json.dumps({"mode": "batched", "workload": "%dx%d fp16, effort %g" % (m, n, effort),
                      "unit": "µs per call (all b vectors)", "points": rows,
                      "first_batch_where_dense_wins": cross}))


MISTRAL = {"dim": 4096, "kv": 1024, "hidden": 14336, "vocab": 32000}


def layer_shapes():
    d, kv, h = MISTRAL["dim"], MISTRAL["kv"], MISTRAL["hidden"]
    return {"wq": (d, d), "wk": (d, kv), "wv": (d, kv), "wo": (d, d), "w1": (d, h), "w3": (d, h),
            "w2": (h, d)}


def run_decode(args, torch, np, E, synth, dev):
    """Every matvec of one decode step of a Mistral-7B-shaped stack (random-init
    fp16 weights, a distinct seeded matrix per layer and role), captured in one
    graph; per-token latency beside the same chain with the dense GEMV."""
    effort, L = args.effort, args.layers
    shapes = layer_shapes()
    layers, dlayers = [], []
    t0 = time.perf_counter()
    weights = 0
    for l in range(L):
        EL, DL = {}, {}
        for r in E.LAYER_ROLES:
            m, n = shapes[r]
            W = synth.matrix("config2", m, n, seed=0, layer=l, w=r)
            EL[r] = E.EffortMatrix(W, P=args.P, device=dev, **layout_opts(args, E))
            DL[r] = torch.from_numpy(W.view(np.int16)).to(dev)
            weights += m * n
        layers.append(EL)
        dlayers.append(DL)
        log("layer %d prepared (%.0fs)" % (l, time.perf_counter() - t0))
    Wh = synth.matrix("config2", MISTRAL["dim"], MISTRAL["vocab"], seed=0, w="head")
    head = E.EffortMatrix(Wh, P=args.P, device=dev)
    dhead = torch.from_numpy(Wh.view(np.int16)).to(dev)
    weights += Wh.size
    del Wh
    to = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
    x = [to(synth.vector("config2/x", MISTRAL["dim"], seed=0, layer=l)) for l in range(L)]
    a = [to(synth.vector("config2/attn", MISTRAL["dim"], seed=0, layer=l)) for l in range(L)]
    hin = to(synth.vector("config2/head_in", MISTRAL["dim"], seed=0))
    step = E.DecodeStep(layers, head, x, a, hin)
    gstep = E.DecodeStep(layers, head, x, a, hin, grouped=True)
    dstep = E.DenseDecodeStep(dlayers, dhead, x, a, hin)
    side = [torch.cuda.Stream() for _ in range(args.streams)] or None
    us1 = graph_time_us(torch, lambda: step.enqueue(effort), 20)
    dus1 = graph_time_us(torch, lambda: dstep.enqueue(), 20)
    us = graph_time_us(torch, lambda: step.enqueue(effort, side_streams=side), 20) if side else us1
    dus = graph_time_us(torch, lambda: dstep.enqueue(side_streams=side), 20) if side else dus1
    gus1 = graph_time_us(torch, lambda: gstep.enqueue(effort), 20)
    gus = graph_time_us(torch, lambda: gstep.enqueue(effort, side_streams=side), 20) if side else gus1
    print(json.dumps({"mode": "decode", "workload": "Mistral-7B-shaped decode step, %d layers + head, "
                      "effort %g, batch 1" % (L, effort), "matvecs": step.calls,
                      "weights": weights, "side_streams": args.streams,
                      "effort_us_per_token": round(us, 1), "dense_us_per_token": round(dus, 1),
                      "speedup_vs_dense": round(dus / us, 3),
                      "one_stream": {"effort_us_per_token": round(us1, 1),
                                     "dense_us_per_token": round(dus1, 1)},
                      "grouped": {"note": "qkv and w1/w3 as multi-matrix calls",
                                  "one_stream_us_per_token": round(gus1, 1),
                                  "side_streams_us_per_token": round(gus, 1),
                                  "speedup_vs_best_dense": round(min(dus, dus1) / min(gus, gus1), 3)},
                      "dense_GBps": round(2.0 * weights / dus / 1e3, 1)}))


def run_moe(args, torch, np, E, synth, dev):
    """A Mixtral-shaped expert block (8 experts of w1/w3 4096x14336 and w2
    14336x4096), top-2 routing from seeded logits; per-token latency of the two
    routed experts' six matvecs and the glue, beside the dense equivalent."""
    d, h = MISTRAL["dim"], MISTRAL["hidden"]
    experts, dexperts = [], []
    for e in range(8):
        Ws = [synth.matrix("config3", d, h, seed=0, expert=e, w="w1"),
              synth.matrix("config3", d, h, seed=0, expert=e, w="w3"),
              synth.matrix("config3", h, d, seed=0, expert=e, w="w2")]
        experts.append(tuple(E.EffortMatrix(W, P=args.P, device=dev, **layout_opts(args, E)) for W in Ws))
        dexperts.append(tuple(torch.from_numpy(W.view(np.int16)).to(dev) for W in Ws))
        log("expert %d prepared" % e)
    moe = E.MoEFFN(experts, dev)
    gmoe = E.MoEFFN(experts, dev, grouped=True)
    tokens = 16
    xs = [torch.from_numpy(synth.vector("config3/x", d, seed=t)).to(dev) for t in range(tokens)]
    routes = [E.route_top2(synth.normals(8, seed=t, stream=synth.stream_id("config3/router")))
              for t in range(tokens)]
    hbuf = torch.empty(h, dtype=torch.float32, device=dev)
    h3buf = torch.empty(h, dtype=torch.float32, device=dev)
    gbuf = torch.empty(h, dtype=torch.float32, device=dev)
    o = [torch.empty(d, dtype=torch.float32, device=dev) for _ in range(2)]
    y = torch.empty(d, dtype=torch.float32, device=dev)

    def dense_token(t):
        e0, e1, g0, g1 = routes[t]
        for k, e in enumerate((e0, e1)):
            w1, w3, w2 = dexperts[e]
            E.dense_gemv(w1, xs[t], d, h, hbuf)
            E.dense_gemv(w3, xs[t], d, h, h3buf)
            E.effort_silu_mul(hbuf, h3buf, h, gbuf)
            E.dense_gemv(w2, gbuf, h, d, o[k])
        E.effort_axpby(o[0], g0, o[1], g1, d, y)

    dus = graph_time_us(torch, lambda: [dense_token(t) for t in range(tokens)], 10) / tokens
    side = [torch.cuda.Stream() for _ in range(max(args.streams, 4))] if args.streams else None
    points = []
    for effort in (0.25, 0.16, 0.12):
        us1 = graph_time_us(torch, lambda: [moe.enqueue(xs[t], routes[t], effort)
                                           for t in range(tokens)], 10) / tokens
        us = graph_time_us(torch, lambda: [moe.enqueue(xs[t], routes[t], effort, side_streams=side)
                                          for t in range(tokens)], 10) / tokens if side else us1
        gus1 = graph_time_us(torch, lambda: [gmoe.enqueue(xs[t], routes[t], effort)
                                            for t in range(tokens)], 10) / tokens
        gus = graph_time_us(torch, lambda: [gmoe.enqueue(xs[t], routes[t], effort, side_streams=side)
                                           for t in range(tokens)], 10) / tokens if side else gus1
        points.append({"effort": effort, "effort_us_per_token": round(us, 1),
                       "one_stream_us_per_token": round(us1, 1),
                       "speedup_vs_dense": round(dus / us, 3),
                       "grouped_us_per_token": round(gus1, 1),
                       "grouped_side_streams_us_per_token": round(gus, 1),
                       "grouped_speedup_vs_dense": round(dus / min(gus, gus1), 3)})
        log(json.dumps(points[-1]))
    print(json.dumps({"mode": "moe", "workload": "Mixtral-shaped expert block, 8 experts, top-2, "
                      "%d tokens" % tokens, "dense_us_per_token": round(dus, 1), "points": points}))


def run_moetraffic(args, torch, np, E, synth, dev):
    """What the expert block reads against what the two routed experts keep:
    `tokens` grouped expert-block calls (the only launches of the *_multi
    kernels, so a FETCH_SIZE counter run can sum exactly their reads), then,
    through the recording entry point on the inputs those calls used, the kept
    products of each of the six matvecs.  Per token it prints the kept bytes
    (the layout's bytes per entry, 3 for r12, per kept entry) and the method's
    algorithmic bytes (kept bytes + 2mP probes + 4m v + 4n y per matvec); the
    layouts of all 8 experts hold four times the two routed experts' entries."""
    d, h = MISTRAL["dim"], MISTRAL["hidden"]
    effort, tokens = 0.25, 4
    experts = []
    for e in range(8):
        Ws = [synth.matrix("config3", d, h, seed=0, expert=e, w="w1"),
              synth.matrix("config3", d, h, seed=0, expert=e, w="w3"),
              synth.matrix("config3", h, d, seed=0, expert=e, w="w2")]
        experts.append(tuple(E.EffortMatrix(W, P=args.P, device=dev, **layout_opts(args, E)) for W in Ws))
        log("expert %d prepared" % e)
    gmoe = E.MoEFFN(experts, dev, grouped=True)
    xs = [torch.from_numpy(synth.vector("config3/x", d, seed=t)).to(dev) for t in range(tokens)]
    routes = [E.route_top2(synth.normals(8, seed=t, stream=synth.stream_id("config3/router")))
              for t in range(tokens)]
    torch.cuda.synchronize()
    w2_inputs = []
    for t in range(tokens):  # the counted calls
        gmoe.enqueue(xs[t], routes[t], effort)
        torch.cuda.synchronize()
        w2_inputs.append([g.clone() for g in gmoe.g])
    rows = []
    for t in range(tokens):
        e0, e1 = routes[t][0], routes[t][1]
        kept = alg = 0
        for k, e in enumerate((e0, e1)):
            w1, w3, w2 = experts[e]
            for M, v in ((w1, xs[t]), (w3, xs[t]), (w2, w2_inputs[t][k])):
                kk = M.matvec_debug(v, effort, with_mask=False)["total_kept"]
                kept += kk
                alg += (entry_bytes(args.format) * kk + 2 * M.in_dim * args.P + 4 * M.in_dim
                        + 4 * M.out_dim)
        rows.append({"token": t, "experts": [int(e0), int(e1)],
                     "kept_bytes": entry_bytes(args.format) * kept, "alg_bytes": alg})
        log(json.dumps(rows[-1]))
    print(json.dumps({"mode": "moetraffic", "workload": "Mixtral-shaped expert block, 8 experts, "
                      "top-2, grouped calls, effort %g, %d tokens" % (effort, tokens),
                      "kernels": "k_chart_hist_multi, k_dispatch*_multi, k_bucketmul_multi, "
                      "k_silu_mul, k_axpby", "points": rows}))


def run_mallcheck(args, torch, np, E, synth, dev):
    """Cross-check of the rotation rule against the 256 MB Infinity Cache: the
    three kernels' own durations (event pairs stamped by each kernel) for calls
    cycling over R layout copies (the headline's method), for calls on one
    layout each after a 1 GiB scratch read or write that evicts the cache (outside
    the timed kernels), and for repeated calls on one layout (warm cache, for
    contrast)."""
    m, n, effort = args.m, args.n, args.effort
    W = synth.matrix("config1", m, n, seed=0)
    M = E.EffortMatrix(W, P=args.P, device=dev, **layout_opts(args, E))
    v0 = torch.from_numpy(synth.vector("config1", m, seed=0)).to(dev)
    kept = M.matvec_debug(v0, effort, with_mask=False)["total_kept"]
    R = rotation_copies(entry_bytes(args.format) * kept, args.rotate_gib)
    layouts = [M.layout] + [M.layout.clone() for _ in range(R - 1)]
    y = torch.empty(n, dtype=torch.float32, device=dev)
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    ev = [E.effort_event_create() for _ in range(6)]
    reps = 60

    def timed(layout, before=None):
        ks = []
        for it in range(reps):
            if before is not None:
                before(it)
            E.effort_matvec_timed(M.desc, layout(it), v0, effort, y, M.ws, M.ws_bytes, ev)
            torch.cuda.synchronize()
            ks.append([E.effort_event_elapsed_ms(ev[2 * k], ev[2 * k + 1]) * 1e3 for k in range(3)])
        ks = np.array(ks)[5:]  # the first calls warm up
        return {"bucketmul_us": round(float(np.median(ks[:, 2])), 2),
                "kernels_us": round(float(np.median(ks.sum(axis=1))), 2)}

    scratch.fill_(1.0)
    torch.cuda.synchronize()
    rows = {
        "rotation": timed(lambda it: layouts[it % R]),
        # a 1 GiB read evicts the cache without leaving dirty lines behind
        "evicted_by_read": timed(lambda it: M.layout, lambda it: scratch.sum()),
        # a 1 GiB write also leaves 1 GiB to be written back while the call runs
        "evicted_by_write": timed(lambda it: M.layout, lambda it: scratch.fill_(float(it))),
        "warm": timed(lambda it: M.layout),
    }
    for e in ev:
        E.effort_event_destroy(e)
    print(json.dumps({"mode": "mallcheck", "workload": "%dx%d fp16, effort %g" % (m, n, effort),
                      "rotation": R, "points": rows}))


EXTRA_MODES = {"sweep": run_sweep, "batched": run_batched, "decode": run_decode, "moe": run_moe,
               "moetraffic": run_moetraffic, "mallcheck": run_mallcheck}


if __name__ == "__main__":
    main()
