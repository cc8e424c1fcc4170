"""Benchmark: one Muon / NorMuon optimizer step over one Llama-3-8B-shaped layer
on one MI355X, through the C ABI (one muon_step_groups call over the layer's
four shape groups).

A step is the whole hot path for the layer's seven matrices: Nesterov
momentum, Frobenius normalization, five quintic Newton-Schulz iterations
(bf16 MFMA, fp32 accumulation), NorMuon and the spectrally scaled fp32 weight
update with its bf16 model copy.  Groups: {q, o} 4096x4096, {k, v} 1024x4096,
{gate, up} 14336x4096, {down} 4096x14336.  Gradients are the seeded power-law
matrices of the workload definition (U diag(i^-0.7) V^T + 0.1 N(0,1)), bf16;
master weights fp32 N(0, 0.02^2); momentum bf16; all resident in HBM before
timing starts.

With --layers L > 1 a step covers L such layers in the same one call (the
model-wide step: 32 layers are the 224 matrices of Llama-3-8B); the gradients
of every layer then come from the device generator (the same power-law signal
per shape, torch's generator for the noise), since host generation of 7e9
values would take minutes.

Prints one JSON line.  `value` is Newton-Schulz orthogonalizations per second
(7 L per step).  `roofline` covers the dominant kernel (the X <- a X + B X
update GEMM) from HIP events recorded around each of its launches inside the
timed region; `cpu_baseline` times the float64 oracle on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 MFMA (published)
METRIC = "NS5 orthogonalizations/sec + TFLOP/s (% bf16 MFMA peak) at Llama-8B shapes"
LAYER = (("q", (4096, 4096)), ("k", (1024, 4096)), ("v", (1024, 4096)), ("o", (4096, 4096)),
         ("gate", (14336, 4096)), ("up", (14336, 4096)), ("down", (4096, 14336)))
WORKLOAD_ID = 2


def ns_flops(rows, cols, steps=5):
    """(L, E) FLOPs of `steps` iterations: L = 4 m^2 n + m^3, E = 3 m^2 n + m^3 per iteration."""
    m, n = min(rows, cols), max(rows, cols)
    return steps * (4 * m * m * n + m ** 3), steps * (3 * m * m * n + m ** 3)


def make_layer_inputs():
    """Seeded inputs of the layer.  U, V and s of the power-law gradients are
    drawn once per shape (key: workload, layer, index of the first matrix of
    that shape); each matrix has its own noise (key: workload, layer, index,
    step 1)."""
    import concurrent.futures as cf
    import synth
    grads, weights = {}, {}
    index = {name: i for i, (name, _) in enumerate(LAYER)}

    def one_shape(item):
        # The shapes are independent draws (their own keys), so they are made
        # in parallel threads (numpy's QR and matmul release the GIL); the
        # values do not depend on the order.
        shape, names = item
        t = time.perf_counter()
        first = index[names[0]]
        gs = synth.power_law_many(shape, (WORKLOAD_ID, 0, first),
                                  [(WORKLOAD_ID, 0, index[n], 1) for n in names], "bf16")
        ws = [synth.gaussian(shape, (WORKLOAD_ID, 0, index[n], 0, synth.ROLE_WEIGHT), "f32", std=0.02)
              for n in names]
        print(f"[bench] generated {'+'.join(names)} {shape} in {time.perf_counter() - t:.1f} s",
              file=sys.stderr, flush=True)
        return names, gs, ws

    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        for names, gs, ws in ex.map(one_shape, groups_of_layer()):
            for n, g, w in zip(names, gs, ws):
                grads[n] = g
                weights[n] = w
    return grads, weights


def make_model_inputs(layers, dev):
    """Device-generated inputs of `layers` layers (layer l, matrix i: the
    shape's signal plus noise keyed (workload 5, l, i, step 1); weights
    N(0, 0.02^2) from the device generator keyed (5, l, i, 0, weight))."""
    import torch
    import synth
    index = {name: i for i, (name, _) in enumerate(LAYER)}
    grads, weights = {}, {}
    for shape, names in groups_of_layer():
        sig = torch.from_numpy(synth.power_law_signal(shape, (WORKLOAD_ID, 0, index[names[0]]))
                               .astype(np.float32)).to(dev)
        for l in range(layers):
            for n in names:
                grads[(l, n)] = synth.power_law_device(sig, (5, l, index[n], 1))
                gen = torch.Generator(device=dev)
                gen.manual_seed(synth.key_seed((5, l, index[n], 0, synth.ROLE_WEIGHT)))
                weights[(l, n)] = 0.02 * torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
        del sig
    return grads, weights


def groups_of_layer():
    order = []
    by_shape = {}
    for name, shape in LAYER:
        if shape not in by_shape:
            by_shape[shape] = []
            order.append(shape)
        by_shape[shape].append(name)
    return [(shape, by_shape[shape]) for shape in order]


def host_info():
    """What the CPU baseline ran on: the host's logical CPUs, its CPU model and
    the BLAS threads numpy uses."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count()
    return {"cpu_count": os.cpu_count(), "cpu_model": model, "blas_threads": int(threads)}


def step_stats(ms):
    """Median, min, p90 and mean of per-step times (ms)."""
    a = np.sort(np.asarray(ms, dtype=np.float64))
    return {"reps": int(a.size), "median": round(float(np.median(a)), 4), "min": round(float(a[0]), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "mean": round(float(a.mean()), 4)}


def cpu_baseline(grads, weights, target_seconds=20.0):
    """The oracle as it stands, on the layer's matrices smallest first until about
    target_seconds of CPU work (k, v, q, o, down, gate, ...), scaled by dense
    float64 NS FLOPs to the whole layer."""
    import oracle
    import synth
    host = host_info()
    hp = oracle.MuonHParams(lr=0.05, normuon=True, mom_dtype="bf16")

    def dense(rows, cols):
        m, n = min(rows, cols), max(rows, cols)
        return 5 * (4 * m * m * n + 2 * m ** 3)

    sample = ["k", "v", "q", "o", "down", "gate", "up"]
    t0 = time.perf_counter()
    done = []
    for name in sample:
        shape = dict(LAYER)[name]
        oracle.muon_step(weights[name].astype(np.float64), synth.bf16_bits_to_f64(grads[name]),
                         np.zeros(shape), np.zeros(shape[0]), hp)
        done.append(name)
        if time.perf_counter() - t0 > target_seconds:
            break
    dt = time.perf_counter() - t0
    f_sample = sum(dense(*dict(LAYER)[n]) for n in done)
    f_layer = sum(dense(*s) for _, s in LAYER)
    layer_seconds = dt * f_layer / f_sample
    return {"value": round(len(LAYER) / layer_seconds, 6), "unit": "orth/s", "cores": host["blas_threads"],
            "kind": "oracle", **host,
            "sample": f"float64 numpy oracle, one Muon/NorMuon step of {'+'.join(done)} "
                      f"({dt:.1f} s), scaled by dense NS FLOPs ({f_sample:.3e} of {f_layer:.3e}) to the 7-matrix layer"}


def source_digest():
    """sha256 over the library's HIP sources (kernels and the host code that lays
    out their operands), in file-name order."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "newton_schulz_ns5_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def traffic_for(kernel_name):
    """HBM bytes per launch from the committed counter summary (profiles/traffic.json),
    used only while the library's sources still have the digest the counters were
    taken with."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        info = json.load(open(path))
        digest = source_digest()
        rec = info.get(kernel_name)
        if rec and rec.get("source_sha256") == digest:
            return rec.get("bytes_per_launch")
    except Exception:
        return None
    return None


def capture(step_fn):
    """One step captured in a HIP graph (the library only enqueues kernels while
    its launch timing is off); returns the graph's replay."""
    import torch
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step_fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return graph.replay


def event_time(fn, steps, warmup):
    """Milliseconds per call of fn (the mean over `steps` calls) and the
    per-call times, from HIP events recorded on the current stream between
    consecutive calls."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record(stream)
    for i in range(steps):
        fn()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return evs[0].elapsed_time(evs[-1]) / steps, per


def calibration_pass(mib, dev):
    """Known HBM traffic for calibrating the counters: a fill writes exactly
    `mib` MiB, a sum over the same buffer reads them once."""
    import torch
    cal = torch.empty(mib << 19, dtype=torch.int16, device=dev)
    torch.cuda.synchronize()
    cal.fill_(1)
    total = cal.sum()
    torch.cuda.synchronize()
    del cal, total


def timed_steps(step_fn, steps, warmup, eager_only=False):
    """Time `steps` steps replayed from a HIP graph and `steps` steps launched
    from the host, then run `steps` more with the library's per-launch events
    on.  These steps are dozens of launches of a few microseconds each, so
    launching them from the host leaves the GPU waiting between kernels; events
    around every launch would add gaps of their own.  Returns ms per step
    (graph, eager) and the per-class launch totals of the third run."""
    import torch
    import newton_schulz_ns5_amd as ns
    ms_eager, per_eager = event_time(step_fn, steps, warmup)
    if eager_only:
        ms, per = ms_eager, per_eager
    else:
        replay = capture(step_fn)
        ms, per = event_time(replay, steps, warmup)
    ns.profile_reset()
    ns.profile_enable(True)
    # A spin kernel of ~0.1 s keeps the GPU busy while the host enqueues the
    # profiled steps, so the launches then run back to back and each event
    # pair brackets its kernel rather than the host's launch latency.
    torch.cuda._sleep(200_000_000)
    for _ in range(steps):
        step_fn()
    torch.cuda.synchronize()
    ns.profile_enable(False)
    return ms, ms_eager, per, {k: ns.profile_query(k) for k in ns.KERNEL_CLASSES}


def class_table(prof):
    """Per kernel class: launches, mean launch time, share of kernel time and the
    rate of its algorithmic work (TFLOP/s for the GEMMs, GB/s for the rest)."""
    per_class = {}
    total = max(sum(x["ms"] for x in prof.values()), 1e-9)
    for k, v in prof.items():
        sec = v["ms"] * 1e-3
        e = {"launches": v["launches"], "avg_us": round(1e3 * v["ms"] / max(v["launches"], 1), 2),
             "share": round(v["ms"] / total, 4)}
        if sec > 0 and v["flop"] > 0:
            e["tflops"] = round(v["flop"] / sec / 1e12, 1)
            e["gbps"] = round(v["bytes"] / sec / 1e9, 1)
        elif sec > 0 and v["bytes"] > 0:
            e["gbps"] = round(v["bytes"] / sec / 1e9, 1)
        per_class[k] = e
    return per_class


def side_workload(args, dev):
    """The per-head, conv-megabatch and fp32 256 x 256 workloads: one JSON line
    in the same format as the layer workload.  Their Newton-Schulz GEMMs have
    m = 128..512, so the roofline names the GEMM class with the largest share
    of time and takes HBM as its bound when its algorithmic FLOP per byte is
    below the ridge (the MFMA peak of the compute dtype over 8 TB/s)."""
    import ctypes
    import torch
    import newton_schulz_ns5_amd as ns
    import oracle
    import synth
    L = ns.lib()
    sptr = lambda: ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    compute = "bf16"
    if args.workload == "c1":
        # One 256 x 256 fp32 N(0,1) gradient, fp32 master and momentum; one
        # Muon step in fp32 compute mode (momentum 0.95 Nesterov, lr 0.05, five
        # quintic iterations, eps 1e-7 on the norm), no NorMuon.
        compute = "f32"
        shape = (256, 256)
        g = synth.gaussian(shape, (1, 0, 0, 1, synth.ROLE_GRAD), "f32")
        w = synth.gaussian(shape, (1, 0, 0, 0, synth.ROLE_WEIGHT), "f32", std=0.02)
        G = [torch.from_numpy(g).to(dev)]
        W = [torch.from_numpy(w).to(dev)]
        M = [torch.zeros(shape, dtype=torch.float32, device=dev)]
        group, keep = ns._make_group(W, G, M, None, None, heads=1)
        hp = ns.hparams(lr=0.05, momentum=0.95, nesterov=True, normuon=False,
                        ns=ns.ns_config(compute_dtype="f32"))
        garr = (ns.Group * 1)(group)
        ws = torch.empty(max(ns.step_groups_workspace_bytes([group], hp), 256), dtype=torch.uint8, device=dev)

        def step_fn():
            rc = L.muon_step_groups(garr, 1, ctypes.byref(hp), ctypes.c_void_p(ws.data_ptr()), ws.numel(), sptr())
            if rc != 0:
                raise RuntimeError(f"muon_step_groups failed: {rc} {L.muon_last_error()}")
        shapes = [(1, 256, 256)]
        workload = "single-256x256-fp32-muon-step"
        extra = {"normuon": False, "step": "full Muon step, fp32 compute (fp32 MFMA)",
                 "grad": "256x256 fp32 N(0,1)"}

        def cpu_leg():
            t0, done = time.perf_counter(), 0
            ohp = oracle.MuonHParams(lr=0.05, normuon=False, mom_dtype="f32")
            while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0) and done < 2000:
                oracle.muon_step(w.astype(np.float64), g.astype(np.float64), np.zeros(shape), None, ohp)
                done += 1
            dt = time.perf_counter() - t0
            return done / dt, f"float64 numpy oracle, {done} Muon steps of the 256 x 256 matrix in {dt:.1f} s"
    elif args.workload == "heads":
        # q_proj 4096 x 4096 as 32 heads of 128 rows, k_proj 1024 x 4096 as 8; N(0,1) bf16; NS only.
        parts = []
        for i, (rows, heads) in enumerate(((4096, 32), (1024, 8))):
            x = synth.gaussian((rows, 4096), (3, 0, i, 1, synth.ROLE_GRAD), "bf16")
            xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev).view(heads, rows // heads, 4096)
            yt = torch.empty_like(xt)
            parts.append((xt, yt, x))
        # Both projections in one muon_ns_groups call: every Newton-Schulz
        # launch covers the 40 heads.
        cfg = ns.ns_config(compute_dtype="bf16")
        probs = (ns.NSProblem * 2)(*[ns.NSProblem(xt.data_ptr(), ns.MUON_BF16, xt.stride(0), xt.stride(1),
                                                  yt.data_ptr(), ns.MUON_BF16, yt.stride(0), yt.stride(1),
                                                  *xt.shape) for xt, yt, _ in parts])
        ws = torch.empty(ns.ns_groups_workspace_bytes([tuple(xt.shape) for xt, _, _ in parts], cfg),
                         dtype=torch.uint8, device=dev)

        def step_fn():
            rc = L.muon_ns_groups(probs, 2, ctypes.byref(cfg), ctypes.c_void_p(ws.data_ptr()), ws.numel(), sptr())
            if rc != 0:
                raise RuntimeError(f"muon_ns_groups failed: {rc} {L.muon_last_error()}")
        shapes = [(32, 128, 4096), (8, 128, 4096)]
        workload = "llama3-8b-q-k-per-head-ns5"
        extra = {"heads": ["q 32x128x4096", "k 8x128x4096"], "normuon": False, "step": "Newton-Schulz only",
                 "call": "muon_ns_groups: q and k heads share every launch"}

        def cpu_leg():
            t0, done = time.perf_counter(), 0
            x = synth.bf16_bits_to_f64(parts[0][2])
            while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0) and done < 32:
                oracle.newton_schulz5(x[128 * done:128 * (done + 1)])
                done += 1
            dt = time.perf_counter() - t0
            return done / dt, f"float64 numpy oracle, Newton-Schulz of {done} q heads (128 x 4096) in {dt:.1f} s"
    else:
        groups, shapes, tensors = [], [], []
        for gi, (name, n, pshape) in enumerate(synth.conv_megabatches()):
            rows, cols = pshape[0], int(np.prod(pshape[1:]))
            gs = synth.power_law_many((rows, cols), (4, gi, 0), [(4, gi, i, 1) for i in range(n)], "bf16")
            G = [torch.from_numpy(g.view(np.int16)).view(torch.bfloat16).to(dev).view(pshape) for g in gs]
            W = [torch.from_numpy(synth.gaussian((rows, cols), (4, gi, i, 0, synth.ROLE_WEIGHT), "f32", std=0.02))
                 .to(dev).view(pshape) for i in range(n)]
            M = [torch.zeros(pshape, dtype=torch.bfloat16, device=dev) for _ in range(n)]
            V = [torch.zeros(rows, dtype=torch.float32, device=dev) for _ in range(n)]
            WM = [w.to(torch.bfloat16) for w in W]
            groups.append(ns._make_group(W, G, M, V, WM, heads=1))  # its `keep` holds the tensors
            tensors.append((G, W, M, V, WM))
            shapes.append((n, rows, cols))
            if gi == 0:
                sample = (synth.bf16_bits_to_f64(gs[0]), synth.gaussian((rows, cols), (4, 0, 0, 0, synth.ROLE_WEIGHT),
                                                                        "f32", std=0.02))
        hp = ns.hparams(lr=0.05, momentum=0.95, nesterov=True, normuon=True, beta2=0.95, norm_eps=1e-8,
                        ns=ns.ns_config(compute_dtype="bf16"))
        garr = (ns.Group * len(groups))(*[g for g, _ in groups])
        wsb = ns.step_groups_workspace_bytes([g for g, _ in groups], hp)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

        def step_fn():
            rc = L.muon_step_groups(garr, len(groups), ctypes.byref(hp), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                    sptr())
            if rc != 0:
                raise RuntimeError(f"muon_step_groups failed: {rc} {L.muon_last_error()}")
        workload = "conv-megabatch-normuon-step"
        extra = {"groups": [f"{n}x{r}x{c}" for n, r, c in shapes], "normuon": True,
                 "step": "full Muon/NorMuon step"}

        def cpu_leg():
            t0, done = time.perf_counter(), 0
            g, w = sample
            ohp = oracle.MuonHParams(lr=0.05, normuon=True, mom_dtype="bf16")
            while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0) and done < 64:
                oracle.muon_step(w.astype(np.float64), g, np.zeros(g.shape), np.zeros(g.shape[0]), ohp)
                done += 1
            dt = time.perf_counter() - t0
            # scaled to the workload's mix by dense float64 NS FLOPs
            f1 = 5 * (4 * 256 * 256 * 1152 + 2 * 256 ** 3)
            fw = sum(n * 5 * (4 * min(r, c) ** 2 * max(r, c) + 2 * min(r, c) ** 3) for n, r, c in shapes)
            nm = sum(n for n, _, _ in shapes)
            return (done / dt) * f1 / fw * nm, (f"float64 numpy oracle, {done} Muon/NorMuon steps of one 256 x 1152 "
                                                f"matrix in {dt:.1f} s, scaled by dense NS FLOPs to the workload")

    if args.copy_calibration_mib > 0:
        calibration_pass(args.copy_calibration_mib, dev)
    ms, ms_eager, per, prof = timed_steps(step_fn, args.steps, args.warmup, args.eager_only)
    nmat = sum(n for n, _, _ in shapes)
    fl_L = sum(n * ns_flops(r, c)[0] for n, r, c in shapes)
    fl_E = sum(n * ns_flops(r, c)[1] for n, r, c in shapes)
    per_class = class_table(prof)
    dom = max(("gram", "poly", "update"), key=lambda k: prof[k]["ms"])
    d = prof[dom]
    sec = d["ms"] * 1e-3
    tf = d["flop"] / sec / 1e12
    gbps = d["bytes"] / sec / 1e9
    peak = PEAK_BF16_TFLOPS if compute == "bf16" else PEAK_F32_TFLOPS
    hbm = d["flop"] / max(d["bytes"], 1) < peak / 8.0
    if compute == "f32":
        kname = "gemm_f32_kernel"
    elif args.workload == "heads" and dom == "update":
        kname = ("updgram128_kernel: the update fused with the next iteration's Gram, iterations 1-4, "
                 "and its update-only variant, the last iteration")
    else:
        kname = "gemm_nt_bf16_kernel"
    out = {
        "metric": METRIC, "value": round(nmat / (ms * 1e-3), 3), "unit": "orth/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": compute, "data": "synthetic",
        "config": dict({"workload": workload, "matrices": nmat, "ns_iterations": 5,
                        "launch": ("host-launched steps (--eager-only)" if args.eager_only
                                   else "HIP graph replay of one step"),
                        "ms_per_step_host_launched": round(ms_eager, 4),
                        "step_ms": step_stats(per),
                        "ns_compute": ("bf16 storage, fp32 accumulate (MFMA)" if compute == "bf16"
                                       else "fp32 throughout (fp32 MFMA)"),
                        "params_per_s": round(sum(n * r * c for n, r, c in shapes) / (ms * 1e-3), 1),
                        "tflops_L": round(fl_L / (ms * 1e-3) / 1e12, 2),
                        "pct_peak_L": round(100 * fl_L / (ms * 1e-3) / 1e12 / peak, 2),
                        "tflops_E": round(fl_E / (ms * 1e-3) / 1e12, 2),
                        "kernel_classes": per_class}, **extra),
        "roofline": {
            "bound": "hbm" if hbm else "mfma",
            "kernel": f"{dom} GEMM class ({kname})",
            "achieved": round(gbps if hbm else tf, 2),
            "peak": 8000.0 if hbm else peak,
            "unit": "GB/s" if hbm else "TFLOP/s",
            "frac": round((gbps / 8000.0) if hbm else (tf / peak), 4),
            "traffic": None,
            "tflops": round(tf, 2), "gbps": round(gbps, 1),
            "launches": d["launches"], "avg_launch_us": round(1e3 * d["ms"] / max(d["launches"], 1), 2),
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the CPU", file=sys.stderr, flush=True)
        v, desc = cpu_leg()
        host = host_info()
        out["cpu_baseline"] = {"value": round(v, 6), "unit": "orth/s", "cores": host["blas_threads"],
                               "kind": "oracle", **host, "sample": desc}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--workload", choices=["layer", "heads", "conv", "c1"], default="layer",
                    help="layer: the Muon/NorMuon step of Llama-3-8B layers (the default line); heads: "
                         "per-head Newton-Schulz of q [32,128,4096] and k [8,128,4096]; conv: the NorMuon step "
                         "of the conv megabatches [64,256,128,3,3] and [32,512,512,5]; c1: the fp32-mode Muon "
                         "step of one 256x256 fp32 gradient")
    ap.add_argument("--layers", type=int, default=1,
                    help="Llama-3-8B layers per step (1: the layer workload; 32: the whole model)")
    ap.add_argument("--print-source-digest", action="store_true",
                    help="print the digest of the HIP sources that profiles/traffic.json is keyed on, and exit")
    ap.add_argument("--eager-only", action="store_true",
                    help="side workloads: time host-launched steps only (no HIP graph), e.g. for counter passes")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the steps, fill and then sum a buffer of this many MiB (known bytes written "
                         "and read, for calibrating HBM traffic counters)")
    args = ap.parse_args()
    if args.print_source_digest:
        print(source_digest())
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the multi-GPU path is not part of this build", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import newton_schulz_ns5_amd as ns
    ns.lib()  # fail loudly if the library is missing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")

    if args.workload != "layer":
        return side_workload(args, dev)

    if args.layers < 1 or args.layers > 64:
        print("--layers must be in 1..64", file=sys.stderr)
        sys.exit(2)
    t_gen = time.perf_counter()
    if args.layers == 1:
        grads, weights = make_layer_inputs()
    else:
        dgrads, dweights = make_model_inputs(args.layers, dev)
    print(f"[bench] inputs generated in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    groups = []
    for shape, names in groups_of_layer():
        if args.layers == 1:
            G = [torch.from_numpy(grads[n].view(np.int16)).view(torch.bfloat16).to(dev) for n in names]
            W = [torch.from_numpy(weights[n]).to(dev) for n in names]
        else:
            keys = [(l, n) for l in range(args.layers) for n in names]
            G = [dgrads[k] for k in keys]
            W = [dweights[k] for k in keys]
            names = [f"{n}{l}" for l, n in keys]
        M = [torch.zeros(shape, dtype=torch.bfloat16, device=dev) for _ in names]
        V = [torch.zeros(shape[0], dtype=torch.float32, device=dev) for _ in names]
        WM = [w.to(torch.bfloat16) for w in W]
        g, keep = ns._make_group(W, G, M, V, WM, heads=1)
        groups.append({"shape": shape, "names": names, "g": g, "keep": keep, "tensors": (G, W, M, V, WM)})
    hp = ns.hparams(lr=0.05, momentum=0.95, nesterov=True, normuon=True, beta2=0.95, norm_eps=1e-8,
                    ns=ns.ns_config(compute_dtype="bf16"))
    import ctypes
    garr = (ns.Group * len(groups))(*[gr["g"] for gr in groups])
    ws_bytes = ns.step_groups_workspace_bytes([gr["g"] for gr in groups], hp)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    print(f"[bench] workspace {ws_bytes / 2**30:.2f} GiB", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream(dev)
    L = ns.lib()
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def one_step():
        rc = L.muon_step_groups(garr, len(groups), ctypes.byref(hp), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                sptr)
        if rc != 0:
            raise RuntimeError(f"muon_step_groups failed: {rc} {L.muon_last_error()}")

    if args.copy_calibration_mib > 0:
        calibration_pass(args.copy_calibration_mib, dev)
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done", file=sys.stderr, flush=True)

    # In the timed region only the update GEMM (the roofline's kernel) is
    # bracketed by events: every event pair serializes the launch boundaries
    # it sits on.
    ns.profile_reset()
    ns.profile_classes(["update"])
    ns.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    # One event between consecutive steps: the per-step times give the
    # median, min and p90 beside the mean.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        one_step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ns.profile_enable(False)
    ms_total = evs[0].elapsed_time(evs[-1])
    ms_per_step = ms_total / args.steps
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step (wall {wall:.2f} s)",
          file=sys.stderr, flush=True)

    upd = ns.profile_query("update")
    # The same number of steps again without any launch events (informative).
    ev2 = torch.cuda.Event(enable_timing=True)
    ev3 = torch.cuda.Event(enable_timing=True)
    ev2.record(stream)
    for _ in range(args.steps):
        one_step()
    ev3.record(stream)
    torch.cuda.synchronize()
    ms_plain = ev2.elapsed_time(ev3) / args.steps
    print(f"[bench] {args.steps} more steps without launch events: {ms_plain:.3f} ms/step", file=sys.stderr,
          flush=True)
    # The per-class table: the same number of steps with events around every launch.
    ns.profile_reset()
    ns.profile_classes(None)
    ns.profile_enable(True)
    for _ in range(args.steps):
        one_step()
    torch.cuda.synchronize()
    ns.profile_enable(False)
    prof = {k: ns.profile_query(k) for k in ns.KERNEL_CLASSES}
    upd_avg_ms = upd["ms"] / max(upd["launches"], 1)
    upd_tflops = upd["flop"] / (upd["ms"] * 1e-3) / 1e12 if upd["ms"] > 0 else 0.0

    nmat = len(LAYER) * args.layers
    fl_L = args.layers * sum(ns_flops(*s)[0] for _, s in LAYER)
    fl_E = args.layers * sum(ns_flops(*s)[1] for _, s in LAYER)
    value = nmat / (ms_per_step * 1e-3)
    tf_L = fl_L / (ms_per_step * 1e-3) / 1e12
    tf_E = fl_E / (ms_per_step * 1e-3) / 1e12
    per_class = class_table(prof)
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "orth/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("llama3-8b-layer-muon-normuon-step" if args.layers == 1
                         else f"llama3-8b-{args.layers}-layer-muon-normuon-step"),
            "matrices": nmat,
            "groups": [f"{len(gr['names'])}x{gr['shape'][0]}x{gr['shape'][1]}" for gr in groups],
            "ns_iterations": 5,
            "ns_compute": "bf16 storage, fp32 accumulate (MFMA)",
            "normuon": True,
            "step_ms": step_stats(per_step),
            "tflops_L": round(tf_L, 2), "pct_peak_L": round(100 * tf_L / PEAK_BF16_TFLOPS, 2),
            "tflops_E": round(tf_E, 2), "pct_peak_E": round(100 * tf_E / PEAK_BF16_TFLOPS, 2),
            "flop_per_step_L": fl_L, "flop_per_step_E": fl_E,
            "kernel_classes": per_class,
            "timed_region": "HIP events around every update-GEMM launch (they give the roofline's kernel time); "
                            "kernel_classes comes from a further pass with events around every launch",
            "ms_per_step_without_launch_events": round(ms_plain, 4),
        },
        "roofline": {
            "bound": "mfma",
            "kernel": f"update GEMM X' = B X + a X, all {nmat} matrices per launch (gemm_nt_bf16_kernel<256, false, true, 8>)",
            "achieved": round(upd_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(upd_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_for("update") if args.layers == 1 else None,
            "launches": upd["launches"],
            "avg_launch_us": round(upd_avg_ms * 1e3, 2),
            "flop_per_launch": upd["flop"] / max(upd["launches"], 1),
        },
    }
    if not args.no_cpu_baseline:
        if args.layers != 1:
            grads, weights = make_layer_inputs()
        print("[bench] timing the oracle on the CPU", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(grads, weights, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
