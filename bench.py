"""Benchmark: effective convolution TFLOP/s on one MI355X.

Default workload: the largest configuration, the Overfeat-fast-style fp32
NCHW stack at batch 128 (L1: 3->96, 231x231, 11x11/s4; L2: 96->256, 24x24,
5x5/s1; L3-L5: 256->512->1024->1024, 12x12, 3x3/s1/pad1; 656.2 GFLOP per
step), synthetic seeded inputs (uniform[-1,1] data, N(0, 0.01) weights).
One step = the workload's forward passes, each one kernel launch of
libmiconv through the C ABI.

Timing: W warm-up steps, then five timed regions of exactly K steps each,
every region bracketed by torch.cuda.synchronize() on both sides;
``ms_per_step`` and ``value`` come from the median region (all five are
reported).  Per-layer kernel times: HIP events on the launch stream around
back-to-back launches, median of five regions; every layer gets the same
launch count, which makes its shortest region at least 100 ms.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
                    [--workload overfeat|alexnet|speech|tiny|prec_f64|prec_bf16|alexnet_pool|
                                alexnet_fc|alexnet_fc_f64|alexnet_fc_bf16]
                    [--op fprop|dgrad|wgrad]

Prints one JSON line.  ``value`` = 2*N*K*C*R*S*P*Q summed over the step's
layers / median-region step time (inputs resident in HBM, no host traffic
inside the timed region).  ``roofline`` covers the kernel with the most time per
step, timed with HIP events on the stream it runs on.  ``cpu_baseline``
times the CPU oracle on a bounded sample of the same workload (the first
few images of every layer).  ``--op dgrad`` / ``--op wgrad`` time the data /
filter gradient of the same layers instead (dy seeded uniform [-1, 1]; the
same FLOP count).  ``--workload alexnet_pool`` times AlexNet's two max-pooling
layers (after conv2 and conv5) and reports bandwidth (|x| + |y| per second)
against the HBM roofline.  ``--block B`` runs the forward pass on
channel-blocked x, filters and y (blocks of B channels).  ``--workload alexnet_fc`` times AlexNet's
fully-connected layers fc6-fc8 at minibatch 128 as batch-reduce GEMMs
(``_f64`` / ``_bf16``: fc6 in that type), 2*m*n*k*batch FLOP per layer.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X dense MFMA peaks (256 CU x 2.4 GHz): fp32 256, fp64 128, bf16 4096 FLOP/clk/CU
MFMA_PEAK_TFLOPS = {"f32": 157.3, "f64": 78.6, "bf16": 2516.6}
# committed rocprofv3 counter summaries, per workload (HBM bytes per launch of the dominant kernel)
PROFILE_TRAFFIC = {"overfeat": os.path.join(ROOT, "profiles", "traffic_overfeat_fp32.md")}
WORKLOADS = ("alexnet", "overfeat", "speech", "tiny", "prec_f64", "prec_bf16", "alexnet_pool", "alexnet_fc",
             "alexnet_fc_f64", "alexnet_fc_bf16")
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=25,
                    help="steps per timed region (five regions; the default keeps an Overfeat region above 100 ms)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="overfeat", choices=WORKLOADS)
    ap.add_argument("--op", default="fprop", choices=("fprop", "dgrad", "wgrad"),
                    help="forward pass (default), data gradient or filter gradient of the layers")
    ap.add_argument("--block", type=int, default=0,
                    help="forward pass on channel-blocked x, filters and y with this block "
                         "(x [N][C/b][H][W][b], filters [K/b][C/b][R][S][b][b], y [N][K/b][P][Q][b]); "
                         "a tensor whose channel count b does not divide stays unblocked")
    ap.add_argument("--layer-reps", type=int, default=0,
                    help="launches per region of the per-layer timing (default 0: enough for the "
                         "shortest layer's region to last 100 ms; counter runs use a few)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before the steps, run one plain device copy of this many MiB, its "
                         "source first pushed out of the caches by a write of as many MiB "
                         "(a known-size kernel to scale rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    return ap.parse_args()


def workload_layers(name):
    from gen import workloads
    if name == "alexnet":
        return workloads.ALEXNET, "alexnet_conv2-5_fp32_nchw_n128"
    if name == "overfeat":
        return workloads.OVERFEAT, "overfeat_l1-5_fp32_nchw_n128"
    if name == "speech":
        return workloads.SPEECH, "speech_l1-2_fp32_nchw_n32"
    if name == "tiny":
        return workloads.TINY, "tiny_fp32_nchw_n2"
    if name == "prec_f64":
        return [l for l in workloads.PRECISION if l.dtype == "f64"], \
            "alexnet_conv3-5_fp64_nchw+nhwc_pitch16_n64"
    return [l for l in workloads.PRECISION if l.dtype == "bf16"], \
        "alexnet_conv3-5_bf16in_fp32acc_nchw+nhwc_pitch16_n64"


# the sources that define the fp32 halo kernels (the default workload's dominant kernel)
TRAFFIC_SOURCES = ("conv_fwd_halo.hip", "mfma_common.h", "conv_params.h", "tile_map.h")


def source_hash():
    """Hash of the halo kernels' sources, to tie stored counter readings to them."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "convolution_forward_conv2d_amd", "csrc")
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary of the
    workload, if it was taken on this exact source and kernel; else None."""
    path = PROFILE_TRAFFIC.get(workload)
    if not path or not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic:"):
                for kv in line[len("traffic:"):].split():
                    k, _, v = kv.partition("=")
                    vals[k] = v
    if vals.get("source") != source_hash() or vals.get("kernel") != kernel:
        return None
    try:
        return float(vals["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


REGIONS = 5
MIN_REGION_S = 0.1


def timed_regions(torch, step, steps):
    """Wall time (s) of REGIONS regions of exactly `steps` steps, each bracketed by
    torch.cuda.synchronize() on both sides."""
    out = []
    for _ in range(REGIONS):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        out.append(time.perf_counter() - t0)
    return out


def region_reps(torch, stream, launches):
    """Back-to-back launches per timed region such that the region of the
    shortest launch lasts at least MIN_REGION_S.  Every launch of the step
    gets the same count, so a profiler's per-kernel average over the whole
    run weights the layers alike, as the per-launch averages here do."""
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    shortest = None
    for launch in launches:
        launch()
        ev0.record(stream)
        launch()
        ev1.record(stream)
        ev1.synchronize()
        one = max(ev0.elapsed_time(ev1), 1e-3)
        shortest = one if shortest is None else min(shortest, one)
    return max(5, int(MIN_REGION_S * 1e3 / shortest) + 1)


def event_ms(torch, stream, launch, reps):
    """Median over REGIONS of one launch's mean duration (ms), from HIP events
    recorded on the launch stream around `reps` back-to-back launches."""
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    launch()
    res = []
    for _ in range(REGIONS):
        ev0.record(stream)
        for _ in range(reps):
            launch()
        ev1.record(stream)
        ev1.synchronize()
        res.append(ev0.elapsed_time(ev1) / reps)
    return sorted(res)[len(res) // 2]


def copy_probe(torch, dev, mib):
    """One plain device copy of `mib` MiB whose source has been pushed out of the
    L2 and the 256 MB last-level cache by a write of another `mib` MiB: the
    known-size reference that scales the FETCH_SIZE / WRITE_SIZE counters."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    evict = torch.empty_like(src)
    evict.fill_(2.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst, evict


def upload(a64, dtype, layout, row_pitch, dev):
    """Logical N,C,H,W float64 data -> device tensor in the layer's storage layout."""
    import torch
    from gen import workloads
    tdt = {"f32": torch.float32, "f64": torch.float64, "bf16": torch.bfloat16}[dtype]
    N, C, H, W = a64.shape
    st = workloads.padded_strides(N, C, H, W, layout, row_pitch)
    base = torch.zeros(workloads.storage_elems(N, C, H, W, st), dtype=tdt, device=dev)
    t = base.as_strided(a64.shape, st)
    t.copy_(torch.from_numpy(a64).to(tdt))
    return t


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import convolution_forward_conv2d_amd as mic
    import gen
    from gen import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    if args.workload == "alexnet_pool":
        return bench_pool(args, torch, mic, gen, workloads, dev)
    if args.workload.startswith("alexnet_fc"):
        return bench_fc(args, torch, mic, gen, workloads, dev)
    layers, wl_name = workload_layers(args.workload)
    dtype = layers[0].dtype
    peak = MFMA_PEAK_TFLOPS[dtype]
    out_dt = torch.float64 if dtype == "f64" else torch.float32
    plans = []
    cache = {}
    for lay in layers:
        key = (lay.config, lay.layer)
        if key not in cache:       # precision variants share their logical values
            cache.clear()
            x = gen.round_to(gen.draw(lay.x_dist, gen.derive_seed(lay.config, lay.layer, 0), lay.x_shape), dtype)
            w = gen.round_to(gen.draw(lay.w_dist, gen.derive_seed(lay.config, lay.layer, 1), lay.w_shape), dtype)
            cache[key] = (x, w)
        x, w = cache[key]
        N, K, P, Q = mic.output_shape(lay.x_shape, lay.w_shape, lay.stride, lay.padding)
        wt = torch.from_numpy(w).to({"f32": torch.float32, "f64": torch.float64,
                                     "bf16": torch.bfloat16}[dtype]).to(dev)
        if args.op == "fprop" and args.block:
            # block every tensor whose channel count the block divides (exact
            # blocks); the others stay NCHW / packed KCRS
            b = args.block
            C = lay.C
            xt = torch.from_numpy(x).to(wt.dtype).to(dev)
            xt = mic.to_blocked(xt, b) if C % b == 0 else xt
            wb = mic.filters_to_blocked(wt, b, b) if C % b == 0 and K % b == 0 else wt
            yt = (torch.zeros((N, K // b, P, Q, b), dtype=out_dt, device=dev) if K % b == 0
                  else torch.zeros((N, K, P, Q), dtype=out_dt, device=dev))
            plans.append((lay, mic.BlockedConvPlan(xt, wb, yt, lay.stride, lay.padding), (x, w)))
        elif args.op == "fprop":
            xt = upload(x, dtype, lay.layout, lay.row_pitch, dev)
            yst = workloads.padded_strides(N, K, P, Q, lay.layout, lay.row_pitch)
            yt = torch.zeros(workloads.storage_elems(N, K, P, Q, yst), dtype=out_dt,
                             device=dev).as_strided((N, K, P, Q), yst)
            plans.append((lay, mic.ConvPlan(xt, wt, yt, lay.stride, lay.padding), (x, w)))
        elif args.op == "wgrad":
            xt = upload(x, dtype, lay.layout, lay.row_pitch, dev)
            dy = gen.round_to(gen.uniform(gen.derive_seed(lay.config, lay.layer, 3), (N, K, P, Q)), dtype)
            dyt = upload(dy, dtype, lay.layout, lay.row_pitch, dev)
            dwt = torch.zeros(lay.w_shape, dtype=out_dt, device=dev)
            plans.append((lay, mic.WgradPlan(xt, dyt, dwt, lay.stride, lay.padding), (x, dy)))
        else:
            dy = gen.round_to(gen.uniform(gen.derive_seed(lay.config, lay.layer, 3), (N, K, P, Q)), dtype)
            dyt = upload(dy, dtype, lay.layout, lay.row_pitch, dev)
            xst = workloads.padded_strides(*lay.x_shape, lay.layout, lay.row_pitch)
            dxt = torch.zeros(workloads.storage_elems(*lay.x_shape, xst), dtype=out_dt,
                              device=dev).as_strided(lay.x_shape, xst)
            plans.append((lay, mic.DgradPlan(dyt, wt, dxt, lay.stride, lay.padding), (dy, w)))
    stream = torch.cuda.current_stream(dev)
    flops_step = sum(p.flops for _, p, _ in plans)
    if args.copy_probe_mib:
        copy_probe(torch, dev, args.copy_probe_mib)

    def step():
        for _, plan, _ in plans:
            plan(1.0, 0.0, stream)

    for _ in range(args.warmup):
        step()
    regions = timed_regions(torch, step, args.steps)
    elapsed = sorted(regions)[len(regions) // 2]
    ms_per_step = 1e3 * elapsed / args.steps
    value = flops_step / (elapsed / args.steps) / 1e12

    # per-layer kernel durations with HIP events on the launch stream
    per_layer = []
    reps = args.layer_reps or region_reps(torch, stream, [lambda plan=plan: plan(1.0, 0.0, stream) for _, plan, _ in plans])
    for lay, plan, _ in plans:
        ms = event_ms(torch, stream, lambda: plan(1.0, 0.0, stream), reps)
        tf = plan.flops / (ms * 1e-3) / 1e12
        rec = {"layer": lay.name, "kernel": plan.kernel_name(), "us": round(ms * 1e3, 2),
               "gflop": round(plan.flops / 1e9, 3), "tflops": round(tf, 2),
               "pct_mfma_peak": round(100 * tf / peak, 1)}
        if isinstance(plan, mic.BlockedConvPlan):
            rec["blocked"] = {"x": plan.x.dim() == 5, "w": plan.w.dim() == 6, "y": plan.y.dim() == 5}
        per_layer.append(rec)

    # dominant kernel: most time per step, launches grouped by kernel variant
    groups = {}
    for rec, (_, plan, _) in zip(per_layer, plans):
        g = groups.setdefault(rec["kernel"], {"us": 0.0, "flops": 0.0, "launches": 0})
        g["us"] += rec["us"]
        g["flops"] += plan.flops
        g["launches"] += 1
    dom = max(groups, key=lambda k: groups[k]["us"])
    g = groups[dom]
    achieved = (g["flops"] / g["launches"]) / (g["us"] / g["launches"] * 1e-6) / 1e12
    traffic = stored_traffic(args.workload, dom) if (args.op == "fprop" and not args.block) else None
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": traffic, "kernel": dom, "launches_per_step": g["launches"],
                "avg_us": round(g["us"] / g["launches"], 2)}

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(plans, args.cpu_seconds, args.op)

    line = {
        "metric": "effective conv TFLOP/s (2NKCRSPQ/t) per layer + % of MFMA peak, 1 MI355X",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "regions_ms": [round(1e3 * r, 3) for r in regions],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded inputs with the workload's value distributions)",
        "config": {"workload": (wl_name if args.op == "fprop" else wl_name + "_" + args.op) +
                               ("_blocked%d" % args.block if args.block else ""), "op": args.op,
                   "global_batch": layers[0].N,
                   "layers": [l.name for l in layers], "gflop_per_step": round(flops_step / 1e9, 3),
                   "pct_mfma_peak": round(100 * value / peak, 1)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "layers": per_layer,
    }
    print(json.dumps(line), flush=True)
    for _, plan, _ in plans:
        plan.close()


def bench_pool(args, torch, mic, gen, workloads, dev):
    """AlexNet's max-pooling layers: bandwidth against the HBM roofline."""
    plans = []
    for lay in workloads.POOLING:
        x = gen.round_to(gen.uniform(gen.derive_seed(lay.config, lay.layer, 0), lay.x_shape), lay.dtype)
        xt = upload(x, lay.dtype, lay.layout, lay.row_pitch, dev)
        shape = mic.pool_output_shape(lay.x_shape, (lay.R, lay.S), lay.stride, lay.padding)
        yt = torch.zeros(shape, dtype=torch.float32, device=dev)
        plans.append((lay, mic.PoolPlan(xt, yt, (lay.R, lay.S), lay.stride, lay.padding, "max"), x))
    stream = torch.cuda.current_stream(dev)
    bytes_step = sum(p.bytes for _, p, _ in plans)

    def step():
        for _, plan, _ in plans:
            plan(1.0, 0.0, stream)

    for _ in range(args.warmup):
        step()
    regions = timed_regions(torch, step, args.steps)
    elapsed = sorted(regions)[len(regions) // 2]
    per_layer = []
    reps = args.layer_reps or region_reps(torch, stream, [lambda plan=plan: plan(1.0, 0.0, stream) for _, plan, _ in plans])
    for lay, plan, _ in plans:
        us = event_ms(torch, stream, lambda: plan(1.0, 0.0, stream), reps) * 1e3
        per_layer.append({"layer": lay.name, "kernel": plan.kernel_name(), "us": round(us, 2),
                          "mb": round(plan.bytes / 1e6, 2), "gbs": round(plan.bytes / (us * 1e-6) / 1e9, 1)})
    dom = max(per_layer, key=lambda r: r["us"])
    cpu = None
    if not args.no_cpu:
        import oracle
        lay, plan, x = plans[0]
        n = max(1, min(lay.N, int(args.cpu_seconds / 0.05)))
        t0 = time.perf_counter()
        oracle.pool2d_forward(x[:n], (lay.R, lay.S), lay.stride, lay.padding, "max")
        dt = time.perf_counter() - t0
        cpu = {"value": round(plan.bytes * n / lay.N / dt / 1e9, 3), "unit": "GB/s",
               "cores": oracle.default_threads(), "kind": "oracle",
               "sample": "first %d of %d images of %s (%.2f s)" % (n, lay.N, lay.name, dt)}
    value = bytes_step / (elapsed / args.steps) / 1e9
    line = {
        "metric": "pooling bandwidth ((|x|+|y|)/t), 1 MI355X",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded uniform [-1, 1])",
        "config": {"workload": "alexnet_pool2+pool5_max_fp32_nchw_n128", "op": "pool",
                   "layers": [l.name for l, _, _ in plans]},
        "roofline": {"bound": "hbm", "achieved": dom["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom["gbs"] / HBM_PEAK_GBS, 4), "traffic": None, "kernel": dom["kernel"],
                     "avg_us": dom["us"]},
        "cpu_baseline": cpu,
        "layers": per_layer,
    }
    print(json.dumps(line), flush=True)
    for _, plan, _ in plans:
        plan.close()


def bench_fc(args, torch, mic, gen, workloads, dev):
    """AlexNet's fully-connected layers as batch-reduce GEMMs: TFLOP/s against the MFMA roofline."""
    if args.workload == "alexnet_fc":
        layers = [workloads.fc_by_name(n) for n in ("alexnet_fc6", "alexnet_fc7", "alexnet_fc8")]
        wl_name = "alexnet_fc6-8_fp32_n128"
    elif args.workload == "alexnet_fc_f64":
        layers, wl_name = [workloads.fc_by_name("alexnet_fc6_f64")], "alexnet_fc6_fp64_n128"
    else:
        layers, wl_name = [workloads.fc_by_name("alexnet_fc6_bf16")], "alexnet_fc6_bf16in_fp32acc_n128"
    dtype = layers[0].dtype
    tdt = {"f32": torch.float32, "f64": torch.float64, "bf16": torch.bfloat16}[dtype]
    odt = torch.float64 if dtype == "f64" else torch.float32
    peak = MFMA_PEAK_TFLOPS[dtype]
    runs = []
    for lay in layers:
        F = lay.features
        x = gen.round_to(gen.draw(lay.x_dist, gen.derive_seed(lay.config, lay.layer, 0), (lay.m, F)), dtype)
        w = gen.round_to(gen.draw(lay.w_dist, gen.derive_seed(lay.config, lay.layer, 1), (lay.n, F)), dtype)
        xt = torch.from_numpy(x).to(tdt).to(dev)
        wt = torch.from_numpy(w).to(tdt).to(dev)
        a = xt.as_strided((lay.batch, lay.m, lay.k), (lay.k, F, 1))
        b = wt.as_strided((lay.batch, lay.k, lay.n), (lay.k, 1, F))
        c = torch.zeros((lay.m, lay.n), dtype=odt, device=dev)
        flops = 2.0 * lay.m * lay.n * F
        runs.append((lay, a, b, c, flops, x, w))
    # algorithmic HBM bytes of a layer: A and B read once, C written once
    esz = {"f32": 4, "f64": 8, "bf16": 2}[dtype]
    osz = 8 if dtype == "f64" else 4
    hbm_bytes = {r[0].name: esz * (r[0].m + r[0].n) * r[0].features + osz * r[0].m * r[0].n for r in runs}
    stream = torch.cuda.current_stream(dev)
    flops_step = sum(r[4] for r in runs)

    def step():
        for _, a, b, c, _, _, _ in runs:
            mic.brgemm(a, b, c)

    for _ in range(args.warmup):
        step()
    regions = timed_regions(torch, step, args.steps)
    elapsed = sorted(regions)[len(regions) // 2]
    per_layer = []
    reps = args.layer_reps or region_reps(torch, stream, [lambda r=r: mic.brgemm(r[1], r[2], r[3]) for r in runs])
    for lay, a, b, c, flops, _, _ in runs:
        us = event_ms(torch, stream, lambda: mic.brgemm(a, b, c), reps) * 1e3
        per_layer.append({"layer": lay.name, "kernel": mic.brgemm_kernel_name_for(a, b, c),
                          "us": round(us, 2), "tflops": round(flops / (us * 1e-6) / 1e12, 2),
                          "gbs": round(hbm_bytes[lay.name] / (us * 1e-6) / 1e9, 1),
                          "flop_per_byte": round(flops / hbm_bytes[lay.name], 1)})
    dom = max(per_layer, key=lambda r: r["us"])
    # the dominant layer's bound: MFMA when its FLOP per HBM byte exceeds the
    # ridge point (peak FLOP/s over peak bytes/s), else HBM
    ridge = peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    if dom["flop_per_byte"] >= ridge:
        roof = {"bound": "mfma", "achieved": dom["tflops"], "peak": peak, "unit": "TFLOP/s",
                "frac": round(dom["tflops"] / peak, 4)}
    else:
        roof = {"bound": "hbm", "achieved": dom["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom["gbs"] / HBM_PEAK_GBS, 4)}
    roof.update({"traffic": None, "kernel": dom["kernel"], "avg_us": dom["us"], "ridge_flop_per_byte": round(ridge, 1)})
    cpu = None
    if not args.no_cpu:
        import numpy as np
        import oracle
        lay, _, _, _, flops, x, w = runs[0]

        def ora(rows):
            xa = np.ascontiguousarray(x[:rows].reshape(rows, lay.batch, lay.k).transpose(1, 0, 2))
            wb = np.ascontiguousarray(w.reshape(lay.n, lay.batch, lay.k).transpose(1, 2, 0))
            t = time.perf_counter()
            oracle.brgemm(xa, wb)
            return time.perf_counter() - t

        t1 = ora(1)
        rows = int(max(1, min(lay.m, args.cpu_seconds / max(t1, 1e-9))))
        dt = ora(rows) if rows > 1 else t1
        cpu = {"value": round(flops * rows / lay.m / dt / 1e12, 5), "unit": "TFLOP/s",
               "cores": oracle.default_threads(), "kind": "oracle",
               "sample": "first %d of %d rows of %s (%.2f s)" % (rows, lay.m, lay.name, dt)}
    value = flops_step / (elapsed / args.steps) / 1e12
    line = {
        "metric": "fully-connected layer throughput as batch-reduce GEMM (2*m*n*k/t), 1 MI355X",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic (seeded uniform [-1, 1] inputs, He-normal weights)",
        "config": {"workload": wl_name, "op": "brgemm", "layers": [r[0].name for r in runs]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "layers": per_layer,
    }
    print(json.dumps(line), flush=True)


def run_oracle(op, lay, a, w):
    """One oracle call on images a (x for the forward pass, dy for the data gradient)."""
    import oracle
    if op == "fprop":
        return oracle.conv2d_fprop(a, w, lay.stride, lay.padding)
    if op == "wgrad":       # (a, w) = (x, dy) images
        return oracle.conv2d_bwd_filter(a, w[:a.shape[0]], lay.w_shape, lay.stride, lay.padding)
    return oracle.conv2d_bwd_data(a, w, (a.shape[0],) + tuple(lay.x_shape[1:]), lay.stride, lay.padding)


def cpu_baseline(plans, target_s, op="fprop"):
    """The oracle as it is, on the first n images of every layer of the step."""
    import oracle
    threads = oracle.default_threads()
    # calibrate on one image of the first layer, then size the sample
    lay, plan, (x, w) = plans[0]
    t0 = time.perf_counter()
    run_oracle(op, lay, x[:1], w)
    t1 = time.perf_counter() - t0
    per_image = t1 * sum(p.flops / l.N for l, p, _ in plans) / (plan.flops / lay.N)
    n_max = min(l.N for l, _, _ in plans)
    n_img = int(max(1, min(n_max, target_s / max(per_image, 1e-9))))
    flops = 0.0
    done = set()
    t0 = time.perf_counter()
    for lay, plan, (x, w) in plans:
        key = (lay.config, lay.layer)
        if key in done:            # one oracle run per logical layer (layouts share values)
            continue
        done.add(key)
        run_oracle(op, lay, x[:n_img], w)
        flops += plan.flops * n_img / lay.N
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "first %d of %d images of each of the %d layers (%.1f GFLOP, %.1f s, fp64 "
                      "7-loop with the error bound)" % (n_img, n_max, len(done), flops / 1e9, dt)}


if __name__ == "__main__":
    main()
