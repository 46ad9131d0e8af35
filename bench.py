"""Benchmark: effective convolution TFLOP/s on one MI355X.

Workload: the AlexNet-style fp32 NCHW stack at batch 128 (conv2: 96->256,
27x27, 5x5/s1/pad2; conv3: 256->384, conv4: 384->384, conv5: 384->256, all
13x13, 3x3/s1/pad1), synthetic seeded inputs (uniform[-1,1] data,
He-normal weights).  One step = the four layers' forward passes, each one
kernel launch of libmiconv through the C ABI.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

Prints one JSON line.  ``value`` = 2*N*K*C*R*S*P*Q summed over the step's
layers / mean step time (inputs resident in HBM, no host traffic inside
the timed region).  ``roofline`` covers the kernel with the most time per
step, timed with HIP events on the stream it runs on.  ``cpu_baseline``
times the CPU oracle on a bounded sample of the same workload (the first
few images of every layer).
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP32_MFMA_PEAK_TFLOPS = 157.3      # MI355X dense fp32 matrix peak (256 CU x 256 FLOP/clk x 2.4 GHz)
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_alexnet_fp32.md")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before the steps, run one plain device copy of this many MiB "
                         "(a known-size kernel to scale rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    return ap.parse_args()


def source_hash():
    """Hash of the kernel sources, to tie stored counter readings to this build."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "convolution_forward_conv2d_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on this exact source and kernel; else None."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    vals = {}
    with open(PROFILE_TRAFFIC) as fh:
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
    layers = workloads.ALEXNET
    plans = []
    for lay in layers:
        x = gen.round_to(gen.draw(lay.x_dist, gen.derive_seed(lay.config, lay.layer, 0), lay.x_shape), "f32")
        w = gen.round_to(gen.draw(lay.w_dist, gen.derive_seed(lay.config, lay.layer, 1), lay.w_shape), "f32")
        xt = torch.from_numpy(x).float().to(dev)
        wt = torch.from_numpy(w).float().to(dev)
        N, K, P, Q = mic.output_shape(lay.x_shape, lay.w_shape, lay.stride, lay.padding)
        yt = torch.empty((N, K, P, Q), dtype=torch.float32, device=dev)
        plans.append((lay, mic.ConvPlan(xt, wt, yt, lay.stride, lay.padding), (x, w)))
    stream = torch.cuda.current_stream(dev)
    flops_step = sum(p.flops for _, p, _ in plans)
    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        for _, plan, _ in plans:
            plan(1.0, 0.0, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    value = flops_step / (elapsed / args.steps) / 1e12

    # per-layer kernel durations with HIP events on the launch stream
    per_layer = []
    reps = max(5, args.steps)
    for lay, plan, _ in plans:
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        plan(1.0, 0.0, stream)
        ev0.record(stream)
        for _ in range(reps):
            plan(1.0, 0.0, stream)
        ev1.record(stream)
        ev1.synchronize()
        ms = ev0.elapsed_time(ev1) / reps
        tf = plan.flops / (ms * 1e-3) / 1e12
        per_layer.append({"layer": lay.name, "kernel": plan.kernel_name(), "us": round(ms * 1e3, 2),
                          "gflop": round(plan.flops / 1e9, 3), "tflops": round(tf, 2),
                          "pct_fp32_mfma_peak": round(100 * tf / FP32_MFMA_PEAK_TFLOPS, 1)})

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
    traffic = stored_traffic(dom)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": FP32_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / FP32_MFMA_PEAK_TFLOPS, 4),
                "traffic": traffic, "kernel": dom, "launches_per_step": g["launches"],
                "avg_us": round(g["us"] / g["launches"], 2)}

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(plans, args.cpu_seconds)

    line = {
        "metric": "effective conv TFLOP/s (2NKCRSPQ/t) per layer + % of MFMA peak, 1 MI355X",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded uniform[-1,1] inputs, He-normal weights)",
        "config": {"workload": "alexnet_conv2-5_fp32_nchw_n128", "global_batch": 128,
                   "layers": [l.name for l in layers], "gflop_per_step": round(flops_step / 1e9, 3),
                   "pct_fp32_mfma_peak": round(100 * value / FP32_MFMA_PEAK_TFLOPS, 1)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "layers": per_layer,
    }
    print(json.dumps(line), flush=True)
    for _, plan, _ in plans:
        plan.close()


def cpu_baseline(plans, target_s):
    """The oracle as it is, on the first n images of every layer of the step."""
    import oracle
    threads = oracle.default_threads()
    # calibrate on one image of the first layer, then size the sample
    lay, plan, (x, w) = plans[0]
    t0 = time.perf_counter()
    oracle.conv2d_fprop(x[:1], w, lay.stride, lay.padding)
    t1 = time.perf_counter() - t0
    per_image = t1 * sum(p.flops for _, p, _ in plans) / plans[0][1].flops
    n_img = int(max(1, min(lay.N, target_s / max(per_image, 1e-9))))
    flops = 0.0
    t0 = time.perf_counter()
    for lay, plan, (x, w) in plans:
        oracle.conv2d_fprop(x[:n_img], w, lay.stride, lay.padding)
        flops += plan.flops * n_img / lay.N
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "first %d of 128 images of each of the 4 layers (%.1f GFLOP, %.1f s, fp64 "
                      "7-loop with the error bound)" % (n_img, flops / 1e9, dt)}


if __name__ == "__main__":
    main()
