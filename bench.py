#!/usr/bin/env python3
"""Benchmark: grouped conv fwd+bwd fp32 TFLOP/s (NCHW) and % of MFMA/HBM roofline.

One step = the whole path on one batch of synthetic input already resident in
HBM: forward (+bias), gradInput, gradWeight and gradBias, each one call
through the C-ABI library on torch's current HIP stream.
  value  = 3 * FLOP_conv * steps / (time of the timed steps)       [TFLOP/s]
  FLOP_conv = 2*N*K*Ho*Wo*(C/G)*kh*kw (the standard count, padded taps included)
The default workload is the dense 3x3 64->64 56x56 batch-32 convolution.
Per op, HIP events bracket every launch in a second timed region of eager
steps; the op with the largest total time is the "dominant kernel" of the
roofline object. The CPU baseline times the fp64 oracle on a bounded sample
(the first images of the same batch) on this host's cores.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload dense3x3]
                    [--all-workloads] [--no-cpu-baseline] [--launch graph|eager]

Each timed step issues the four C-ABI calls; --launch graph replays one HIP
graph holding the step's four launches instead (captured once from prepared
plans), which takes the host's launch cost out of small workloads. Per-op
times come from a second timed region of eager steps with events around each
launch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_F32 = 157.3e12      # MI355X dense fp32 matrix (MFMA) FLOP/s
PEAK_VALU_F32 = 157.3e12      # MI355X fp32 vector FLOP/s (published, packed FMA)
PEAK_HBM = 8.0e12             # MI355X HBM3E bytes/s
RIDGE = PEAK_MFMA_F32 / PEAK_HBM
OPS = ("fwd", "bwd_data", "bwd_filter", "bwd_bias")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def conv_flop(wl, Ho, Wo):
    N, C, H, W = wl.x_shape
    K, Cg, kh, kw = wl.w_shape
    return 2.0 * N * K * Ho * Wo * Cg * kh * kw


def op_bytes(wl, Ho, Wo, has_bias):
    """Compulsory fp32 HBM traffic per op (each tensor read or written once)."""
    N, C, H, W = wl.x_shape
    K, Cg, kh, kw = wl.w_shape
    x, w, y = N * C * H * W, K * Cg * kh * kw, N * K * Ho * Wo
    return {"fwd": 4.0 * (x + w + y + (K if has_bias else 0)),
            "bwd_data": 4.0 * (y + w + x),
            "bwd_filter": 4.0 * (x + y + w),
            "bwd_bias": 4.0 * (y + K)}


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_tag):
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE and
    WRITE_SIZE, scaled by the copy-kernel calibration), if recorded for the
    current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel_tag)
    if not rec:
        return None
    srcs = [os.path.join(ROOT, p) for p in rec["sources"]]
    if not all(os.path.exists(p) for p in srcs) or source_digest(srcs) != rec["source_digest"]:
        return None
    return float(rec["bytes_per_launch"])


def run_gpu(args, wl_name):
    import torch
    import grouped_convolution_amd as G
    from grouped_convolution_amd.workloads import WORKLOADS, make_inputs

    wl = WORKLOADS[wl_name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(wl_name)
    # make_inputs gives NCHW arrays; channels-last workloads store them transposed.
    store = (lambda a: np.ascontiguousarray(a.transpose(0, 2, 3, 1))) if wl.layout == "nhwc" else (lambda a: a)
    x = torch.from_numpy(store(inp["x"])).to(dev)
    w = torch.from_numpy(inp["w"]).to(dev)
    b = None if inp["b"] is None else torch.from_numpy(inp["b"]).to(dev)
    dy = torch.from_numpy(store(inp["dy"])).to(dev)
    kw = dict(stride=wl.stride, padding=wl.padding, dilation=wl.dilation, groups=wl.groups,
              layout=wl.layout)
    N, C, H, W = wl.x_shape
    K, Cg, kh, kwid = wl.w_shape
    desc = G.make_desc(N, C, H, W, K, kh, kwid, **kw)
    Ho, Wo = G.gconv_output_dims(desc)
    y = torch.empty((N, Ho, Wo, K) if wl.layout == "nhwc" else (N, K, Ho, Wo), device=dev)
    dx = torch.empty_like(x)
    dw = torch.empty_like(w)
    db = torch.empty((K,), device=dev)
    plans = {
        "fwd": G.Plan.fwd(x, w, b, y, **kw),
        "bwd_data": G.Plan.bwd_data(dy, w, dx, **kw),
        "bwd_filter": G.Plan.bwd_filter(x, dy, dw, **kw),
        "bwd_bias": G.Plan.bwd_bias(dy, db, layout=wl.layout),
    }
    paths = {op: G.PATH_NAMES[G.gconv_select_path(desc, i)] for i, op in enumerate(OPS)}
    for _ in range(args.warmup):
        for op in OPS:
            plans[op]()
    torch.cuda.synchronize()

    K_steps = args.steps

    # Timed region 1 -> `value`: K whole steps, bracketed by synchronisations.
    # By default each step is the four C-ABI calls; with --launch graph it is
    # one replay of a HIP graph holding the four launches (captured once from
    # the prepared plans; every replay recomputes all four results). If the
    # capture fails the calls are issued directly.
    launch = args.launch
    graph = None
    if launch == "graph":
        try:
            cs = torch.cuda.Stream()
            cs.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cs):
                gplans = [G.Plan.fwd(x, w, b, y, **kw), G.Plan.bwd_data(dy, w, dx, **kw),
                          G.Plan.bwd_filter(x, dy, dw, **kw), G.Plan.bwd_bias(dy, db, layout=wl.layout)]
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph, stream=cs):
                    for p in gplans:
                        p()
            torch.cuda.current_stream().wait_stream(cs)
            for _ in range(args.warmup):
                graph.replay()
        except Exception as e:  # launch mode only: the same kernels run eagerly
            log("HIP graph capture failed (%s); timing eager launches" % e)
            graph, launch = None, "eager"
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for s in range(K_steps):
        if graph is not None:
            graph.replay()
        else:
            for op in OPS:
                plans[op]()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)

    # Timed region 2 -> per-op times (the roofline object): K more eager steps
    # with HIP events around every launch on its stream (an event between two
    # launches costs a small pipeline bubble, so these are not summed into
    # `value`).
    ev = {op: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(K_steps)] for op in OPS}
    torch.cuda.synchronize()
    for s in range(K_steps):
        for op in OPS:
            e0, e1 = ev[op][s]
            e0.record()
            plans[op]()
            e1.record()
    torch.cuda.synchronize()
    per_op_ms = {op: sum(a.elapsed_time(b_) for a, b_ in ev[op]) / K_steps for op in OPS}

    flop = conv_flop(wl, Ho, Wo)
    nbytes = op_bytes(wl, Ho, Wo, b is not None)
    ops = {}
    for op in OPS:
        t = per_op_ms[op] * 1e-3
        f = 0.0 if op == "bwd_bias" else flop
        ai = f / nbytes[op]
        if op == "bwd_bias" or paths[op] in ("direct", "smallgroup"):
            bound = "hbm" if ai < RIDGE else "alu"
        else:
            bound = "mfma"
        peak = {"hbm": PEAK_HBM, "alu": PEAK_VALU_F32, "mfma": PEAK_MFMA_F32}[bound]
        achieved = nbytes[op] / t if bound == "hbm" else f / t
        ops[op] = {"ms": round(per_op_ms[op], 5), "path": paths[op],
                   "tflops": round(f / t / 1e12, 3), "gbs": round(nbytes[op] / t / 1e9, 1),
                   "bound": bound, "frac": round(achieved / peak, 4)}
    dom = max(OPS, key=lambda o: per_op_ms[o])
    d = ops[dom]
    t_dom = per_op_ms[dom] * 1e-3
    if d["bound"] == "hbm":
        roof = {"bound": "hbm", "achieved": round(nbytes[dom] / t_dom / 1e9, 1),
                "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": d["bound"], "achieved": round(flop / t_dom / 1e12, 3),
                "peak": (PEAK_MFMA_F32 if d["bound"] == "mfma" else PEAK_VALU_F32) / 1e12,
                "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    tb = traffic_from_profiles("%s:%s:%s" % (wl_name, dom, d["path"]))
    roof["traffic"] = tb
    roof["kernel"] = "%s (%s path)" % (dom, d["path"])
    roof["launch_ms"] = round(per_op_ms[dom], 5)
    roof["algorithmic_per_launch"] = (nbytes[dom] if d["bound"] == "hbm" else flop)

    ms_per_step = total_ms / K_steps
    value = 3.0 * flop / (ms_per_step * 1e-3) / 1e12

    return {
        "value": value, "ms_per_step": ms_per_step, "wall_s": wall, "ops": ops,
        "roofline": roof, "Ho": Ho, "Wo": Wo, "flop_conv": flop, "launch": launch,
        "device": torch.cuda.get_device_name(dev),
    }


def cpu_baseline(wl_name, budget_s=12.0, max_images=None):
    """The fp64 oracle on the first images of the same batch, all four ops per
    image, until about `budget_s` of wall time is spent."""
    import oracle
    from grouped_convolution_amd.workloads import WORKLOADS, make_inputs

    wl = WORKLOADS[wl_name]
    inp = make_inputs(wl_name)
    kw = dict(stride=wl.stride, padding=wl.padding, dilation=wl.dilation, groups=wl.groups)
    N = wl.x_shape[0]
    K, Cg, kh, kwid = wl.w_shape
    Ho, Wo = wl.dy_shape[2], wl.dy_shape[3]
    per_image_flop = 3.0 * 2.0 * K * Ho * Wo * Cg * kh * kwid
    done, t_total = 0, 0.0
    limit = N if max_images is None else min(N, max_images)
    while done < limit and t_total < budget_s:
        sl = slice(done, done + 1)
        x, dy = inp["x"][sl], inp["dy"][sl]
        t0 = time.perf_counter()
        oracle.fwd(x, inp["w"], inp["b"], **kw)
        oracle.bwd_data(dy, inp["w"], x.shape, **kw)
        oracle.bwd_filter(x, dy, inp["w"].shape, **kw)
        oracle.bwd_bias(dy)
        t_total += time.perf_counter() - t0
        done += 1
    return {"value": per_image_flop * done / t_total / 1e12, "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "first %d of %d images of the %s batch, all four ops, fp64 direct loops "
                      "(%.1f s)" % (done, N, wl_name, t_total)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense3x3")
    ap.add_argument("--all-workloads", action="store_true",
                    help="also time every workload and print one line each to stderr")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--launch", choices=("eager", "graph"), default="eager",
                    help="how the timed steps are issued: the four C-ABI calls directly "
                         "(default), or replays of one HIP graph holding the four launches")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy 5 times (for scaling the HBM "
                         "byte counters of a profiler run) and exit")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        n = 64 * 1024 * 1024                      # 64 Mi floats = 256 MiB read + 256 MiB written
        src = torch.ones(n, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written":
                          4 * n, "launches": 5}), flush=True)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    from grouped_convolution_amd.workloads import WORKLOAD_ORDER, WORKLOADS
    wl = WORKLOADS[args.workload]
    log("workload %s: x %s w %s groups %d" % (wl.name, wl.x_shape, wl.w_shape, wl.groups))
    res = run_gpu(args, args.workload)
    log("gpu done: %.4f ms/step, %.3f TFLOP/s" % (res["ms_per_step"], res["value"]))

    if args.all_workloads:
        for name in WORKLOAD_ORDER:
            if name == args.workload:
                r = res
            else:
                r = run_gpu(args, name)
            log(json.dumps({"workload": name, "tflops": round(r["value"], 3),
                            "ms_per_step": round(r["ms_per_step"], 4), "launch": r["launch"],
                            "ops": r["ops"]}))

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle (bounded sample)...")
        cpu = cpu_baseline(args.workload, budget_s=args.cpu_budget)
        log("cpu baseline: %s" % cpu)

    N, C, H, W = wl.x_shape
    K, Cg, kh, kwid = wl.w_shape
    line = {
        "metric": "grouped conv fwd+bwd fp32 TFLOP/s (NCHW) and % of MFMA/HBM roofline",
        "value": round(res["value"], 4),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "x": list(wl.x_shape), "w": list(wl.w_shape),
                   "groups": wl.groups, "stride": wl.stride, "padding": wl.padding,
                   "dilation": wl.dilation, "bias": wl.b_dist is not None,
                   "ops": list(OPS), "flop_per_step": 3 * res["flop_conv"],
                   "launch": res["launch"]},
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "ops": res["ops"],
        "device": res["device"],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
