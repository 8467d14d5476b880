#!/usr/bin/env python3
"""Benchmark: grouped conv fwd+bwd fp32 TFLOP/s (NCHW) and % of MFMA/HBM roofline.

One step = the whole path on one batch of synthetic input already resident in
HBM: forward (+bias), gradInput, gradWeight and gradBias, each one call
through the C-ABI library on torch's current HIP stream.
  value  = 3 * FLOP_conv / (median cold step time)                  [TFLOP/s]
  FLOP_conv = 2*N*K*Ho*Wo*(C/G)*kh*kw (the standard count, padded taps included)

The headline workload is the largest of the five configurations, the
kernel == input ("fully-connected mode") problem of "SpatialConvolution running
in fully-connected mode is very slow, even with R4": 1600 images of 256x6x6
into 4096 planes with a 6x6 kernel. The same JSON line carries a `per_config`
block with every op of all five configurations (tiny grouped, dense 3x3,
AlexNet conv2, ResNeXt 32x4d, fully-connected mode).

Timing is cold by default: before every timed step, and before every timed op
in the per-op region, a 1 GiB buffer is read on the same stream, which evicts
the 256 MB last-level cache (MALL), so each op reads its inputs from HBM.
Each step (or op) is bracketed by HIP events on the stream the kernels run
on, and the line gives the median, min and p90 over the timed steps; `ms_per_step` is the cold median. The warm figure (the K steps back to
back, no eviction) is reported beside it. A plain device copy of 256 MiB,
timed cold in the same run, gives the achievable HBM rate that HBM-bound
fractions are also quoted against.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload fc_mode]
                    [--extra-workloads] [--no-cpu-baseline] [--launch eager|graph]

The CPU baseline times the fp64 oracle on a bounded sample (the first images of
the headline batch) on this host's cores.
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
# The five configurations of the metric, smallest first.
CONFIGS = ("tiny_grouped", "dense3x3", "alexnet_conv2", "resnext_32x4d", "fc_mode")
HEADLINE = "fc_mode"
EVICT_BYTES = 1 << 30         # read between timed steps / ops
COPY_BYTES = 256 << 20        # plain copy for the achievable HBM rate


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


def summary(ms):
    """median / min / p90 / mean of a list of times in ms."""
    a = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 5), "min": round(float(a.min()), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "mean": round(float(a.mean()), 5),
            "n": int(a.size)}


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


class Evictor:
    """Reads a 1 GiB buffer on the current stream (a sum over it), so that
    whatever an op reads next comes from HBM, not the MALL. Reading rather than
    writing leaves the cache holding clean lines, so the timed op pays no
    write-back of someone else's data."""

    def __init__(self, torch, dev, nbytes=EVICT_BYTES):
        self.buf = torch.ones(nbytes // 4, device=dev)
        self.out = torch.empty((), device=dev)

    def __call__(self):
        import torch
        torch.sum(self.buf, dim=0, out=self.out)


def copy_rate(torch, dev, evict, reps=7):
    """Achievable HBM rate: a plain 256 MiB device-to-device copy (read + write),
    each repetition cold, timed with events; returns (GB/s of the median, ms list)."""
    src = torch.ones(COPY_BYTES // 4, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ms = []
    for _ in range(reps):
        evict()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    del src, dst
    return 2.0 * COPY_BYTES / (float(np.median(ms)) * 1e-3) / 1e9, ms


def setup(wl_name, dev):
    """Device tensors, plans and chosen paths of one workload."""
    import torch
    import grouped_convolution_amd as G
    from grouped_convolution_amd.workloads import WORKLOADS, make_inputs

    wl = WORKLOADS[wl_name]
    inp = make_inputs(wl_name)
    # make_inputs gives NCHW arrays; channels-last workloads store them transposed.
    store = (lambda a: np.ascontiguousarray(a.transpose(0, 2, 3, 1))) if wl.layout == "nhwc" else (lambda a: a)
    x = torch.from_numpy(store(inp["x"])).to(dev)
    w = torch.from_numpy(inp["w"]).to(dev)
    b = None if inp["b"] is None else torch.from_numpy(inp["b"]).to(dev)
    dy = torch.from_numpy(store(inp["dy"])).to(dev)
    del inp
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
    t = dict(x=x, w=w, b=b, dy=dy, y=y, dx=dx, dw=dw, db=db)

    def make_plans():
        return {"fwd": G.Plan.fwd(x, w, b, y, **kw),
                "bwd_data": G.Plan.bwd_data(dy, w, dx, **kw),
                "bwd_filter": G.Plan.bwd_filter(x, dy, dw, **kw),
                "bwd_bias": G.Plan.bwd_bias(dy, db, layout=wl.layout)}

    paths = {op: G.PATH_NAMES[G.gconv_select_path(desc, i)] for i, op in enumerate(OPS)}
    return wl, t, make_plans, paths, Ho, Wo


def run_gpu(args, wl_name, evict, copy_gbs, headline=False):
    """Time one workload: cold steps (-> value), warm steps, cold per-op times."""
    import torch

    dev = torch.device("cuda:0")
    wl, t, make_plans, paths, Ho, Wo = setup(wl_name, dev)
    plans = make_plans()
    Ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    for _ in range(args.warmup):
        for op in OPS:
            plans[op]()
    torch.cuda.synchronize()
    K_steps = args.steps

    # Optional: one HIP graph holding a step's four launches, replayed per step.
    launch, graph = args.launch, None
    if launch == "graph" and headline:
        try:
            cs = torch.cuda.Stream()
            cs.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cs):
                gplans = make_plans()
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph, stream=cs):
                    for op in OPS:
                        gplans[op]()
            torch.cuda.current_stream().wait_stream(cs)
            for _ in range(args.warmup):
                graph.replay()
        except Exception as e:  # launch mode only: the same kernels run eagerly
            log("HIP graph capture failed (%s); timing eager launches" % e)
            graph, launch = None, "eager"
    else:
        launch = "eager"

    def step():
        if graph is not None:
            graph.replay()
        else:
            for op in OPS:
                plans[op]()

    # Timed region 1 -> value: K cold steps. Each step (its four ops, back to
    # back) is bracketed by events; the eviction runs before the start event.
    sev = [(Ev(), Ev()) for _ in range(K_steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K_steps):
        evict()
        sev[s][0].record()
        step()
        sev[s][1].record()
    torch.cuda.synchronize()
    wall_cold = time.perf_counter() - t0
    cold_steps = [a.elapsed_time(b) for a, b in sev]

    # Timed region 2: K warm steps back to back (no eviction), one event pair.
    e0, e1 = Ev(), Ev()
    torch.cuda.synchronize()
    e0.record()
    for s in range(K_steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    warm_ms = e0.elapsed_time(e1) / K_steps

    # Timed region 3 -> per-op times and the roofline object: K more steps with
    # the eviction before every op and events around every launch.
    oev = {op: [(Ev(), Ev()) for _ in range(K_steps)] for op in OPS}
    torch.cuda.synchronize()
    for s in range(K_steps):
        for op in OPS:
            evict()
            a, b = oev[op][s]
            a.record()
            plans[op]()
            b.record()
    torch.cuda.synchronize()
    per_op = {op: [a.elapsed_time(b) for a, b in oev[op]] for op in OPS}

    flop = conv_flop(wl, Ho, Wo)
    nbytes = op_bytes(wl, Ho, Wo, t["b"] is not None)
    ops = {}
    for op in OPS:
        st = summary(per_op[op])
        tm = st["median"] * 1e-3
        f = 0.0 if op == "bwd_bias" else flop
        ai = f / nbytes[op]
        # Below the ridge the op is bound by HBM whatever unit computes it;
        # above it, by the matrix cores (MFMA families) or the vector ALUs.
        if ai < RIDGE:
            bound = "hbm"
        else:
            bound = "alu" if paths[op] == "direct" else "mfma"
        peak = {"hbm": PEAK_HBM, "alu": PEAK_VALU_F32, "mfma": PEAK_MFMA_F32}[bound]
        achieved = nbytes[op] / tm if bound == "hbm" else f / tm
        rec = {"ms": st["median"], "ms_min": st["min"], "ms_p90": st["p90"], "ms_mean": st["mean"],
               "path": paths[op], "tflops": round(f / tm / 1e12, 3),
               "gbs": round(nbytes[op] / tm / 1e9, 1), "bound": bound, "frac": round(achieved / peak, 4)}
        if bound == "hbm":
            rec["frac_of_copy"] = round(nbytes[op] / tm / 1e9 / copy_gbs, 4)
        ops[op] = rec
    cold = summary(cold_steps)
    res = {
        "workload": wl.name, "ms_per_step": cold["median"],
        "tflops": round(3.0 * flop / (cold["median"] * 1e-3) / 1e12, 3),
        "step_cold_ms": cold, "step_warm_ms": round(warm_ms, 5),
        "tflops_warm": round(3.0 * flop / (warm_ms * 1e-3) / 1e12, 3),
        "ops": ops, "flop_conv": flop, "launch": launch, "wall_cold_s": wall_cold,
        "Ho": Ho, "Wo": Wo, "has_bias": t["b"] is not None,
    }
    if headline:
        # The dominant kernel: the op with the largest mean cold time; achieved
        # = algorithmic FLOP (or bytes) per launch / its mean event time, the
        # figure rocprofv3's average kernel duration is compared with.
        dom = max(OPS, key=lambda o: ops[o]["ms_mean"])
        d = ops[dom]
        t_dom = d["ms_mean"] * 1e-3
        if d["bound"] == "hbm":
            roof = {"bound": "hbm", "achieved": round(nbytes[dom] / t_dom / 1e9, 1),
                    "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
        else:
            roof = {"bound": d["bound"], "achieved": round(flop / t_dom / 1e12, 3),
                    "peak": (PEAK_MFMA_F32 if d["bound"] == "mfma" else PEAK_VALU_F32) / 1e12,
                    "unit": "TFLOP/s"}
        roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
        roof["traffic"] = traffic_from_profiles("%s:%s:%s" % (wl.name, dom, d["path"]))
        roof["kernel"] = "%s (%s path)" % (dom, d["path"])
        roof["launch_ms"] = d["ms_mean"]
        roof["algorithmic_per_launch"] = nbytes[dom] if d["bound"] == "hbm" else flop
        res["roofline"] = roof
        import torch as _t
        res["device"] = _t.cuda.get_device_name(dev)
    del plans, t
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def cpu_baseline(wl_name, budget_s=12.0, max_images=None):
    """The fp64 oracle on the first images of the same batch, all four ops per
    image, until about `budget_s` of wall time is spent."""
    import oracle
    from grouped_convolution_amd.workloads import WORKLOADS, make_inputs

    wl = WORKLOADS[wl_name]
    N = wl.x_shape[0]
    limit = N if max_images is None else min(N, max_images)
    inp = make_inputs(wl_name, batch=min(limit, 64))
    kw = dict(stride=wl.stride, padding=wl.padding, dilation=wl.dilation, groups=wl.groups)
    K, Cg, kh, kwid = wl.w_shape
    Ho, Wo = wl.dy_shape[2], wl.dy_shape[3]
    per_image_flop = 3.0 * 2.0 * K * Ho * Wo * Cg * kh * kwid
    done, t_total = 0, 0.0
    limit = min(limit, inp["x"].shape[0])
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
    ap.add_argument("--workload", default=HEADLINE,
                    help="workload of the headline value (default: fc_mode, the largest configuration)")
    ap.add_argument("--only", action="store_true",
                    help="time the --workload alone (no per_config block)")
    ap.add_argument("--extra-workloads", action="store_true",
                    help="also time the workloads beyond the five configurations (depthwise, "
                         "pointwise, channels-last) and add them to the line as `next_rows`")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--launch", choices=("eager", "graph"), default="eager",
                    help="how the headline's timed steps are issued: the four C-ABI calls "
                         "directly (default), or replays of one HIP graph holding them")
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

    import torch
    from grouped_convolution_amd.workloads import WORKLOAD_ORDER, WORKLOADS
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    evict = Evictor(torch, dev)
    copy_gbs, copy_ms = copy_rate(torch, dev, evict)
    log("cold 256 MiB copy: %.0f GB/s (median of %d)" % (copy_gbs, len(copy_ms)))

    wl = WORKLOADS[args.workload]
    log("headline workload %s: x %s w %s groups %d" % (wl.name, wl.x_shape, wl.w_shape, wl.groups))
    res = run_gpu(args, args.workload, evict, copy_gbs, headline=True)
    log("headline done: cold median %.4f ms/step (%.3f TFLOP/s), warm %.4f ms/step"
        % (res["ms_per_step"], res["tflops"], res["step_warm_ms"]))

    per_config = {}
    if not args.only:
        for name in CONFIGS:
            r = res if name == args.workload else run_gpu(args, name, evict, copy_gbs)
            per_config[name] = {k: r[k] for k in ("ms_per_step", "tflops", "step_cold_ms",
                                                  "step_warm_ms", "tflops_warm", "ops")}
            log(json.dumps({"workload": name, **per_config[name]}))
    next_rows = {}
    if args.extra_workloads:
        for name in WORKLOAD_ORDER:
            if name in CONFIGS:
                continue
            r = run_gpu(args, name, evict, copy_gbs)
            next_rows[name] = {k: r[k] for k in ("ms_per_step", "tflops", "step_warm_ms", "ops")}
            log(json.dumps({"workload": name, **next_rows[name]}))

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle (bounded sample)...")
        cpu = cpu_baseline(args.workload, budget_s=args.cpu_budget)
        log("cpu baseline: %s" % cpu)

    N, C, H, W = wl.x_shape
    K, Cg, kh, kwid = wl.w_shape
    line = {
        "metric": "grouped conv fwd+bwd fp32 TFLOP/s (NCHW) and % of MFMA/HBM roofline",
        "value": res["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "x": list(wl.x_shape), "w": list(wl.w_shape),
                   "groups": wl.groups, "stride": wl.stride, "padding": wl.padding,
                   "dilation": wl.dilation, "bias": wl.b_dist is not None,
                   "ops": list(OPS), "flop_per_step": 3 * res["flop_conv"],
                   "launch": res["launch"], "timing": "cold (1 GiB read before each step)"},
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "timing": {"step_cold_ms": res["step_cold_ms"], "step_warm_ms": res["step_warm_ms"],
                   "value_warm": res["tflops_warm"], "copy_gbs": round(copy_gbs, 1),
                   "copy_ms": [round(v, 5) for v in copy_ms]},
        "ops": res["ops"],
        "per_config": per_config,
        "device": res["device"],
    }
    if next_rows:
        line["next_rows"] = next_rows
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
