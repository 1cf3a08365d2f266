#!/usr/bin/env python3
"""Benchmark of the stream-K engine on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic
input resident in HBM: a single skg_run_gemm / skg_run_wgrad call (argument
checks, plan, resets, the stream-K kernel with its fix-up, and the second
stage when the reduction has one).  The headline workload (default: the bf16
GEMM 4864 x 4096 x 4096 with 256x256x64 tiles, 256 data-parallel tiles and 48
spread stream-K over a 256-CTA pool, tree fix-up) is timed over exactly
--steps steps after --warmup untimed ones.

Printed as one JSON line: TFLOP/s of the headline step, the roofline of its
stream-K kernel (timed alone with HIP events on the stream it runs on), a
table of all five workloads (the kernel and the whole step per launch: median,
p10 and p90 of 100 launches after 50 warm-up ones, as the pages' parity runs
time them), the data-parallel-only launch of the same kernel on the two
wgrad workloads, a cold-cache run of the grouped wgrad, and the CPU oracle
timed on a bounded sample of the headline workload (plus single-core
samples of workloads 1 and 4).
"""

import argparse
import dataclasses
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Dense MFMA peaks of MI355X (TFLOP/s) and its HBM3E bandwidth (GB/s).
MFMA_PEAK = {"f16": 2516.6, "bf16": 2516.6, "e4m3": 5033.2, "e5m2": 5033.2}
HBM_PEAK_GBS = 8000.0
NUM_CUS = 256
METRIC = "TFLOP/s and % of MFMA peak, stream-K GEMM and conv wgrad on 1 MI355X"
# Timing protocol of the workload table (the pages' parity runs: warm-up 50,
# repeat 100).
TABLE_WARMUP, TABLE_REPEAT = 50, 100
# Scrub buffer written between the launches of a cold-cache run (larger than
# the L2s and the 256 MB MALL together).
SCRUB_BYTES = 512 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # A step of the headline workload takes ~0.16 ms: 200 untimed steps
    # (~30 ms) bring the GPU to its steady state (with 10, the kernel ran
    # 168 instead of 150 us per launch on the same box), 400 timed ones
    # take ~60 ms.
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", type=int, default=2, choices=list(range(1, 11)),
                    help="headline workload (value, roofline, cpu_baseline); 6-9 are the "
                         "forward and dgrad convolutions of the two wgrad layers, 10 the fp8 "
                         "GEMM with MX block scales")
    ap.add_argument("--no-table", action="store_true",
                    help="time the headline workload only (no table of all five)")
    ap.add_argument("--mode", default=None)
    ap.add_argument("--reduction", default=None)
    ap.add_argument("--ctas", type=int, default=None)
    ap.add_argument("--tile", default=None)
    ap.add_argument("--sk-order", default="auto", choices=["auto", "block", "xcd", "kmajor"],
                    help="stream-K CTA order (auto: kmajor for wgrad, block for GEMM)")
    ap.add_argument("--dtype", default=None, choices=["e4m3", "e5m2"],
                    help="fp8 operand format of the fp8 GEMM workload (default e4m3)")
    ap.add_argument("--scale-mode", default=None, choices=["rowcol", "tensor"],
                    help="scales of the fp8 GEMM workload (default rowcol)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle sample (0 disables the CPU legs)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "hbm_traffic.json"),
                    help="JSON file of HBM bytes per launch measured with rocprofv3 byte "
                         "counters; used only while the kernel sources still hash to the "
                         "value recorded with them")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the workload, run a plain device copy of MIB MiB "
                         "(the reference for scaling HBM byte counters)")
    return ap.parse_args()


def copy_calibration(mib, steps):
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": steps}), flush=True)


def _code_only(src):
    """C/C++ source without its comments and with whitespace runs folded, so
    that an edit to a comment does not change the hash (string literals are
    kept as they are)."""
    import re
    tok = re.compile(r'"(?:\\.|[^"\\\n])*"|//[^\n]*|/\*.*?\*/', re.S)
    out = tok.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", src)
    return re.sub(r"\s+", " ", out).strip()


def kernel_source_hash():
    """Hash of the HIP sources' code (comments and layout left out), so that
    counters taken on other code are not used."""
    import hashlib
    d = os.path.join(ROOT, "implicit_gemm_conv_dp_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp", ".cpp", ".h")):
            h.update(f.encode())
            with open(os.path.join(d, f), encoding="utf-8") as fh:
                h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(path, name, tile, mode, red, ctas):
    """HBM bytes per launch from the counter file, or None when the file is
    missing, was taken on other kernel sources or on another launch."""
    if not path or not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash():
        return None
    e = t.get("workloads", {}).get(name)
    if not e or (e["tile"], e["mode"], e["reduction"], e["ctas"]) != (tile, mode, red, ctas):
        return None
    return e["bytes_per_launch"]


def alg_bytes(wl):
    """Each input read once plus the output written once."""
    if wl.op in ("fwd", "dgrad"):
        ho, wo = wl.out_hw
        x, y = wl.n * wl.h * wl.w * wl.c, wl.n * ho * wo * wl.k
        eo = 4 if wl.dtype_out == "f32" else 2
        filt = 2 * wl.k * wl.r * wl.s * (wl.c // wl.groups)
        return (2 * x + eo * y if wl.op == "fwd" else 2 * y + eo * x) + filt
    if wl.op == "gemm":
        eab = 1 if wl.dtype_ab in ("e4m3", "e5m2") else 2
        ec = 4 if wl.dtype_c == "f32" else 2
        extra = 0
        if wl.scales:
            extra = {"rowcol": 4 * (wl.M + wl.N), "tensor": 8,
                     "mx": (wl.M + wl.N) * (wl.K // 32)}[wl.scale_mode]
        return eab * (wl.M * wl.K + wl.N * wl.K) + ec * wl.M * wl.N + extra
    ho, wo = wl.out_hw
    return 2 * (wl.n * wl.h * wl.w * wl.c + wl.n * ho * wo * wl.k) + \
        4 * wl.k * wl.r * wl.s * (wl.c // wl.groups)


def host_cpus():
    """(CPUs this process may run on, CPU model name)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def cpu_baseline(wl, inp, target_s, threads):
    """The oracle as it stands, timed on a bounded sample of the workload
    with its BLAS limited to `threads` threads."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle.gemm import gemm as oracle_gemm
    from oracle.wgrad import wgrad as oracle_wgrad

    def run(units):
        t0 = time.perf_counter()
        if wl.op == "gemm":
            rows = units
            oracle_gemm(wl.dtype_ab, inp["A"][:rows * wl.K], inp["B"], rows, wl.N, wl.K,
                        scale_a=None if "scale_a" not in inp else
                        (inp["scale_a"][:rows] if wl.scale_mode == "rowcol" else inp["scale_a"]),
                        scale_b=inp.get("scale_b"), scale_mode=wl.scale_mode)
            flops = 2.0 * rows * wl.N * wl.K
        else:
            imgs = units
            ho, wo = wl.out_hw
            oracle_wgrad(wl.dtype, inp["x"][:imgs * wl.h * wl.w * wl.c],
                         inp["dy"][:imgs * ho * wo * wl.k], imgs, wl.h, wl.w, wl.c, wl.k, wl.r,
                         wl.s, wl.stride[0], wl.stride[1], wl.pad[0], wl.pad[1], wl.groups)
            flops = wl.flops() * imgs / wl.n
        return time.perf_counter() - t0, flops

    with threadpool_limits(limits=threads):
        used = max((d.get("num_threads", 1) for d in threadpool_info()), default=1)
        # One small warm-up run, then grow the sample (at most 8x per step, by
        # the measured rate) until it takes the target time or covers the
        # whole workload.
        full = wl.M if wl.op == "gemm" else wl.n
        units = max(1, full // 64)
        run(units)
        while True:
            t, flops = run(units)
            if t >= target_s or units >= full:
                break
            grow = min(8.0, max(2.0, target_s / max(t, 1e-3)))
            units = min(full, int(units * grow))
        # The whole workload takes less than the target: repeat it.
        reps = 1
        while t < target_s and units >= full and reps < 256:
            t_more, _ = run(units)
            t += t_more
            reps += 1
    flops *= reps
    what = ("rows [0, %d) of the %d-row output" % (units, full)) if wl.op == "gemm" else \
        ("images [0, %d) of %d" % (units, full))
    if reps > 1:
        what += ", %d runs" % reps
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(used), "kind": "oracle",
            "sample": "%s of %s, fp64 oracle (numpy float64 matmul, its BLAS at %d threads), %.1f s"
                      % (what, wl.name, used, t),
            "seconds": t}


def names(enum):
    return {v: k for k, v in enum.items()}


def pct(xs, q):
    s = sorted(xs)
    if not s:
        return None
    i = min(len(s) - 1, max(0, int(round(q / 100.0 * (len(s) - 1)))))
    return s[i]


def stats_us(ms_list):
    return {"median": pct(ms_list, 50) * 1e3, "p10": pct(ms_list, 10) * 1e3,
            "p90": pct(ms_list, 90) * 1e3, "n": len(ms_list)}


class Runner:
    """Inputs of one workload resident on the device and one launch of it."""

    def __init__(self, wl, dev, tile, mode, red, ctas, sk_order, inp=None):
        import numpy as np
        import torch
        import implicit_gemm_conv_dp_amd as skg
        self.skg, self.torch, self.wl, self.dev = skg, torch, wl, dev
        self.inp = inp if inp is not None else wl.inputs()

        def up(codes):
            a = np.ascontiguousarray(codes)
            a = a.view(np.uint8) if a.dtype.itemsize == 1 else a.view(np.int16)
            return torch.from_numpy(a).to(dev)

        if wl.op in ("fwd", "dgrad"):
            ho, wo = wl.out_hw
            self.a, self.b = up(self.inp["act"]), up(self.inp["filt"])
            nout = wl.n * ho * wo * wl.k if wl.op == "fwd" else wl.n * wl.h * wl.w * wl.c
            self.out = torch.empty(nout, dtype=torch.float32 if wl.dtype_out == "f32" else torch.int16,
                                   device=dev)
            self.dtype = wl.dtype
        elif wl.op == "gemm":
            self.a, self.b = up(self.inp["A"]), up(self.inp["B"])
            self.sa = torch.from_numpy(self.inp["scale_a"]).to(dev) if wl.scales else None
            self.sb = torch.from_numpy(self.inp["scale_b"]).to(dev) if wl.scales else None
            self.out = torch.empty(wl.M * wl.N, dtype=torch.float32 if wl.dtype_c == "f32"
                                   else torch.int16, device=dev)
            self.dtype = wl.dtype_ab
        else:
            self.a, self.b = up(self.inp["x"]), up(self.inp["dy"])
            self.out = torch.empty(wl.k * wl.r * wl.s * (wl.c // wl.groups), dtype=torch.float32,
                                   device=dev)
            self.dtype = wl.dtype
        self.set_launch(tile, mode, red, ctas, sk_order)

    def set_launch(self, tile, mode, red, ctas, sk_order):
        wl, skg = self.wl, self.skg
        self.tile, self.mode, self.red, self.ctas = tile, mode, red, ctas
        if wl.op in ("fwd", "dgrad"):
            self.kw = dict(n=wl.n, h=wl.h, w=wl.w, c=wl.c, k=wl.k, r=wl.r, s=wl.s,
                           stride=wl.stride, pad=wl.pad, groups=wl.groups, dtype=wl.dtype,
                           dtype_out=wl.dtype_out, tile=tile, mode=mode, reduction=red, ctas=ctas,
                           sk_order=sk_order)
            self.plan = (skg.plan_fwd if wl.op == "fwd" else skg.plan_dgrad)(**self.kw)
        elif wl.op == "gemm":
            self.kw = dict(M=wl.M, N=wl.N, K=wl.K, dtype_ab=wl.dtype_ab, dtype_c=wl.dtype_c,
                           tile=tile, mode=mode, reduction=red, ctas=ctas,
                           scale_mode=wl.scale_mode, sk_order=sk_order)
            self.plan = skg.plan_gemm(**self.kw)
        else:
            self.kw = dict(n=wl.n, h=wl.h, w=wl.w, c=wl.c, k=wl.k, r=wl.r, s=wl.s,
                           stride=wl.stride, pad=wl.pad, groups=wl.groups, dtype=wl.dtype,
                           tile=tile, mode=mode, reduction=red, ctas=ctas, sk_order=sk_order)
            self.plan = skg.plan_wgrad(**self.kw)
        self.ws = skg.workspace_for(self.plan, self.dev)

    def step(self):
        if self.wl.op in ("fwd", "dgrad"):
            (self.skg.fwd if self.wl.op == "fwd" else self.skg.dgrad)(
                self.a, self.b, self.out, workspace=self.ws, **self.kw)
        elif self.wl.op == "gemm":
            self.skg.gemm(self.a, self.b, self.out, self.sa, self.sb, workspace=self.ws, **self.kw)
        else:
            self.skg.wgrad(self.a, self.b, self.out, workspace=self.ws, **self.kw)

    def timed(self, warmup, repeat, scrub=None):
        """Per-launch times (ms) of the stream-K kernel alone and of the
        whole step, each from its own HIP event pair on the launch stream.
        With `scrub`, the buffer is overwritten before every launch, outside
        the timed region."""
        torch, skg = self.torch, self.skg
        stream = torch.cuda.current_stream()
        for _ in range(warmup):
            self.step()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(repeat)]
        for row in ev:  # create the underlying HIP events
            for e in row:
                e.record(stream)
        torch.cuda.synchronize()
        for i, (s0, k0, k1, s1) in enumerate(ev):
            if scrub is not None:
                scrub.fill_(i & 0xFF)
            skg.skg_profile_events(k0.cuda_event, k1.cuda_event)
            s0.record(stream)
            self.step()
            s1.record(stream)
        skg.skg_profile_events(None, None)
        torch.cuda.synchronize()
        kern = [k0.elapsed_time(k1) for _, k0, k1, _ in ev]
        step = [s0.elapsed_time(s1) for s0, _, _, s1 in ev]
        return kern, step


def roofline_of(wl, kernel_ms, dtype, tile, mode, red, ctas, traffic_path, pool=None):
    """Bound, achieved rate, peak and fraction of one kernel time."""
    flops = wl.flops()
    if wl.op != "gemm" and wl.groups > 1:
        achieved = alg_bytes(wl) / (kernel_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    else:
        achieved = flops / (kernel_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_PEAK[dtype],
                "unit": "TFLOP/s", "frac": achieved / MFMA_PEAK[dtype]}
        if pool is not None and pool < NUM_CUS:
            # A pool of fewer CTAs than CUs (one CTA per CU) caps the kernel at
            # its share of the chip.
            cap = MFMA_PEAK[dtype] * pool / NUM_CUS
            roof["pool_cap"] = cap
            roof["frac_of_pool_cap"] = achieved / cap
    roof["traffic"] = measured_traffic(traffic_path, wl.name, tile, mode, red, ctas)
    roof["kernel_ms"] = kernel_ms
    roof["alg_flop"] = flops
    roof["alg_bytes"] = alg_bytes(wl)
    return roof


def table(args, dev, headline_runner):
    """The five workloads in the launch each is benchmarked in, plus the
    data-parallel-only launch of the same kernel on the wgrad workloads and a
    cold-cache run of the grouped wgrad."""
    import torch
    from implicit_gemm_conv_dp_amd import synth
    rows = []
    allw = dict(synth.WORKLOADS)
    allw.update(synth.NEXT_WORKLOADS)
    for i in sorted(allw):
        wl = allw[i]
        t0 = time.perf_counter()
        if headline_runner is not None and i == args.workload:
            r = headline_runner
            r.set_launch(wl.tile, wl.modes[0], wl.reductions[0], wl.ctas, "auto")
        else:
            r = Runner(wl, dev, wl.tile, wl.modes[0], wl.reductions[0], wl.ctas, "auto")
        kern, step = r.timed(TABLE_WARMUP, TABLE_REPEAT)
        k = stats_us(kern)
        roof = roofline_of(wl, k["median"] * 1e-3, r.dtype, r.tile, r.mode, r.red, r.ctas,
                           args.traffic, pool=r.plan["pool"] if r.plan["sk_ctas"] else None)
        row = {"index": i, "workload": wl.name, "tile": r.tile, "mode": r.mode,
               "reduction": r.red, "ctas": r.ctas, "dtype": r.dtype,
               "plan": {f: r.plan[f] for f in ("tiles", "iters_per_tile", "dp_tiles", "sk_tiles",
                                               "sk_ctas", "iters_per_sk_cta", "extra_iters",
                                               "grid", "max_contrib")},
               "kernel_us": k, "step_us": stats_us(step),
               "bound": roof["bound"], "achieved": roof["achieved"], "unit": roof["unit"],
               "peak": roof["peak"], "frac": roof["frac"]}
        if r.red == "scatter":
            # the linear fix-up's sums in its order, split over the contributors
            row["same_bits_as"] = "linear"
        for key in ("pool_cap", "frac_of_pool_cap", "traffic"):
            if key in roof:
                row[key] = roof[key]
        extra = []
        for (tile, mode, red, ctas) in synth.EXTRA_LAUNCHES.get(i, []):
            r.set_launch(tile, mode, red, ctas, "auto")
            ek, es = r.timed(TABLE_WARMUP // 5, TABLE_REPEAT // 5)
            e = stats_us(ek)
            eroof = roofline_of(wl, e["median"] * 1e-3, r.dtype, tile, mode, red, ctas,
                                args.traffic, pool=r.plan["pool"] if r.plan["sk_ctas"] else None)
            extra.append({"tile": tile, "mode": mode, "reduction": red, "ctas": ctas,
                          "kernel_us": e, "step_us": stats_us(es), "achieved": eroof["achieved"],
                          "unit": eroof["unit"], "frac": eroof["frac"]})
        if extra:
            row["extra_launches"] = extra
            r.set_launch(wl.tile, wl.modes[0], wl.reductions[0], wl.ctas, "auto")
        if wl.op != "gemm":
            # The same kernel with every tile data-parallel (grid = tiles).
            r.set_launch(wl.tile, "dp", "linear", wl.ctas, "auto")
            dk, ds = r.timed(TABLE_WARMUP // 5, TABLE_REPEAT // 5)
            row["dp_only"] = {"grid": r.plan["grid"], "kernel_us": stats_us(dk),
                              "step_us": stats_us(ds)}
            row["speedup_vs_dp_only"] = row["dp_only"]["step_us"]["median"] / \
                row["step_us"]["median"]
            if wl.op == "wgrad" and wl.groups > 1:
                # Cold caches: a 512 MB scrub buffer rewritten before every
                # launch (outside the timed region).
                r.set_launch(wl.tile, wl.modes[0], wl.reductions[0], wl.ctas, "auto")
                scrub = torch.empty(SCRUB_BYTES, dtype=torch.uint8, device=dev)
                ck, cs = r.timed(5, 30, scrub=scrub)
                del scrub
                row["cold"] = {"kernel_us": stats_us(ck), "step_us": stats_us(cs),
                               "achieved": alg_bytes(wl) / (pct(ck, 50) * 1e-3) / 1e9,
                               "unit": "GB/s"}
        row["seconds"] = time.perf_counter() - t0
        rows.append(row)
        print("# workload %d %s: kernel median %.1f us (p10 %.1f, p90 %.1f), %.4g %s, frac %.3f"
              % (i, wl.name, k["median"], k["p10"], k["p90"], roof["achieved"], roof["unit"],
                 roof["frac"]), file=sys.stderr, flush=True)
        if r is not headline_runner:
            del r
            torch.cuda.empty_cache()
    return rows


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the engine has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return

    import torch

    import implicit_gemm_conv_dp_amd as skg
    from implicit_gemm_conv_dp_amd import synth

    wl = synth.WORKLOADS.get(args.workload) or synth.NEXT_WORKLOADS[args.workload]
    if args.dtype or args.scale_mode:
        if wl.op != "gemm" or not wl.scales:
            sys.exit("--dtype / --scale-mode apply to the fp8 GEMM workload only")
        dt, sm = args.dtype or wl.dtype_ab, args.scale_mode or wl.scale_mode
        wl = dataclasses.replace(wl, dtype_ab=dt, scale_mode=sm, name="gemm_%s_%dx%dx%d_%s_scales" % (
            dt, wl.M, wl.N, wl.K, "rowcol" if sm == "rowcol" else "per_tensor"))
    mode = args.mode or wl.modes[0]
    red = args.reduction or wl.reductions[0]
    ctas = args.ctas if args.ctas is not None else wl.ctas
    tile = args.tile or wl.tile
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    run = Runner(wl, dev, tile, mode, red, ctas, args.sk_order)
    plan = run.plan
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        run.step()
    # One event pair per timed step brackets the stream-K kernel alone.
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    for a, b in pairs:   # create the underlying HIP events
        a.record(stream)
        b.record(stream)
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for a, b in pairs:
        skg.skg_profile_events(a.cuda_event, b.cuda_event)
        run.step()
    skg.skg_profile_events(None, None)
    t_stop.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_stop)
    ms_per_step = total_ms / args.steps
    kernel_times = [a.elapsed_time(b) for a, b in pairs]
    kernel_ms = sum(kernel_times) / args.steps
    dtype = run.dtype

    flops = wl.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    peak = MFMA_PEAK[dtype]
    roof = roofline_of(wl, kernel_ms, dtype, tile, mode, red, ctas, args.traffic,
                       pool=plan["pool"] if plan["sk_ctas"] else None)
    roof["kernel_us_median"] = pct(kernel_times, 50) * 1e3
    # The headline is over: hand its inputs to the CPU legs and the table.
    inp = run.inp

    cpu = None
    if args.cpu_seconds > 0:
        nproc, model = host_cpus()
        env_threads = os.environ.get("OMP_NUM_THREADS")
        threads = int(env_threads) if env_threads and env_threads.isdigit() else nproc
        cpu = cpu_baseline(wl, inp, args.cpu_seconds, threads)
        cpu.update({"nproc": nproc, "cpu_model": model, "threads_requested": threads})
        single = []
        for i in (1, 4):
            w = synth.WORKLOADS[i]
            s = cpu_baseline(w, w.inputs(), max(1.0, args.cpu_seconds / 4), 1)
            single.append({"workload": w.name, "value": s["value"], "unit": s["unit"],
                           "cores": s["cores"], "sample": s["sample"]})
        cpu["single_core"] = single

    rows = None
    if not args.no_table:
        rows = table(args, dev, run)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "pct_of_mfma_peak": 100.0 * value / peak,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "tile": tile, "mode": mode, "reduction": red,
                   "ctas": ctas, "plan": {k: plan[k] for k in (
                       "tiles", "iters_per_tile", "dp_tiles", "sk_tiles", "sk_ctas",
                       "iters_per_sk_cta", "extra_iters", "grid", "max_contrib", "tree_rounds")},
                   "resolved": {"mode": names(skg.MODES)[plan["mode"]],
                                "reduction": names(skg.REDUCTIONS)[plan["reduction"]],
                                "ctas": plan["pool"], "slices": plan["slices"],
                                "sk_order": names(skg.SK_ORDERS)[plan["sk_order"]]}},
        "roofline": roof,
        "cpu_baseline": cpu,
        "workloads": rows,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
