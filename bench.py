#!/usr/bin/env python3
"""Benchmark of the stream-K engine on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic
input resident in HBM: a single skg_run_gemm / skg_run_wgrad call (argument
checks, plan, resets, the stream-K kernel with its fix-up, and the second
stage when the reduction has one).  Default workload: the bf16 GEMM
4864 x 4096 x 4096 with 256x256x64 tiles (256 data-parallel tiles, 48 spread
stream-K over a 256-CTA pool, tree fix-up).

Prints one JSON line: TFLOP/s of the whole step, the roofline of the
stream-K kernel (timed alone with HIP events on the stream it runs on), and
the CPU oracle timed on a bounded sample of the same workload.
"""

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Dense MFMA peaks of MI355X (TFLOP/s) and its HBM3E bandwidth (GB/s).
MFMA_PEAK = {"f16": 2516.6, "bf16": 2516.6, "e4m3": 5033.2, "e5m2": 5033.2}
HBM_PEAK_GBS = 8000.0
METRIC = "TFLOP/s and % of MFMA peak, stream-K GEMM and conv wgrad on 1 MI355X"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--mode", default=None)
    ap.add_argument("--reduction", default=None)
    ap.add_argument("--ctas", type=int, default=None)
    ap.add_argument("--tile", default=None)
    ap.add_argument("--sk-order", default="auto", choices=["auto", "block", "xcd"],
                    help="stream-K CTA order (auto: xcd for wgrad, block for GEMM)")
    ap.add_argument("--dtype", default=None, choices=["e4m3", "e5m2"],
                    help="fp8 operand format of the fp8 GEMM workload (default e4m3)")
    ap.add_argument("--scale-mode", default=None, choices=["rowcol", "tensor"],
                    help="scales of the fp8 GEMM workload (default rowcol)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle sample (0 disables it)")
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


def kernel_source_hash():
    """Hash of the HIP sources, so that counters taken on other code are not used."""
    import hashlib
    d = os.path.join(ROOT, "implicit_gemm_conv_dp_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp", ".cpp", ".h")):
            h.update(f.encode())
            with open(os.path.join(d, f), "rb") as fh:
                h.update(fh.read())
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
    if wl.op == "gemm":
        eab = 1 if wl.dtype_ab in ("e4m3", "e5m2") else 2
        ec = 4 if wl.dtype_c == "f32" else 2
        extra = (4 * (wl.M + wl.N) if wl.scale_mode == "rowcol" else 8) if wl.scales else 0
        return eab * (wl.M * wl.K + wl.N * wl.K) + ec * wl.M * wl.N + extra
    ho, wo = wl.out_hw
    return 2 * (wl.n * wl.h * wl.w * wl.c + wl.n * ho * wo * wl.k) + \
        4 * wl.k * wl.r * wl.s * (wl.c // wl.groups)


def cpu_baseline(wl, inp, target_s):
    """The oracle as it stands, timed on a bounded sample of the workload."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle.gemm import gemm as oracle_gemm
    from oracle.wgrad import wgrad as oracle_wgrad

    def run(frac_units):
        t0 = time.perf_counter()
        if wl.op == "gemm":
            rows = frac_units
            oracle_gemm(wl.dtype_ab, inp["A"][:rows * wl.K], inp["B"], rows, wl.N, wl.K,
                        scale_a=None if "scale_a" not in inp else
                        (inp["scale_a"][:rows] if wl.scale_mode == "rowcol" else inp["scale_a"]),
                        scale_b=inp.get("scale_b"), scale_mode=wl.scale_mode)
            flops = 2.0 * rows * wl.N * wl.K
        else:
            imgs = frac_units
            ho, wo = wl.out_hw
            oracle_wgrad(wl.dtype, inp["x"][:imgs * wl.h * wl.w * wl.c],
                         inp["dy"][:imgs * ho * wo * wl.k], imgs, wl.h, wl.w, wl.c, wl.k, wl.r,
                         wl.s, wl.stride[0], wl.stride[1], wl.pad[0], wl.pad[1], wl.groups)
            flops = wl.flops() * imgs / wl.n
        return time.perf_counter() - t0, flops

    # One small warm-up run, then grow the sample (at most 8x per step, by
    # the measured rate) until it takes the target time or covers the whole
    # workload.
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
    threads = max((d.get("num_threads", 1) for d in threadpool_info()), default=1)
    what = ("rows [0, %d) of the %d-row output" % (units, full)) if wl.op == "gemm" else \
        ("images [0, %d) of %d" % (units, full))
    if reps > 1:
        what += ", %d runs" % reps
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": "%s, fp64 oracle (numpy float64 matmul), %.1f s" % (what, t),
            "seconds": t}


def names(enum):
    return {v: k for k, v in enum.items()}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the engine has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return

    import numpy as np
    import torch

    import implicit_gemm_conv_dp_amd as skg
    from implicit_gemm_conv_dp_amd import synth

    wl = synth.WORKLOADS[args.workload]
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
    inp = wl.inputs()

    def up(codes):
        a = np.ascontiguousarray(codes)
        a = a.view(np.uint8) if a.dtype.itemsize == 1 else a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    if wl.op == "gemm":
        dA, dB = up(inp["A"]), up(inp["B"])
        sa = torch.from_numpy(inp["scale_a"]).to(dev) if wl.scales else None
        sb = torch.from_numpy(inp["scale_b"]).to(dev) if wl.scales else None
        out = torch.empty(wl.M * wl.N, dtype=torch.float32 if wl.dtype_c == "f32" else torch.int16,
                          device=dev)
        kw = dict(M=wl.M, N=wl.N, K=wl.K, dtype_ab=wl.dtype_ab, dtype_c=wl.dtype_c, tile=tile,
                  mode=mode, reduction=red, ctas=ctas, scale_mode=wl.scale_mode,
                  sk_order=args.sk_order)
        plan = skg.plan_gemm(**kw)
        ws = skg.workspace_for(plan, dev)

        def step():
            skg.gemm(dA, dB, out, sa, sb, workspace=ws, **kw)
        dtype = wl.dtype_ab
    else:
        dx, ddy = up(inp["x"]), up(inp["dy"])
        out = torch.empty(wl.k * wl.r * wl.s * (wl.c // wl.groups), dtype=torch.float32, device=dev)
        kw = dict(n=wl.n, h=wl.h, w=wl.w, c=wl.c, k=wl.k, r=wl.r, s=wl.s, stride=wl.stride,
                  pad=wl.pad, groups=wl.groups, dtype=wl.dtype, tile=tile, mode=mode,
                  reduction=red, ctas=ctas, sk_order=args.sk_order)
        plan = skg.plan_wgrad(**kw)
        ws = skg.workspace_for(plan, dev)

        def step():
            skg.wgrad(dx, ddy, out, workspace=ws, **kw)
        dtype = wl.dtype

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step()
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
        step()
    skg.skg_profile_events(None, None)
    t_stop.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_stop)
    ms_per_step = total_ms / args.steps
    kernel_ms = sum(a.elapsed_time(b) for a, b in pairs) / args.steps

    flops = wl.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    peak = MFMA_PEAK[dtype]
    hbm_bound = args.workload == 4
    traffic = measured_traffic(args.traffic, wl.name, tile, mode, red, ctas)
    if hbm_bound:
        achieved = alg_bytes(wl) / (kernel_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic}
    else:
        achieved = flops / (kernel_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": traffic}
    roof["kernel_ms"] = kernel_ms
    roof["alg_flop"] = flops
    roof["alg_bytes"] = alg_bytes(wl)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(wl, inp, args.cpu_seconds)

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
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
