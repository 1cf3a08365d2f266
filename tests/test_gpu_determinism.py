"""Deterministic fix-ups: linear and tree results are bit-identical across 20
launches when the whole workspace (flags and partials) and the output are
poisoned (all bytes 0xFF, a NaN in every float format) before each launch,
so a partial read before its release would show up as a NaN or a different
value (rocm-libraries PR #13151, GPU test plan and the review finding that
only the flags had been reset between launches).  Workloads: the fp16 GEMM
over a 6-CTA pool whose ranges straddle tiles, the bf16 GEMM with 48
stream-K tiles over 256 CTAs, both conv wgrad workloads (the grouped one
on the block-diagonal and on the per-group tile), each in the dp_sk and
persistent modes; the reduce-scatter launches; and forward / dgrad
convolutions with shared stream-K tiles.  That no bounded flag wait gave up during these
launches is checked for every GPU test by the fixture in conftest.py (the
library counts give-ups; skg_fixup_timeouts).
"""

import numpy as np
import pytest
import torch

import implicit_gemm_conv_dp_amd as skg
from implicit_gemm_conv_dp_amd import synth

from helpers import to_dev

pytestmark = pytest.mark.gpu

REPEATS = 20


def repeat(launch, out, ws):
    first = None
    for i in range(REPEATS):
        ws.fill_(0xFF)
        out.view(torch.uint8).fill_(0xFF)
        launch()
        torch.cuda.synchronize()
        got = out.clone()
        assert not torch.isnan(got.float()).any(), "launch %d left unwritten outputs" % i
        if first is None:
            first = got
        else:
            assert torch.equal(got.view(torch.uint8), first.view(torch.uint8)), "launch %d differs" % i


@pytest.mark.parametrize("reduction", ["linear", "tree"])
@pytest.mark.parametrize("mode", ["dp_sk", "persistent"])
def test_gemm_bf16_large_repeat(mode, reduction):
    wl = synth.WORKLOADS[2]
    inp = wl.inputs()
    dA, dB = to_dev(inp["A"], "bf16"), to_dev(inp["B"], "bf16")
    C = torch.empty(wl.M * wl.N, dtype=torch.bfloat16, device="cuda")
    kw = dict(M=wl.M, N=wl.N, K=wl.K, dtype_ab="bf16", dtype_c="bf16", tile=wl.tile, mode=mode,
              reduction=reduction, ctas=wl.ctas)
    plan = skg.plan_gemm(**kw)
    assert plan["sk_ctas"] == 256 and plan["max_contrib"] == 6
    ws = skg.workspace_for(plan, "cuda")
    repeat(lambda: skg.gemm(dA, dB, C, workspace=ws, **kw), C, ws)


@pytest.mark.parametrize("reduction", ["linear", "tree"])
@pytest.mark.parametrize("mode", ["dp_sk", "persistent"])
def test_gemm_f16_pool6_repeat(mode, reduction):
    wl = synth.WORKLOADS[1]
    inp = wl.inputs()
    dA, dB = to_dev(inp["A"], "f16"), to_dev(inp["B"], "f16")
    C = torch.empty(wl.M * wl.N, dtype=torch.float16, device="cuda")
    kw = dict(M=wl.M, N=wl.N, K=wl.K, dtype_ab="f16", dtype_c="f16", tile=wl.tile, mode=mode,
              reduction=reduction, ctas=wl.ctas)
    plan = skg.plan_gemm(**kw)
    # 4 tiles x 128 iterations over 6 CTAs: ranges of 85-86 iterations that
    # straddle tiles; a tile has up to 3 contributors.
    assert (plan["sk_ctas"], plan["iters_per_sk_cta"], plan["extra_iters"],
            plan["max_contrib"]) == (6, 85, 2, 3)
    ws = skg.workspace_for(plan, "cuda")
    repeat(lambda: skg.gemm(dA, dB, C, workspace=ws, **kw), C, ws)


@pytest.mark.parametrize("reduction", ["linear", "tree"])
@pytest.mark.parametrize("mode", ["dp_sk", "persistent"])
@pytest.mark.parametrize("index", [3, 4])
def test_wgrad_repeat(index, mode, reduction):
    wl = synth.WORKLOADS[index]
    inp = wl.inputs()
    dx, ddy = to_dev(inp["x"], wl.dtype), to_dev(inp["dy"], wl.dtype)
    dw = torch.empty(wl.k * wl.r * wl.s * (wl.c // wl.groups), dtype=torch.float32, device="cuda")
    kw = dict(n=wl.n, h=wl.h, w=wl.w, c=wl.c, k=wl.k, r=wl.r, s=wl.s, stride=wl.stride,
              pad=wl.pad, groups=wl.groups, dtype=wl.dtype, tile=wl.tile, mode=mode,
              reduction=reduction, ctas=wl.ctas)
    plan = skg.plan_wgrad(**kw)
    assert plan["sk_ctas"] > 0 and plan["max_contrib"] >= 2
    ws = skg.workspace_for(plan, "cuda")
    repeat(lambda: skg.wgrad(dx, ddy, dw, workspace=ws, **kw), dw, ws)


@pytest.mark.parametrize("reduction", ["linear", "tree"])
@pytest.mark.parametrize("mode", ["dp_sk", "persistent"])
def test_wgrad_per_group_tile_repeat(mode, reduction):
    # The grouped layer on the per-group 32x64x64 tile (one partial 32-row M
    # tile per group): 96 tiles of 196 iterations over 512 CTAs.
    wl = synth.WORKLOADS[4]
    inp = wl.inputs()
    dx, ddy = to_dev(inp["x"], wl.dtype), to_dev(inp["dy"], wl.dtype)
    dw = torch.empty(wl.k * wl.r * wl.s * (wl.c // wl.groups), dtype=torch.float32, device="cuda")
    kw = dict(n=wl.n, h=wl.h, w=wl.w, c=wl.c, k=wl.k, r=wl.r, s=wl.s, stride=wl.stride,
              pad=wl.pad, groups=wl.groups, dtype=wl.dtype, tile="32x64x64", mode=mode,
              reduction=reduction, ctas=512)
    plan = skg.plan_wgrad(**kw)
    assert plan["sk_ctas"] == 512 and plan["max_contrib"] >= 2
    ws = skg.workspace_for(plan, "cuda")
    repeat(lambda: skg.wgrad(dx, ddy, dw, workspace=ws, **kw), dw, ws)


@pytest.mark.parametrize("index,tile", [(3, "256x128x64"), (3, "256x256x64"), (4, "32x64x64")])
def test_wgrad_scatter_repeat(index, tile):
    # Split-K over the default pool with the reduce-scatter fix-up, k-major
    # order: every launch bit-identical on random data.
    wl = synth.WORKLOADS[index]
    inp = wl.inputs()
    dx, ddy = to_dev(inp["x"], wl.dtype), to_dev(inp["dy"], wl.dtype)
    dw = torch.empty(wl.k * wl.r * wl.s * (wl.c // wl.groups), dtype=torch.float32, device="cuda")
    kw = dict(n=wl.n, h=wl.h, w=wl.w, c=wl.c, k=wl.k, r=wl.r, s=wl.s, stride=wl.stride,
              pad=wl.pad, groups=wl.groups, dtype=wl.dtype, tile=tile, mode="splitk",
              reduction="scatter", ctas=-1, sk_order="kmajor")
    plan = skg.plan_wgrad(**kw)
    assert plan["slices"] > 1 and plan["sk_ctas"] == plan["tiles"] * plan["slices"]
    ws = skg.workspace_for(plan, "cuda")
    repeat(lambda: skg.wgrad(dx, ddy, dw, workspace=ws, **kw), dw, ws)


def test_wgrad_block_diagonal_scatter_repeat():
    # The grouped layer's benchmark launch: block-diagonal tile, dp_sk over
    # 224 CTAs = 28 whole slices per tile, reduce-scatter fix-up.
    wl = synth.WORKLOADS[4]
    inp = wl.inputs()
    dx, ddy = to_dev(inp["x"], wl.dtype), to_dev(inp["dy"], wl.dtype)
    dw = torch.empty(wl.k * wl.r * wl.s * (wl.c // wl.groups), dtype=torch.float32, device="cuda")
    kw = dict(n=wl.n, h=wl.h, w=wl.w, c=wl.c, k=wl.k, r=wl.r, s=wl.s, stride=wl.stride,
              pad=wl.pad, groups=wl.groups, dtype=wl.dtype, tile="64x144x32", mode="dp_sk",
              reduction="scatter", ctas=224)
    plan = skg.plan_wgrad(**kw)
    assert plan["sk_ctas"] == 224 and plan["max_contrib"] == 28
    ws = skg.workspace_for(plan, "cuda")
    repeat(lambda: skg.wgrad(dx, ddy, dw, workspace=ws, **kw), dw, ws)


# Convolutions with stream-K tiles shared by several CTAs: the dense layer's
# forward / dgrad on 256x256x64 tiles (the benchmark's launch), and grouped
# shapes on the block-diagonal tile (dgrad by stride phase).
CONV_REPEATS = [
    ("fwd", (32, 56, 56, 256, 256, 3, 3, (1, 1), (1, 1), 1), "f16", "256x256x64", 256),
    ("dgrad", (32, 56, 56, 256, 256, 3, 3, (1, 1), (1, 1), 1), "f16", "256x256x64", 256),
    ("fwd", (64, 28, 28, 512, 512, 3, 3, (2, 2), (1, 1), 32), "bf16", "128x64x32", 512),
    ("dgrad", (4, 14, 14, 64, 64, 3, 3, (2, 2), (1, 1), 4), "bf16", "128x64x32", 5),
]


@pytest.mark.parametrize("reduction", ["linear", "tree"])
@pytest.mark.parametrize("mode", ["dp_sk", "persistent"])
@pytest.mark.parametrize("case", range(len(CONV_REPEATS)))
def test_conv_repeat(case, mode, reduction):
    op, shape, fmt, tile, ctas = CONV_REPEATS[case]
    n, h, w, c, k, r, s, st, pd, g = shape
    ho = (h + 2 * pd[0] - r) // st[0] + 1
    wo = (w + 2 * pd[1] - s) // st[1] + 1
    na = n * h * w * c if op == "fwd" else n * ho * wo * k
    act = to_dev(synth.to_codes(synth.draw("uniform", na, 301), fmt), fmt)
    filt = to_dev(synth.to_codes(synth.draw("uniform", k * r * s * (c // g), 302), fmt), fmt)
    out = torch.empty(n * ho * wo * k if op == "fwd" else n * h * w * c, dtype=torch.bfloat16,
                      device="cuda")
    kw = dict(n=n, h=h, w=w, c=c, k=k, r=r, s=s, stride=st, pad=pd, groups=g, dtype=fmt,
              dtype_out="bf16", tile=tile, mode=mode, reduction=reduction, ctas=ctas)
    plan = (skg.plan_fwd if op == "fwd" else skg.plan_dgrad)(**kw)
    assert plan["sk_ctas"] > 0 and plan["max_contrib"] >= 2, plan
    ws = skg.workspace_for(plan, "cuda")
    call = skg.fwd if op == "fwd" else skg.dgrad
    repeat(lambda: call(act, filt, out, workspace=ws, **kw), out, ws)
