"""The allocation-free wgrad entry point (skg_run_wgrad_static, for callers
that cannot allocate) against the existing one (skg_run_wgrad), through the
C ABI: two calls in a row, the second on a smaller problem, for every
reduction; bit-identical results on integer-exact data (every product and
fp32 partial sum exact, so even the atomic orders agree) and equal to the
oracle; linear/tree bit-identical on random data too; a plan larger than the
static scratch is rejected with -2 and leaves the output untouched."""

import numpy as np
import pytest
import torch

import implicit_gemm_conv_dp_amd as skg
from implicit_gemm_conv_dp_amd import synth, _lib
from oracle.wgrad import out_size, wgrad as oracle_wgrad

from helpers import out_buffer, to_dev

pytestmark = pytest.mark.gpu

# N, H, W, C, K, R, S, stride, pad, groups
BIG = (4, 28, 28, 128, 128, 3, 3, (1, 1), (1, 1), 1)
SMALL = (2, 12, 12, 64, 32, 3, 3, (2, 2), (1, 1), 4)


def inputs(shape, integer, seed):
    n, h, w, c, k, r, s, st, pd, g = shape
    ho, wo = out_size(h, w, r, s, st[0], st[1], pd[0], pd[1])
    if integer:
        x = synth.integer_codes("bf16", n * h * w * c, seed, 0.5)
        dy = synth.integer_codes("bf16", n * ho * wo * k, seed + 1, 0.5)
    else:
        x = synth.to_codes(synth.draw("uniform", n * h * w * c, seed), "bf16")
        dy = synth.to_codes(synth.draw("uniform", n * ho * wo * k, seed + 1), "bf16")
    R = oracle_wgrad("bf16", x, dy, n, h, w, c, k, r, s, st[0], st[1], pd[0], pd[1], g)
    return to_dev(x, "bf16"), to_dev(dy, "bf16"), R.reshape(-1)


def both(shape, dx, ddy, tile, mode, red, ctas):
    """(static result, existing result) as float64 arrays, poisoned outputs."""
    n, h, w, c, k, r, s, st, pd, g = shape
    outs = []
    for static in (True, False):
        dw = out_buffer("f32", k * r * s * (c // g))
        kw = dict(n=n, h=h, w=w, c=c, k=k, r=r, s=s, stride=st, pad=pd, groups=g, dtype="bf16",
                  tile=tile, mode=mode, reduction=red, ctas=ctas)
        args = skg.wgrad_args(dx, ddy, dw.view(torch.float32), **kw)
        stream = torch.cuda.current_stream().cuda_stream
        if static:
            skg.skg_run_wgrad_static(args, stream)
        else:
            plan = skg.plan_wgrad(**kw)
            ws = skg.workspace_for(plan, "cuda")
            skg.skg_run_wgrad(args, ws.data_ptr(), ws.numel(), stream)
        torch.cuda.synchronize()
        outs.append(dw.view(torch.float32).cpu().numpy().astype(np.float64))
    return outs


@pytest.mark.parametrize("red", ["linear", "tree", "workspace", "atomic"])
def test_static_equals_existing_two_calls(red):
    big, small = inputs(BIG, True, 61), inputs(SMALL, True, 63)
    for shape, (dx, ddy, R), tile, ctas in ((BIG, big, "256x128x64", 48),
                                            (SMALL, small, "32x64x64", 7)):
        plan = skg.plan_wgrad(n=shape[0], h=shape[1], w=shape[2], c=shape[3], k=shape[4],
                              r=shape[5], s=shape[6], stride=shape[7], pad=shape[8],
                              groups=shape[9], dtype="bf16", tile=tile, mode="dp_sk",
                              reduction=red, ctas=ctas)
        assert plan["sk_ctas"] == ctas and plan["max_contrib"] >= 2, plan
        Ys, Ye = both(shape, dx, ddy, tile, "dp_sk", red, ctas)
        assert np.array_equal(Ys, Ye), "%s %s: static differs from the existing entry point" % (red, tile)
        assert np.array_equal(Ys, R), "%s %s: not the oracle" % (red, tile)


@pytest.mark.parametrize("mode", ["dp_sk", "persistent"])
def test_static_random_data_bit_identical_linear_tree(mode):
    dx, ddy, R = inputs(BIG, False, 71)
    for red in ("linear", "tree"):
        Ys, Ye = both(BIG, dx, ddy, "256x128x64", mode, red, 48)
        assert np.array_equal(Ys, Ye), "%s %s" % (mode, red)
        assert np.max(np.abs(Ys - R)) / np.max(np.abs(R)) <= 5e-3


def test_static_rejects_plans_beyond_its_scratch():
    # N=32 56x56 C=K=256 3x3 with 256x256x64 tiles and a linear pool of 256:
    # 256 partial tiles of 256 KiB = 64 MiB > the static scratch.
    shape = (32, 56, 56, 256, 256, 3, 3, (1, 1), (1, 1), 1)
    kw = dict(n=32, h=56, w=56, c=256, k=256, r=3, s=3, stride=(1, 1), pad=(1, 1), groups=1,
              dtype="f16", tile="256x256x64", mode="dp_sk", reduction="linear", ctas=256)
    plan = skg.plan_wgrad(**kw)
    assert plan["workspace_bytes"] > _lib.STATIC_SCRATCH_BYTES
    dx = torch.zeros(32 * 56 * 56 * 256, dtype=torch.int16, device="cuda")
    dw = out_buffer("f32", 256 * 9 * 256)
    before = dw.clone()
    with pytest.raises(skg.SkgError) as ei:
        skg.skg_run_wgrad_static(skg.wgrad_args(dx, dx, dw.view(torch.float32), **kw),
                                 torch.cuda.current_stream().cuda_stream)
    assert ei.value.status == -2 and "static scratch" in ei.value.msg
    torch.cuda.synchronize()
    assert torch.equal(dw.view(torch.uint8), before.view(torch.uint8))
    # The workload's own launch (256x128x64, pool 256) fits, with every reduction.
    for red in ("linear", "tree", "workspace", "atomic"):
        kw2 = dict(kw, tile="256x128x64", reduction=red)
        assert skg.plan_wgrad(**kw2)["workspace_bytes"] <= _lib.STATIC_SCRATCH_BYTES
