"""GPU parity of the conv-wgrad path (implicit GEMM) against the oracle.

Dense, strided and grouped shapes with a partial last M tile per group, zero
padding and a ragged reduction tail; every tile instance x launch mode x
fix-up; random data within 5e-3 and integer-exact data bit for bit; the two
wgrad workloads at full size in the benchmark's launch configuration against
the full oracle; stream-K beats nothing here -- that is the benchmark's job.
"""

import numpy as np
import pytest
import torch

import implicit_gemm_conv_dp_amd as skg
from implicit_gemm_conv_dp_amd import synth
from oracle.wgrad import out_size, wgrad as oracle_wgrad

from helpers import assert_close, decode_out, out_buffer, to_dev

pytestmark = pytest.mark.gpu

MODES = ["dp", "dp_sk", "persistent"]
REDS = ["linear", "tree", "atomic", "workspace"]

# N, H, W, C, K, R, S, stride, pad, groups
SHAPES = {
    "dense": (2, 9, 9, 16, 24, 3, 3, (1, 1), (1, 1), 1),
    "strided": (3, 11, 10, 32, 16, 3, 3, (2, 2), (1, 1), 1),
    "grouped": (2, 12, 12, 64, 32, 3, 3, (2, 2), (1, 1), 4),
    "wide": (1, 17, 15, 144, 40, 3, 2, (1, 2), (1, 0), 1),
    # reductions shorter than one K tile: a single pixel, and 9 pixels
    "one_pixel": (1, 1, 1, 16, 16, 1, 1, (1, 1), (0, 0), 1),
    "short": (1, 3, 3, 16, 24, 3, 3, (1, 1), (1, 1), 1),
}
TILES = ["128x128x32", "32x64x64", "128x128x64", "256x128x64", "256x256x64"]


def run(x, dy, shape, fmt, tile, mode, red, ctas, ws=None, sk_order="auto"):
    n, h, w, c, k, r, s, st, pd, g = shape
    dx, ddy = to_dev(x, fmt), to_dev(dy, fmt)
    dw = out_buffer("f32", k * r * s * (c // g))
    plan = skg.wgrad(dx, ddy, dw.view(torch.float32), workspace=ws,
                     n=n, h=h, w=w, c=c, k=k, r=r, s=s, stride=st, pad=pd, groups=g, dtype=fmt,
                     tile=tile, mode=mode, reduction=red, ctas=ctas, sk_order=sk_order)
    torch.cuda.synchronize()
    return decode_out(dw, "f32").reshape(k, -1), plan


def inputs(shape, fmt, integer, seed):
    n, h, w, c, k, r, s, st, pd, g = shape
    ho, wo = out_size(h, w, r, s, st[0], st[1], pd[0], pd[1])
    if integer:
        x = synth.integer_codes(fmt, n * h * w * c, seed, 0.5)
        dy = synth.integer_codes(fmt, n * ho * wo * k, seed + 1, 0.5)
    else:
        x = synth.to_codes(synth.draw("uniform", n * h * w * c, seed), fmt)
        dy = synth.to_codes(synth.draw("uniform", n * ho * wo * k, seed + 1), fmt)
    R = oracle_wgrad(fmt, x, dy, n, h, w, c, k, r, s, st[0], st[1], pd[0], pd[1], g)
    return x, dy, R.reshape(k, -1)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("name", list(SHAPES))
def test_random_all_modes_and_fixups(name, tile):
    shape = SHAPES[name]
    fmt = "bf16" if name in ("grouped", "wide") else "f16"
    x, dy, R = inputs(shape, fmt, False, 5)
    for mode in MODES:
        for red in REDS:
            if mode == "dp" and red != "linear":
                continue
            for ctas in (3, 5, 11):
                Y, plan = run(x, dy, shape, fmt, tile, mode, red, ctas)
                assert_close(Y, R, fmt, "%s %s %s %s ctas=%d" % (name, tile, mode, red, ctas))
                if mode == "dp":
                    break


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("name", list(SHAPES))
def test_integer_exact_all_modes_and_fixups(name, tile):
    shape = SHAPES[name]
    x, dy, R = inputs(shape, "bf16", True, 31)
    for mode in MODES:
        for red in REDS:
            if mode == "dp" and red != "linear":
                continue
            Y, plan = run(x, dy, shape, "bf16", tile, mode, red, 7)
            assert np.array_equal(Y, R), "%s %s %s %s not bit-exact" % (name, tile, mode, red)


@pytest.mark.parametrize("index", [3, 4])
def test_workload_full_size(index):
    wl = synth.WORKLOADS[index]
    inp = wl.inputs()
    shape = (wl.n, wl.h, wl.w, wl.c, wl.k, wl.r, wl.s, wl.stride, wl.pad, wl.groups)
    R = oracle_wgrad(wl.dtype, inp["x"], inp["dy"], wl.n, wl.h, wl.w, wl.c, wl.k, wl.r, wl.s,
                     wl.stride[0], wl.stride[1], wl.pad[0], wl.pad[1], wl.groups).reshape(wl.k, -1)
    for mode in wl.modes:
        for red in wl.reductions:
            Y, plan = run(inp["x"], inp["dy"], shape, wl.dtype, wl.tile, mode, red, wl.ctas)
            assert_close(Y, R, wl.dtype, "%s %s %s" % (wl.name, mode, red))


@pytest.mark.parametrize("tile", ["32x64x64", "128x128x64", "256x256x64"])
@pytest.mark.parametrize("name", ["dense", "grouped"])
def test_split_k_and_auto_integer_exact(name, tile):
    shape = SHAPES[name]
    x, dy, R = inputs(shape, "bf16", True, 61)
    for mode, red, ctas in [("splitk", "workspace", 2), ("splitk", "tree", 3),
                            ("splitk", "linear", 7), ("splitk", "atomic", 4),
                            ("auto", "auto", 5), ("auto", "linear", 9), ("auto", "auto", -1),
                            ("splitk", "auto", -1)]:
        Y, plan = run(x, dy, shape, "bf16", tile, mode, red, ctas)
        assert np.array_equal(Y, R), "%s %s %s %s ctas=%d not bit-exact" % (name, tile, mode, red,
                                                                             ctas)
        assert plan["requested_mode"] == skg.MODES[mode]


@pytest.mark.parametrize("mode", ["auto", "splitk"])
def test_workload_auto_and_split_k_full_size(mode):
    # The dense wgrad workload on the default pool: "auto" resolves to
    # stream-K with the workspace fix-up, split-K to equal K slices.
    wl = synth.WORKLOADS[3]
    inp = wl.inputs()
    shape = (wl.n, wl.h, wl.w, wl.c, wl.k, wl.r, wl.s, wl.stride, wl.pad, wl.groups)
    R = oracle_wgrad(wl.dtype, inp["x"], inp["dy"], wl.n, wl.h, wl.w, wl.c, wl.k, wl.r, wl.s,
                     wl.stride[0], wl.stride[1], wl.pad[0], wl.pad[1], wl.groups).reshape(wl.k, -1)
    Y, plan = run(inp["x"], inp["dy"], shape, wl.dtype, wl.tile, mode, "auto", -1)
    if mode == "auto":
        assert plan["mode"] == skg.MODES["dp_sk"] and plan["sk_ctas"] > 0 and plan["slices"] == 1
    else:
        assert plan["slices"] > 1 and plan["dp_tiles"] == 0
    assert plan["reduction"] == skg.REDUCTIONS["workspace"]
    assert_close(Y, R, wl.dtype, "%s %s" % (wl.name, mode))


def divisors(n):
    return [d for d in range(2, n + 1) if n % d == 0]


LONG = (4, 16, 16, 32, 48, 3, 3, (1, 1), (1, 1), 1)  # 16 MAC iterations per tile


@pytest.mark.parametrize("tile", ["32x64x64", "256x128x64"])
@pytest.mark.parametrize("name", ["grouped", "long"])
def test_kmajor_sk_order_integer_exact(name, tile):
    # Whole slices dealt slice by slice (pools of tiles x S with S dividing
    # the iterations per tile): bit-exact in every mode and fix-up.
    shape = LONG if name == "long" else SHAPES[name]
    x, dy, R = inputs(shape, "bf16", True, 96)
    _, p0 = run(x, dy, shape, "bf16", tile, "dp_sk", "workspace", 8)
    T, ipt = p0["tiles"], p0["iters_per_tile"]
    ds = divisors(ipt)
    for S in sorted({ds[0], ds[len(ds) // 2], ipt}):
        for mode in ("dp_sk", "persistent"):
            for red in REDS:
                Y, plan = run(x, dy, shape, "bf16", tile, mode, red, T * S, sk_order="kmajor")
                assert plan["sk_order"] == skg.SK_ORDERS["kmajor"], (T, S, plan)
                assert np.array_equal(Y, R), "%s %s %s %s S=%d kmajor order" % (name, tile, mode,
                                                                               red, S)


@pytest.mark.parametrize("tile", ["32x64x64", "128x128x64", "256x128x64", "256x256x64"])
@pytest.mark.parametrize("name", ["grouped", "long"])
def test_scatter_fixup_integer_exact(name, tile):
    # The reduce-scatter fix-up on whole-slice pools (tiles x S, S dividing
    # the iterations per tile), both launch modes, both CTA orders that
    # apply: bit-exact.
    shape = LONG if name == "long" else SHAPES[name]
    x, dy, R = inputs(shape, "bf16", True, 97)
    _, p0 = run(x, dy, shape, "bf16", tile, "dp_sk", "workspace", 8)
    T, ipt = p0["tiles"], p0["iters_per_tile"]
    ds = divisors(ipt)
    for S in sorted({ds[0], ds[len(ds) // 2], ipt}):
        for mode in ("dp_sk", "persistent"):
            for order in ("xcd", "kmajor"):
                Y, plan = run(x, dy, shape, "bf16", tile, mode, "scatter", T * S, sk_order=order)
                assert plan["reduction"] == skg.REDUCTIONS["scatter"] and plan["sk_ctas"] == T * S
                assert np.array_equal(Y, R), "%s %s %s S=%d %s scatter" % (name, tile, mode, S,
                                                                          order)


@pytest.mark.parametrize("tile", ["32x64x64", "256x256x64", "64x144x32"])
def test_scatter_is_linear_bit_for_bit(tile):
    # The reduce-scatter fix-up adds the tile's partials in the linear
    # fix-up's order -- the first contributor's, then each later one in CTA
    # order -- only split over the contributors: on random data, for the same
    # partition, both give the same bits.
    shape = (8, 16, 16, 64, 64, 3, 3, (2, 2), (1, 1), 4) if tile == "64x144x32" else LONG
    x, dy, _ = inputs(shape, "f16", False, 131)
    _, p0 = run(x, dy, shape, "f16", tile, "dp_sk", "workspace", 8)
    T, ipt = p0["tiles"], p0["iters_per_tile"]
    ds = divisors(ipt)
    for S in sorted({ds[0], ds[len(ds) // 2], ipt}):
        for mode in ("dp_sk", "persistent"):
            for order in ("xcd", "kmajor"):
                Ys, ps = run(x, dy, shape, "f16", tile, mode, "scatter", T * S, sk_order=order)
                Yl, pl = run(x, dy, shape, "f16", tile, mode, "linear", T * S, sk_order=order)
                assert ps["sk_ctas"] == pl["sk_ctas"] == T * S and ps["sk_order"] == pl["sk_order"]
                assert np.array_equal(Ys, Yl), "%s %s S=%d %s" % (tile, mode, S, order)


@pytest.mark.parametrize("index", [3, 4])
def test_scatter_is_linear_bit_for_bit_full_size(index):
    # Both wgrad workloads in the benchmark's launch (pool, mode, CTA order):
    # the reduce-scatter and the linear fix-up give the same bits.
    wl = synth.WORKLOADS[index]
    inp = wl.inputs()
    shape = (wl.n, wl.h, wl.w, wl.c, wl.k, wl.r, wl.s, wl.stride, wl.pad, wl.groups)
    mode = wl.modes[0]
    Ys, ps = run(inp["x"], inp["dy"], shape, wl.dtype, wl.tile, mode, "scatter", wl.ctas)
    Yl, pl = run(inp["x"], inp["dy"], shape, wl.dtype, wl.tile, mode, "linear", wl.ctas)
    assert ps["sk_ctas"] == pl["sk_ctas"] == wl.ctas and ps["sk_order"] == pl["sk_order"]
    assert np.array_equal(Ys, Yl), wl.name


def test_scatter_fixup_full_layer():
    # The 56x56 layer, split-K over the default pool with the scatter fix-up
    # in k-major order, element by element against the oracle.
    wl = synth.WORKLOADS[3]
    inp = wl.inputs()
    shape = (wl.n, wl.h, wl.w, wl.c, wl.k, wl.r, wl.s, wl.stride, wl.pad, wl.groups)
    R = oracle_wgrad(wl.dtype, inp["x"], inp["dy"], wl.n, wl.h, wl.w, wl.c, wl.k, wl.r, wl.s,
                     wl.stride[0], wl.stride[1], wl.pad[0], wl.pad[1], wl.groups).reshape(wl.k, -1)
    for tile in ("256x128x64", "256x256x64"):
        Y, plan = run(inp["x"], inp["dy"], shape, wl.dtype, tile, "splitk", "scatter", -1,
                      sk_order="kmajor")
        assert plan["slices"] > 1 and plan["sk_order"] == skg.SK_ORDERS["kmajor"]
        assert_close(Y.reshape(wl.k, -1), R, wl.dtype, "%s %s scatter" % (wl.name, tile))


@pytest.mark.parametrize("tile", ["32x64x64", "256x128x64"])
@pytest.mark.parametrize("name", ["grouped", "wide"])
def test_block_sk_order_integer_exact(name, tile):
    # Stream-K CTAs in block order (not the wgrad default): bit-exact too.
    shape = SHAPES[name]
    x, dy, R = inputs(shape, "bf16", True, 95)
    for mode in ("dp_sk", "persistent"):
        for red in REDS:
            for ctas in (7, 16):
                Y, plan = run(x, dy, shape, "bf16", tile, mode, red, ctas, sk_order="block")
                assert plan["sk_order"] == skg.SK_ORDERS["block"]
                assert np.array_equal(Y, R), "%s %s %s %s block order" % (name, tile, mode, red)


# Block-diagonal grouped tile (16 input and 16 output channels per group,
# four groups per 64-row tile; nine filter taps per 144-column tile).
BD_TILE = "64x144x32"
BD_SHAPES = {
    # 2 M tiles, 32 iterations each (the ring wraps), stride 1
    "bd_two_tiles": (4, 16, 16, 128, 128, 3, 3, (1, 1), (1, 1), 8),
    # 4 + 2 groups (ragged last M tile), reduction 243 = 7 iterations + a tail
    "bd_ragged": (3, 9, 9, 96, 96, 3, 3, (1, 1), (1, 1), 6),
    # stride 2 with padding, like the workload's layer
    "bd_strided": (8, 14, 14, 64, 64, 3, 3, (2, 2), (1, 1), 4),
    # one group, uneven padding
    "bd_one_group": (3, 7, 5, 16, 16, 3, 3, (1, 1), (0, 1), 1),
    # 1x1: one tap used, eight taps past R*S
    "bd_1x1": (2, 8, 8, 64, 64, 1, 1, (1, 1), (0, 0), 4),
    # 5x5: 25 taps in three N tiles (the last holds 7), strides 2 x 1
    "bd_5x5": (2, 11, 9, 80, 80, 5, 5, (2, 1), (2, 2), 5),
    # a 6-pixel reduction: one MAC iteration, mostly past its end
    "bd_short": (1, 2, 3, 16, 16, 3, 3, (1, 1), (1, 1), 1),
}


@pytest.mark.parametrize("name", list(BD_SHAPES))
def test_block_diagonal_integer_exact_all_modes_and_fixups(name):
    shape = BD_SHAPES[name]
    x, dy, R = inputs(shape, "bf16", True, 131)
    for mode in MODES:
        for red in REDS:
            if mode == "dp" and red != "linear":
                continue
            for ctas in (3, 7, 16):
                Y, plan = run(x, dy, shape, "bf16", BD_TILE, mode, red, ctas)
                assert np.array_equal(Y, R), "%s %s %s ctas=%d not bit-exact" % (name, mode, red,
                                                                                 ctas)
                if mode == "dp":
                    break


@pytest.mark.parametrize("name", list(BD_SHAPES))
def test_block_diagonal_random(name):
    shape = BD_SHAPES[name]
    for fmt in ("f16", "bf16"):
        x, dy, R = inputs(shape, fmt, False, 137)
        for mode, red, ctas in [("dp", "linear", 1), ("dp_sk", "tree", 5),
                                ("persistent", "linear", 11), ("dp_sk", "atomic", 6),
                                ("persistent", "workspace", 9)]:
            Y, plan = run(x, dy, shape, fmt, BD_TILE, mode, red, ctas)
            assert_close(Y, R, fmt, "%s %s %s %s" % (name, fmt, mode, red))


@pytest.mark.parametrize("name", ["bd_two_tiles", "bd_ragged", "bd_5x5"])
def test_block_diagonal_split_k_scatter_and_orders(name):
    shape = BD_SHAPES[name]
    x, dy, R = inputs(shape, "bf16", True, 139)
    for mode, red, ctas, order in [("splitk", "scatter", 2, "kmajor"),
                                   ("splitk", "scatter", 4, "auto"),
                                   ("splitk", "tree", 5, "xcd"),
                                   ("splitk", "workspace", 2, "block"),
                                   ("dp_sk", "linear", 9, "block"),
                                   ("persistent", "tree", 13, "xcd"),
                                   ("auto", "auto", -1, "auto")]:
        Y, plan = run(x, dy, shape, "bf16", BD_TILE, mode, red, ctas, sk_order=order)
        assert np.array_equal(Y, R), "%s %s %s %d %s not bit-exact" % (name, mode, red, ctas,
                                                                       order)


def test_block_diagonal_full_layer():
    # The grouped 28x28 layer (N=64, 32 groups, stride 2) on the
    # block-diagonal tile, element by element against the oracle, in the
    # hand-off fix-ups at the full pool and with split-K scatter.
    wl = synth.WORKLOADS[4]
    inp = wl.inputs()
    shape = (wl.n, wl.h, wl.w, wl.c, wl.k, wl.r, wl.s, wl.stride, wl.pad, wl.groups)
    R = oracle_wgrad(wl.dtype, inp["x"], inp["dy"], wl.n, wl.h, wl.w, wl.c, wl.k, wl.r, wl.s,
                     wl.stride[0], wl.stride[1], wl.pad[0], wl.pad[1], wl.groups).reshape(wl.k, -1)
    for mode, red, ctas in [("dp_sk", "linear", 256), ("persistent", "tree", 256),
                            ("dp_sk", "atomic", 256), ("splitk", "scatter", 28)]:
        Y, plan = run(inp["x"], inp["dy"], shape, wl.dtype, BD_TILE, mode, red, ctas)
        assert (plan["tiles_m"], plan["tiles_n"]) == (8, 1)
        assert_close(Y, R, wl.dtype, "%s %s %s %s" % (wl.name, BD_TILE, mode, red))
